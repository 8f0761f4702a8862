"""Seeded synthetic inputs for FP8 paged MLA decode.

Shared by the oracle-side tests and the HIP-side tests and benchmark.  This
module draws random numbers and lays them out; it holds none of the method's
arithmetic (no FP8 decoding, no attention).  FP8 encoding of the drawn values
is torch's own ``.to(torch.float8_e4m3fn)`` after a clip to the format's
finite range.

The shapes follow the serving setups the pages profile: a latent KV row of
576 bytes (512 latent + 64 rope), pools of 495,552 slots, batch 40 with 16
query heads per KV head, FP8-E4M3FN storage ("The KV Cache Cast Bottleneck",
*The Context*; "When a Faster Kernel Doesn't Speed Up Serving", *Setup*).
There is no public dataset behind these pages' numbers; these synthetic
tensors stand in for live serving traffic.

Structure (lengths, slot permutations, scale) comes from
``numpy.random.default_rng(seed)``; element values from a
``torch.Generator`` on the target device seeded with the same seed, so large
pools can be drawn directly in device memory.  ``seed = 1000 * config +
replica``.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

KV_WIDTH = 576
V_WIDTH = 512
E4M3_MAX = 448.0

CONFIG_NAMES = {
    1: "tiny: B=1 H=16 L=64 page=1 pool=1024",
    2: "batch40: B=40 H=16 L~U[1024,8192] page=1 pool=495552 scale~U[0.5,2]",
    3: "cast-path layer: B=1 H=64 L=4096 page=1 pool=495552 (x78 layers)",
    4: "long-context: B=8 H=128 L~U[32768,131072] page=64 pool=2^21",
    5: "serving-mix: B=256 H=16 L~lognormal(2048,1) page=64 pool=2^20 1% +-448",
}


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    H: int
    page_size: int
    num_slots: int
    lengths: np.ndarray            # int64 [B]
    pool: torch.Tensor             # uint8 [num_slots, 576]  (E4M3FN bytes)
    indptr: torch.Tensor           # int32 [B+1]
    indices: torch.Tensor          # int32 [sum(lengths)]
    q: torch.Tensor                # bfloat16 [B, H, 576]
    scale: float
    sm_scale: float
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def useful_kv_bytes(self) -> int:
        return KV_WIDTH * self.total_tokens

    def to(self, device):
        return Workload(self.name, self.seed, self.B, self.H, self.page_size,
                        self.num_slots, self.lengths, self.pool.to(device),
                        self.indptr.to(device), self.indices.to(device),
                        self.q.to(device), self.scale, self.sm_scale, dict(self.meta))


def quantize_e4m3(x: torch.Tensor) -> torch.Tensor:
    """Clip to +-448 and encode with torch's E4M3FN cast; returns the bytes (uint8)."""
    return x.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def random_pool(num_slots: int, seed: int, device="cpu", sigma: float = 1.0,
                outlier_frac: float = 0.0, chunk_rows: int = 1 << 18) -> torch.Tensor:
    """uint8 [num_slots, 576]: N(0, sigma^2) values in E4M3FN, optional +-448 outliers."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pool = torch.empty((num_slots, KV_WIDTH), dtype=torch.uint8, device=device)
    for r0 in range(0, num_slots, chunk_rows):
        r1 = min(num_slots, r0 + chunk_rows)
        x = torch.randn((r1 - r0, KV_WIDTH), generator=g, device=device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        if outlier_frac > 0.0:
            u = torch.rand((r1 - r0, KV_WIDTH), generator=g, device=device)
            sgn = torch.where(torch.rand((r1 - r0, KV_WIDTH), generator=g, device=device) < 0.5,
                              -E4M3_MAX, E4M3_MAX)
            x = torch.where(u < outlier_frac, sgn, x)
        pool[r0:r1] = quantize_e4m3(x)
    return pool


def random_q(B: int, H: int, seed: int, device="cpu", sigma: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed + 7919)
    q = torch.randn((B, H, KV_WIDTH), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        q.mul_(sigma)
    return q.to(torch.bfloat16)


def new_kv_rows(n: int, seed: int, device="cpu", sigma: float = 1.0,
                outlier_frac: float = 0.0) -> torch.Tensor:
    """bfloat16 [n, 576]: freshly computed KV rows for the write path, N(0, sigma^2),
    with a fraction of elements replaced by magnitudes U[400, 600] (random sign)
    that straddle the E4M3FN range."""
    g = torch.Generator(device=device)
    g.manual_seed(seed + 104729)
    x = torch.randn((n, KV_WIDTH), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    if outlier_frac > 0.0:
        u = torch.rand((n, KV_WIDTH), generator=g, device=device)
        mag = 400.0 + 200.0 * torch.rand((n, KV_WIDTH), generator=g, device=device)
        sgn = torch.where(torch.rand((n, KV_WIDTH), generator=g, device=device) < 0.5, -1.0, 1.0)
        x = torch.where(u < outlier_frac, sgn * mag, x)
    return x.to(torch.bfloat16)


def free_slots(n: int, num_slots: int, seed: int) -> np.ndarray:
    """int32 [n]: n distinct destination slots drawn at random from the pool."""
    rng = np.random.default_rng(seed)
    return rng.choice(num_slots, size=n, replace=False).astype(np.int32)


def assign_slots(lengths, num_slots: int, page_size: int, rng) -> np.ndarray:
    """Concatenated slot ids for requests of the given lengths.

    page_size 1: one random permutation of the pool, consumed in order, so
    requests never share a slot.  page_size P > 1: the pool is cut into pages
    of P consecutive slots, pages are handed out by a random permutation, and a
    request's token t sits at slot page[t // P] * P + t % P (the last page of a
    request is partly used).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    if page_size == 1:
        if lengths.sum() > num_slots:
            raise ValueError("pool too small for the requested tokens")
        return rng.permutation(num_slots)[: lengths.sum()].astype(np.int64)
    num_pages = num_slots // page_size
    pages_needed = (lengths + page_size - 1) // page_size
    if pages_needed.sum() > num_pages:
        raise ValueError("pool too small for the requested pages")
    perm = rng.permutation(num_pages)
    out = np.empty(int(lengths.sum()), dtype=np.int64)
    pos = 0
    pg = 0
    for L in lengths:
        L = int(L)
        t = np.arange(L)
        pages = perm[pg: pg + (L + page_size - 1) // page_size]
        out[pos: pos + L] = pages[t // page_size] * page_size + t % page_size
        pos += L
        pg += (L + page_size - 1) // page_size
    return out


def build(name, seed, B, H, lengths, num_slots, page_size, scale, sm_scale,
          device="cpu", q_sigma=1.0, outlier_frac=0.0, rng=None, meta=None,
          indices=None) -> Workload:
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int64)
    if indices is None:
        indices = assign_slots(lengths, num_slots, page_size, rng)
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(lengths)
    pool = random_pool(num_slots, seed, device=device, outlier_frac=outlier_frac)
    q = random_q(B, H, seed, device=device, sigma=q_sigma)
    return Workload(name, seed, B, H, page_size, num_slots, lengths, pool,
                    torch.from_numpy(indptr.astype(np.int32)).to(device),
                    torch.from_numpy(np.asarray(indices).astype(np.int32)).to(device),
                    q, float(scale), float(sm_scale), dict(meta or {}))


def config(cfg: int, replica: int = 0, device="cpu") -> Workload:
    """One of the five standard workloads (see CONFIG_NAMES)."""
    seed = 1000 * cfg + replica
    rng = np.random.default_rng(seed)
    sm = 1.0 / math.sqrt(192.0)
    if cfg == 1:
        num_slots = 1024
        idx = rng.permutation(num_slots)[:64]
        return build(CONFIG_NAMES[1], seed, 1, 16, [64], num_slots, 1, 1.0, sm,
                     device=device, rng=rng, indices=idx)
    if cfg == 2:
        lengths = rng.integers(1024, 8192, size=40, endpoint=True)
        scale = float(rng.uniform(0.5, 2.0))
        return build(CONFIG_NAMES[2], seed, 40, 16, lengths, 495552, 1, scale, sm,
                     device=device, rng=rng)
    if cfg == 3:
        return build(CONFIG_NAMES[3], seed, 1, 64, [4096], 495552, 1, 1.0, sm,
                     device=device, rng=rng)
    if cfg == 4:
        lengths = rng.integers(32768, 131072, size=8, endpoint=True)
        return build(CONFIG_NAMES[4], seed, 8, 128, lengths, 1 << 21, 64, 1.0, sm,
                     device=device, rng=rng)
    if cfg == 5:
        num_slots = 1 << 20
        for _ in range(100):
            lengths = np.clip(np.rint(rng.lognormal(math.log(2048.0), 1.0, size=256)),
                              16, 32768).astype(np.int64)
            if ((lengths + 63) // 64).sum() <= num_slots // 64:
                break
        else:
            raise RuntimeError("could not draw a config-5 batch that fits the pool")
        return build(CONFIG_NAMES[5], seed, 256, 16, lengths, num_slots, 64, 1.0, sm,
                     device=device, q_sigma=2.0, outlier_frac=0.01, rng=rng,
                     meta={"q_sigma_reading": "N(0,2) read as sigma=2"})
    raise ValueError("unknown config %r" % (cfg,))


def small(B, H, lengths, num_slots=None, page_size=1, seed=0, scale=1.0,
          sm_scale=1.0 / math.sqrt(192.0), device="cpu", q_sigma=1.0,
          outlier_frac=0.0) -> Workload:
    """A small custom workload (tests: ragged tails, edge cases)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if num_slots is None:
        need = int(((lengths + page_size - 1) // page_size).sum()) * page_size
        num_slots = max(page_size, 2 * need + 3 * page_size)
    return build("custom B=%d H=%d" % (B, H), seed, B, H, lengths, num_slots, page_size,
                 scale, sm_scale, device=device, q_sigma=q_sigma, outlier_frac=outlier_frac)


# ---------------------------------------------------------------- extend / prefill

EXTEND_NAMES = {
    "spec4": "extend spec4: B=40 H=16 q_len=4 history~U[1024,8192] page=1 pool=495552",
    "chunk1k": "extend chunk1k: B=4 H=16 q_len=1024 history~U[2048,8192] page=1 pool=495552",
    "prefill4k_h64": "extend prefill4k_h64: B=1 H=64 q_len=4096 history=0 page=1 pool=495552",
}


@dataclass
class ExtendWorkload:
    name: str
    seed: int
    B: int
    H: int
    q_lens: np.ndarray             # int64 [B] new query tokens per request
    kv_lens: np.ndarray            # int64 [B] cache tokens per request (history + new)
    num_slots: int
    pool: torch.Tensor             # uint8 [num_slots, 576]
    qo_indptr: torch.Tensor        # int32 [B+1]
    kv_indptr: torch.Tensor        # int32 [B+1]
    kv_indices: torch.Tensor       # int32 [sum(kv_lens)]; request b's new tokens are its last q_len
    q: torch.Tensor                # bfloat16 [sum(q_lens), H, 576]
    scale: float
    sm_scale: float
    causal: bool = True

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    def visible_tokens(self) -> int:
        """Sum over query tokens of the cache tokens each sees."""
        tot = 0
        for ql, kl in zip(self.q_lens.tolist(), self.kv_lens.tolist()):
            if self.causal:
                i = np.arange(ql)
                tot += int(np.clip(kl - ql + i + 1, 0, kl).sum())
            else:
                tot += ql * kl
        return tot

    def kv_bytes(self) -> int:
        return KV_WIDTH * int(self.kv_lens.sum())


def extend(B, H, q_lens, history, num_slots=None, page_size=1, seed=0, scale=1.0,
           sm_scale=1.0 / math.sqrt(192.0), device="cpu", causal=True, q_sigma=1.0,
           outlier_frac=0.0, name=None) -> ExtendWorkload:
    """An extend batch: request b has history[b] cached tokens and q_lens[b] new
    ones, whose KV is already in the cache as the last q_lens[b] entries of its
    list.  Slots, pool values and queries are drawn as for decode."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(history, dtype=np.int64) + q_lens
    rng = np.random.default_rng(seed)
    if num_slots is None:
        need = int(((kv_lens + page_size - 1) // page_size).sum()) * page_size
        num_slots = max(page_size, 2 * need + 3 * page_size)
    indices = assign_slots(kv_lens, num_slots, page_size, rng)
    qo = np.zeros(B + 1, dtype=np.int64)
    qo[1:] = np.cumsum(q_lens)
    kv = np.zeros(B + 1, dtype=np.int64)
    kv[1:] = np.cumsum(kv_lens)
    pool = random_pool(num_slots, seed, device=device, outlier_frac=outlier_frac)
    g = torch.Generator(device=device)
    g.manual_seed(seed + 7919)
    q = torch.randn((int(qo[-1]), H, KV_WIDTH), generator=g, device=device, dtype=torch.float32)
    if q_sigma != 1.0:
        q.mul_(q_sigma)
    to = lambda a: torch.from_numpy(np.asarray(a).astype(np.int32)).to(device)
    return ExtendWorkload(name or "extend B=%d H=%d" % (B, H), seed, B, H, q_lens, kv_lens,
                          num_slots, pool, to(qo), to(kv), to(indices), q.to(torch.bfloat16),
                          float(scale), float(sm_scale), bool(causal))


def extend_config(name: str, replica: int = 0, device="cpu") -> ExtendWorkload:
    """One of the named extend workloads (see EXTEND_NAMES)."""
    seed = 9000 + 100 * list(EXTEND_NAMES).index(name) + replica
    rng = np.random.default_rng(seed)
    if name == "spec4":
        hist = rng.integers(1024, 8192, size=40, endpoint=True)
        return extend(40, 16, [4] * 40, hist, 495552, seed=seed, device=device,
                      name=EXTEND_NAMES[name])
    if name == "chunk1k":
        hist = rng.integers(2048, 8192, size=4, endpoint=True)
        return extend(4, 16, [1024] * 4, hist, 495552, seed=seed, device=device,
                      name=EXTEND_NAMES[name])
    if name == "prefill4k_h64":
        return extend(1, 64, [4096], [0], 495552, seed=seed, device=device,
                      name=EXTEND_NAMES[name])
    raise ValueError(name)
