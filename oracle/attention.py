"""MLA decode attention over a paged FP8 latent cache -- oracle (test infrastructure).

Plain definition, float64 throughout, no blocking or reordering beyond what
the definition states.  For request b with pool slots
``kv_indices[kv_indptr[b]:kv_indptr[b+1]]`` (one token per slot; "The
Gather-Then-Cast Pivot", *The Subject Message*: the wrapper reads the pool
slots that ``kv_indices`` names) and each query head h:

    K[t, :]  = scale * e4m3(pool[slot_t, :])             (576 wide)
    s[t]     = sm_scale * sum_{d<576} q[b,h,d] * K[t,d]  (scores over 512 latent + 64 rope)
    p[t]     = exp(s[t] - max_t s)                       (max-subtracted softmax)
    out[b,h] = sum_t p[t] * K[t, :512] / sum_t p[t]      (values = the 512 latent dims)

The 576 = 512 + 64 split is the pages' ``kv_lora_rank`` + ``qk_rope_head_dim``
("The KV Cache Cast Bottleneck", *The Context*); the cache is one KV head
shared by every query head (the pool's middle dimension is 1).  ``scale`` is
a per-tensor dequantisation factor; the pages never apply one (their casts are
plain ``.to()``), so it multiplies both the score and the value operand here,
and scale = 1 reduces to the pages' path.  A request with no tokens yields a
zero row.
"""
import math

import numpy as np

from .e4m3 import decode_table

KV_WIDTH = 576  # 512 latent + 64 rope
V_WIDTH = 512   # latent part, the value operand

_TABLE = None


def _table() -> np.ndarray:
    global _TABLE
    if _TABLE is None:
        _TABLE = decode_table()
    return _TABLE


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of BF16 bit patterns (uint16 / int16 arrays)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _check(q_bits, pool, indptr, indices):
    q_bits = np.asarray(q_bits)
    pool = np.asarray(pool)
    indptr = np.asarray(indptr).astype(np.int64)
    indices = np.asarray(indices).astype(np.int64)
    if q_bits.ndim != 3 or q_bits.shape[2] != KV_WIDTH:
        raise ValueError("q must be [B, H, 576] BF16 bits")
    if pool.dtype != np.uint8 or pool.ndim != 2 or pool.shape[1] != KV_WIDTH:
        raise ValueError("pool must be uint8 [num_slots, 576]")
    B = q_bits.shape[0]
    if indptr.shape != (B + 1,) or indptr[0] != 0 or np.any(np.diff(indptr) < 0):
        raise ValueError("kv_indptr must be [B+1], start at 0, non-decreasing")
    if indptr[-1] > indices.shape[0]:
        raise ValueError("kv_indptr[B] exceeds len(kv_indices)")
    return q_bits, pool, indptr, indices


def _request_kv(pool, indices, lo, hi, scale):
    slots = indices[lo:hi]
    if slots.size and (slots.min() < 0 or slots.max() >= pool.shape[0]):
        raise IndexError("kv index outside the pool")
    return _table()[pool[slots]] * float(scale)  # [L, 576] float64, exact


def mla_decode_ref(q_bits, pool, indptr, indices, scale, sm_scale,
                   requests=None, heads=None) -> np.ndarray:
    """float64 [len(requests), len(heads), 512]; all requests/heads by default."""
    q_bits, pool, indptr, indices = _check(q_bits, pool, indptr, indices)
    B, H, _ = q_bits.shape
    requests = list(range(B)) if requests is None else list(requests)
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(requests), len(heads), V_WIDTH), dtype=np.float64)
    for i, b in enumerate(requests):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        if hi == lo:
            continue
        K = _request_kv(pool, indices, lo, hi, scale)
        qd = bf16_bits_to_f64(q_bits[b, heads, :])          # [h, 576]
        s = float(sm_scale) * (qd @ K.T)                     # [h, L]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[i] = (p @ K[:, :V_WIDTH]) / p.sum(axis=1, keepdims=True)
    return out


def mla_decode_partial_ref(q_bits, pool, indptr, indices, scale, sm_scale, b, lo, hi):
    """Attention of request b over its tokens [lo, hi) only (request-relative).

    Returns ``(o, lse)``: o float64 [H, 512] is the softmax-normalised output
    over that token subset and lse float64 [H] is ``log(sum_t exp(s[t]))``
    over the same subset (natural log).  An empty subset gives o = 0 and
    lse = -inf.
    """
    q_bits, pool, indptr, indices = _check(q_bits, pool, indptr, indices)
    H = q_bits.shape[1]
    start = int(indptr[b])
    L = int(indptr[b + 1]) - start
    if not 0 <= lo <= hi <= L:
        raise ValueError("token range outside the request")
    if hi == lo:
        return np.zeros((H, V_WIDTH)), np.full(H, -np.inf)
    K = _request_kv(pool, indices, start + lo, start + hi, scale)
    qd = bf16_bits_to_f64(q_bits[b])
    s = float(sm_scale) * (qd @ K.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    denom = p.sum(axis=1)
    o = (p @ K[:, :V_WIDTH]) / denom[:, None]
    lse = m[:, 0] + np.log(denom)
    return o, lse


def combine_partials_ref(parts):
    """Merge (o, lse) pairs of disjoint token subsets of one request.

    The softmax over a union of subsets weights each subset's normalised
    output by its share of the total exponential mass, exp(lse_i) / sum_j
    exp(lse_j); the maximum lse is subtracted first so no exponential
    overflows.  Subsets with lse = -inf (empty) carry zero weight.
    """
    os_ = np.stack([np.asarray(o, dtype=np.float64) for o, _ in parts])     # [S, H, 512]
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])    # [S, H]
    M = lses.max(axis=0)                                                    # [H]
    out = np.zeros(os_.shape[1:])
    live = np.isfinite(M)
    w = np.where(np.isfinite(lses), np.exp(lses - np.where(live, M, 0.0)), 0.0)
    num = (w[:, :, None] * os_).sum(axis=0)
    den = w.sum(axis=0)
    out[live] = num[live] / den[live][:, None]
    return out


def lse_natural_to_log2(lse):
    return np.asarray(lse) / math.log(2.0)
