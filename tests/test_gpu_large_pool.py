"""GPU parity on a pool larger than 4 GiB: every entry point reads or writes
rows whose byte offset slot * 576 does not fit in 32 bits.

The pool has 2^23 slots (4.83 GB).  Slots from HI0 = floor(2^32 / 576) + 1 on
start past 4 GiB.  The oracle sees only the rows a call names, gathered into a
compact pool with the indices renumbered 0..n-1 (the result depends on the
rows, not on where they sit, which test_gpu_decode checks by relocating
slots).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, bf16_bits

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")

NUM_SLOTS = 1 << 23
HI0 = (1 << 32) // workloads.KV_WIDTH + 1


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


@pytest.fixture(scope="module")
def pool(dev):
    print("large pool: %d slots (%.2f GB)" % (NUM_SLOTS, NUM_SLOTS * 576 / 1e9), flush=True)
    p = workloads.random_pool(NUM_SLOTS, seed=4242, device=dev, outlier_frac=0.001)
    torch.cuda.synchronize()
    yield p
    del p
    torch.cuda.empty_cache()


def _high_slots(n, seed, low=0):
    """n distinct slots: all but `low` of them past 4 GiB, the last slot included."""
    rng = np.random.default_rng(seed)
    hi = rng.choice(NUM_SLOTS - HI0 - 1, size=n - low - 1, replace=False) + HI0
    lo = rng.choice(HI0, size=low, replace=False)
    s = np.concatenate([hi, lo, [NUM_SLOTS - 1]]).astype(np.int64)
    rng.shuffle(s)
    assert (s >= HI0).sum() == n - low and s.max() == NUM_SLOTS - 1
    return s


def _compact(pool, slots):
    """The named rows as a host pool, in index order (slot i -> row i)."""
    idx = torch.from_numpy(slots).to(pool.device)
    return pool.index_select(0, idx).cpu().numpy()


def _decode_case(dev, pool, H, lengths, seed):
    total = int(sum(lengths))
    slots = _high_slots(total, seed, low=total // 10)
    indptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = workloads.random_q(len(lengths), H, seed, device=dev)
    scale, sm = 1.25, 1.0 / np.sqrt(192.0)
    print("decode H=%d lengths=%s" % (H, list(lengths)), flush=True)
    out = fm.mla_decode_fp8(q, pool, torch.from_numpy(indptr).to(dev),
                            torch.from_numpy(slots.astype(np.int32)).to(dev), scale, sm)
    torch.cuda.synchronize()
    ref = oracle.mla_decode_ref(bf16_bits(q), _compact(pool, slots), indptr,
                                np.arange(total, dtype=np.int32), scale, sm)
    assert_attention_close(out, ref, "decode past 4 GiB, H=%d" % H)


def test_decode_rows_past_4gib(dev, pool):
    _decode_case(dev, pool, 16, [700, 300, 1500, 129], seed=1)


def test_decode_64_head_kernel_rows_past_4gib(dev, pool):
    # 36,000 tokens at 128 heads: at least 4 tiles of 64 tokens per workgroup
    # slot of a 256-CU device, so the 64-heads-per-workgroup kernel runs
    _decode_case(dev, pool, 128, [20000, 16000], seed=2)


def test_extend_rows_past_4gib(dev, pool):
    q_lens, hist = [3, 5], [900, 2100]
    kv_lens = [h + n for h, n in zip(hist, q_lens)]
    total_kv, total_q, H = sum(kv_lens), sum(q_lens), 16
    slots = _high_slots(total_kv, seed=3, low=50)
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    q = workloads.random_q(total_q, H, 3, device=dev)
    print("extend q_lens=%s history=%s" % (q_lens, hist), flush=True)
    out = fm.mla_extend_fp8(q, pool, torch.from_numpy(qo).to(dev), torch.from_numpy(kv).to(dev),
                            torch.from_numpy(slots.astype(np.int32)).to(dev), 1.0,
                            1.0 / np.sqrt(192.0), causal=True)
    torch.cuda.synchronize()
    ref = oracle.mla_extend_ref(bf16_bits(q), _compact(pool, slots), qo, kv,
                                np.arange(total_kv, dtype=np.int32), 1.0, 1.0 / np.sqrt(192.0),
                                causal=True)
    assert_attention_close(out, ref, "extend past 4 GiB")


def test_gather_cast_rows_past_4gib(dev, pool):
    slots = _high_slots(5000, seed=4, low=100)
    print("gather_cast n=%d" % len(slots), flush=True)
    out = fm.gather_cast_fp8_bf16(pool, torch.from_numpy(slots.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    rows = _compact(pool, slots)
    assert np.array_equal(bf16_bits(out), oracle.gather_ref(rows, np.arange(len(slots))))


def test_cast_pool_past_4gib(dev, pool):
    print("cast_pool of %d slots" % NUM_SLOTS, flush=True)
    out = fm.cast_pool_fp8_bf16(pool)
    torch.cuda.synchronize()
    check = _high_slots(3000, seed=5, low=300)
    got = bf16_bits(out.index_select(0, torch.from_numpy(check).to(dev)))
    del out
    torch.cuda.empty_cache()
    assert np.array_equal(got, oracle.cast_ref(_compact(pool, check)))


def test_scatter_cast_rows_past_4gib(dev, pool):
    slots = _high_slots(3000, seed=6, low=200)
    src = workloads.new_kv_rows(len(slots), 6, device=dev, outlier_frac=0.01)
    before = _compact(pool, slots)
    print("scatter_cast n=%d" % len(slots), flush=True)
    fm.scatter_cast_bf16_fp8(src, torch.from_numpy(slots.astype(np.int32)).to(dev), pool,
                             inv_scale=0.5, saturate=True)
    torch.cuda.synchronize()
    after = _compact(pool, slots)
    want = oracle.scatter_ref(before, bf16_bits(src), np.arange(len(slots)), 0.5, saturate=True)
    assert np.array_equal(after, want)
