"""GPU parity of the write path (BF16 rows -> E4M3FN pool slots) against the
oracle encoder: bit-exact, including every byte the call must leave alone."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import bf16_bits

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")

SCALES = [1.0, 0.5, 1.0 / 3.0, 7.25, 1e-3, 300.0, 2.0 ** 100, 2.0 ** -100]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _run(dev, src, slots_np, pool_np, inv_scale, saturate):
    pool = torch.from_numpy(pool_np).to(dev)
    out = fm.scatter_cast_bf16_fp8(src.to(dev), torch.from_numpy(slots_np).to(dev), pool,
                                   inv_scale, saturate)
    assert out is pool
    torch.cuda.synchronize()
    return pool.cpu().numpy()


def _all_bf16_rows():
    """Every BF16 bit pattern once, 114 rows of 576 (the tail wraps around)."""
    bits = (np.arange(114 * 576) % 65536).astype(np.uint16).reshape(114, 576)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16), bits


@pytest.mark.parametrize("saturate", [False, True])
@pytest.mark.parametrize("inv_scale", SCALES)
def test_all_bf16_patterns(dev, inv_scale, saturate):
    src, bits = _all_bf16_rows()
    rng = np.random.default_rng(17)
    pool0 = rng.integers(0, 256, size=(300, 576), dtype=np.uint8)
    slots = rng.permutation(300)[:114].astype(np.int32)
    got = _run(dev, src, slots, pool0, inv_scale, saturate)
    ref = oracle.scatter_ref(pool0, bits, slots, np.float32(inv_scale), saturate)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_matches_torch_copy(dev):
    """inv_scale = 1, copy mode: the same bytes as the pages' aten::copy_ path,
    pool[slots] = src.to(float8_e4m3fn)."""
    src = workloads.new_kv_rows(500, seed=5, device=dev, sigma=30.0, outlier_frac=0.02)
    pool = workloads.random_pool(2048, seed=6, device=dev)
    slots = torch.from_numpy(workloads.free_slots(500, 2048, seed=7)).to(dev)
    theirs = pool.clone()
    theirs[slots.long()] = src.to(torch.float8_e4m3fn).view(torch.uint8)
    fm.scatter_cast_bf16_fp8(src, slots, pool)
    torch.cuda.synchronize()
    assert torch.equal(pool, theirs)


@pytest.mark.parametrize("n", [1, 7, 8, 31, 32, 33, 40, 1000, 4097])
def test_ragged_row_counts(dev, n):
    src = workloads.new_kv_rows(n, seed=n, sigma=4.0, outlier_frac=0.01)
    pool0 = workloads.random_pool(n + 300, seed=n + 1).numpy()
    slots = workloads.free_slots(n, n + 300, seed=n + 2)
    got = _run(dev, src, slots, pool0, 0.75, False)
    assert np.array_equal(got, oracle.scatter_ref(pool0, bf16_bits(src), slots, np.float32(0.75)))


def test_out_of_range_slots_are_skipped(dev):
    n = 64
    src = workloads.new_kv_rows(n, seed=1)
    pool0 = workloads.random_pool(100, seed=2).numpy()
    slots = workloads.free_slots(n, 100, seed=3)
    slots[::5] = -1
    slots[1::7] = 100
    slots[2::11] = np.iinfo(np.int32).min
    slots[3::13] = np.iinfo(np.int32).max
    got = _run(dev, src, slots, pool0, 1.0, False)
    ref = oracle.scatter_ref(pool0, bf16_bits(src), slots, 1.0)
    assert np.array_equal(got, ref)
    kept = [s for s in slots if 0 <= s < 100]
    assert len(kept) < n and np.array_equal(np.delete(got, kept, 0), np.delete(pool0, kept, 0))


def test_strided_and_3d_sources(dev):
    n = 70
    wide = workloads.new_kv_rows(n, seed=9).repeat(1, 2)[:, :640].contiguous()   # row stride 640
    src = wide[:, :576]
    assert src.stride(0) == 640 and not src.is_contiguous()
    pool0 = workloads.random_pool(200, seed=10).numpy()
    slots = workloads.free_slots(n, 200, seed=11)
    ref = oracle.scatter_ref(pool0, bf16_bits(src.contiguous()), slots, 2.0, True)
    assert np.array_equal(_run(dev, src, slots, pool0, 2.0, True), ref)
    got3 = _run(dev, src.contiguous().view(n, 1, 576), slots, pool0, 2.0, True)
    assert np.array_equal(got3, ref)
    pool_f8 = torch.from_numpy(pool0).to(dev).view(torch.float8_e4m3fn).view(200, 1, 576)
    fm.scatter_cast_bf16_fp8(src.to(dev), torch.from_numpy(slots).to(dev), pool_f8, 2.0, True)
    torch.cuda.synchronize()
    assert np.array_equal(pool_f8.view(torch.uint8).view(200, 576).cpu().numpy(), ref)


def test_empty_is_a_no_op(dev):
    pool = workloads.random_pool(10, seed=1, device=dev)
    before = pool.clone()
    fm.scatter_cast_bf16_fp8(torch.empty((0, 576), dtype=torch.bfloat16, device=dev),
                             torch.empty(0, dtype=torch.int32, device=dev), pool)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)


def test_round_trip_through_the_read_path(dev):
    """Rows written by the write path and read back by gather_cast give the
    nearest E4M3FN values of the source (within half a step, or NaN past 464)."""
    n = 256
    src = workloads.new_kv_rows(n, seed=21, sigma=3.0, device=dev)
    pool = workloads.random_pool(1000, seed=22, device=dev)
    slots = torch.from_numpy(workloads.free_slots(n, 1000, seed=23)).to(dev)
    fm.scatter_cast_bf16_fp8(src, slots, pool)
    back = fm.gather_cast_fp8_bf16(pool, slots)
    torch.cuda.synchronize()
    assert torch.equal(back, src.to(torch.float8_e4m3fn).to(torch.bfloat16))


@pytest.mark.parametrize("n", [40, 16384])
def test_decode_step_and_extend_chunk_in_a_layer_pool(dev, n):
    """A decode step's 40 new rows and a 16k-row extend chunk, written into one
    layer's 495,552-slot pool: written rows match the oracle, every other row
    of the pool is unchanged."""
    num_slots = 495552
    pool = workloads.random_pool(num_slots, seed=31, device=dev)
    before = pool.clone()
    src = workloads.new_kv_rows(n, seed=32, device=dev, outlier_frac=0.001)
    slots_np = workloads.free_slots(n, num_slots, seed=33)
    slots = torch.from_numpy(slots_np).to(dev)
    fm.scatter_cast_bf16_fp8(src, slots, pool, 1.0 / 1.5)
    torch.cuda.synchronize()
    written = pool[slots.long()].cpu().numpy()
    ref = oracle.scatter_ref(np.zeros((n, 576), np.uint8), bf16_bits(src), np.arange(n),
                             np.float32(1.0 / 1.5))
    assert np.array_equal(written, ref)
    mask = torch.ones(num_slots, dtype=torch.bool, device=dev)
    mask[slots.long()] = False
    assert torch.equal(pool[mask], before[mask])
