"""GPU parity of the two cast kernels against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import bf16_bits

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _all_codes_pool(rows):
    codes = np.arange(rows * 576) % 256
    return torch.from_numpy(codes.astype(np.uint8).reshape(rows, 576))


# 1-3 rows: less than one 2 KB chunk; 4, 37, 1000: a few chunks and a tail;
# 100003: 27-28 chunks per wave over 1,024 waves and a 1,728-byte tail
@pytest.mark.parametrize("rows", [1, 3, 4, 37, 1000, 100003])
def test_cast_pool_all_codes(dev, rows):
    pool = _all_codes_pool(rows)
    out = fm.cast_pool_fp8_bf16(pool.to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), oracle.cast_ref(pool.numpy()))


def test_cast_pool_accepts_fp8_dtype_and_3d_view(dev):
    pool = _all_codes_pool(8).to(dev)
    a = fm.cast_pool_fp8_bf16(pool.view(torch.float8_e4m3fn).view(8, 1, 576))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(a).reshape(8, 576), oracle.cast_ref(pool.cpu().numpy()))


def test_cast_pool_matches_torch_to(dev):
    # the pages' path is torch's .to(bfloat16); it must agree bit for bit
    pool = _all_codes_pool(64).to(dev)
    ours = fm.cast_pool_fp8_bf16(pool)
    theirs = pool.view(torch.float8_e4m3fn).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(ours), bf16_bits(theirs))


def test_cast_pool_layer_sized(dev):
    # one layer of the pages' pool: 495,552 slots x 576
    pool = workloads.random_pool(495552, seed=3003, device=dev, outlier_frac=0.01)
    out = fm.cast_pool_fp8_bf16(pool)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), oracle.cast_ref(pool.cpu().numpy()))


@pytest.mark.parametrize("n", [1, 15, 16, 63, 64, 65, 4096, 184321])
def test_gather_cast_random(dev, n):
    rng = np.random.default_rng(n)
    pool = _all_codes_pool(300)
    pool = pool[torch.from_numpy(rng.permutation(300))].contiguous()
    idx = rng.integers(0, 300, size=n).astype(np.int32)
    out = fm.gather_cast_fp8_bf16(pool.to(dev), torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), oracle.gather_ref(pool.numpy(), idx))


def test_gather_cast_empty(dev):
    pool = _all_codes_pool(4).to(dev)
    out = fm.gather_cast_fp8_bf16(pool, torch.zeros(0, dtype=torch.int32, device=dev))
    assert out.shape == (0, 576)


def test_gather_cast_active_slots_of_a_request_mix(dev):
    w = workloads.config(3, device=dev)
    out = fm.gather_cast_fp8_bf16(w.pool, w.indices)
    torch.cuda.synchronize()
    idx = w.indices.cpu().numpy()
    assert np.array_equal(bf16_bits(out), oracle.gather_ref(w.pool.cpu().numpy(), idx))


def test_gather_cast_clamps_out_of_range_indices(dev):
    pool = _all_codes_pool(10)
    idx = torch.tensor([0, 9, 10, 1 << 30, -1], dtype=torch.int32)
    out = fm.gather_cast_fp8_bf16(pool.to(dev), idx.to(dev))
    torch.cuda.synchronize()
    want = oracle.gather_ref(pool.numpy(), np.array([0, 9, 9, 9, 9]))
    assert np.array_equal(bf16_bits(out), want)
