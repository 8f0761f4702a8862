"""GPU parity of the BF16-row decode (the cast-then-attend fallback's
attention) against the float64 oracle.  Its rows are the exact BF16 images of
E4M3 rows, so the oracle of the FP8 pool is the oracle of the BF16 rows."""
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, oracle_args

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _check_cast_pool_path(w, label):
    kv = fm.cast_pool_fp8_bf16(w.pool)
    out = fm.mla_decode_bf16(w.q, kv, w.indptr, w.indices, w.scale, w.sm_scale)
    torch.cuda.synchronize()
    ref = oracle.mla_decode_ref(*oracle_args(w))
    return assert_attention_close(out, ref, label)


def test_tiny(dev):
    _check_cast_pool_path(workloads.config(1, device=dev), "bf16 config1")


@pytest.mark.parametrize("H", [1, 16, 17, 64])
def test_head_counts(dev, H):
    w = workloads.small(3, H, [1, 130, 37], seed=50 + H, device=dev)
    _check_cast_pool_path(w, "bf16 H=%d" % H)


@pytest.mark.parametrize("lengths", [[1], [63], [64], [65], [255, 1, 3], [0, 5, 0], [1] * 40])
def test_ragged_lengths(dev, lengths):
    w = workloads.small(len(lengths), 16, lengths, seed=7 + sum(lengths), device=dev)
    _check_cast_pool_path(w, "bf16 %s" % lengths)


def test_requests_span_many_segments(dev):
    w = workloads.small(3, 16, [3000, 50, 9000], seed=12, device=dev, scale=1.7)
    _check_cast_pool_path(w, "bf16 multi-segment")


def test_gather_path_matches(dev):
    # gather-then-cast: attention over the compact buffer with indices 0..n-1
    w = workloads.small(4, 16, [700, 64, 1, 2049], page_size=16, seed=31, device=dev)
    kv = fm.gather_cast_fp8_bf16(w.pool, w.indices)
    seq = torch.arange(w.indices.numel(), dtype=torch.int32, device=dev)
    out = fm.mla_decode_bf16(w.q, kv, w.indptr, seq, w.scale, w.sm_scale)
    torch.cuda.synchronize()
    assert_attention_close(out, oracle.mla_decode_ref(*oracle_args(w)), "bf16 gather path")


def test_agrees_with_fp8_kernel(dev):
    w = workloads.small(5, 32, [700, 64, 65, 1, 2049], seed=3, device=dev)
    a = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale)
    b = fm.mla_decode_bf16(w.q, fm.cast_pool_fp8_bf16(w.pool), w.indptr, w.indices, w.scale,
                           w.sm_scale)
    torch.cuda.synchronize()
    ref = oracle.mla_decode_ref(*oracle_args(w))
    assert_attention_close(a, ref, "fp8")
    assert_attention_close(b, ref, "bf16")


def test_config3_layer(dev):
    w = workloads.config(3, device=dev)
    _check_cast_pool_path(w, "bf16 config3")


def test_empty(dev):
    w = workloads.small(3, 16, [0, 0, 0], num_slots=64, device=dev)
    out = fm.mla_decode_bf16(w.q, fm.cast_pool_fp8_bf16(w.pool), w.indptr, w.indices, w.scale,
                             w.sm_scale)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()).item() == 0


@pytest.mark.parametrize("H", [16, 64, 100, 128])
def test_outliers_and_large_scores(dev, H):
    """1% of cache values at +-448 with queries 4 x N(0,1) and scale 2: near
    one-hot softmax over values of opposite sign that cancel, the case in
    which BF16 probabilities (8 significant bits) miss the tolerance."""
    w = workloads.small(5, H, [700, 64, 65, 1, 2049], seed=60 + H, device=dev, scale=2.0,
                        q_sigma=4.0, outlier_frac=0.01)
    e = _check_cast_pool_path(w, "bf16 outliers H=%d" % H)
    print("bf16 outliers H=%d" % H, e, flush=True)


@pytest.mark.parametrize("H", [100, 128])
def test_high_head_counts(dev, H):
    w = workloads.small(3, H, [3000, 50, 9000], seed=H, device=dev, scale=1.3)
    _check_cast_pool_path(w, "bf16 H=%d" % H)


def test_config5_serving_mix_full(dev):
    """The serving mix (256 requests, 1% +-448 outliers, q = 2 N(0,1)) through
    the BF16 rows of its cast pool: every request against the oracle."""
    w = workloads.config(5, device=dev)
    e = _check_cast_pool_path(w, "bf16 config5")
    print("bf16 config5", e, flush=True)
