"""GPU parity of the fused FP8 MLA decode against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, attention_errors, bf16_bits, oracle_args

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _run(w):
    out = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale)
    torch.cuda.synchronize()
    return out


def _check_full(w, label):
    out = _run(w)
    ref = oracle.mla_decode_ref(*oracle_args(w))
    return assert_attention_close(out, ref, label)


def test_config1_tiny(dev):
    e = _check_full(workloads.config(1, device=dev), "config1")
    print("config1", e)


@pytest.mark.parametrize("H", [1, 8, 16, 17, 32, 64, 128])
def test_head_counts(dev, H):
    w = workloads.small(3, H, [1, 130, 37], seed=H, device=dev)
    _check_full(w, "H=%d" % H)


@pytest.mark.parametrize("lengths", [
    [1], [2], [127], [128], [129], [255, 1, 3], [0, 5, 0], [64] * 7, [1] * 40,
])
def test_ragged_lengths(dev, lengths):
    w = workloads.small(len(lengths), 16, lengths, seed=len(lengths) + sum(lengths), device=dev)
    _check_full(w, str(lengths))


# Many short requests: segments start at nearly every request index, on
# both sides of the first 64-entry kv_indptr window that the segment search
# hands to the tile cursor (segments start at requests 62, 63 and 65; request
# 64 is empty, so the cursor steps over it from 63).
@pytest.mark.parametrize("seed", [0, 1])
def test_many_requests_across_indptr_windows(dev, seed):
    rng = np.random.default_rng(700 + seed)
    lengths = [int(x) for x in rng.integers(1, 200, size=200)]
    lengths[64] = 0
    lengths[130] = 0
    w = workloads.small(len(lengths), 16, lengths, seed=seed, device=dev)
    _check_full(w, "B=200 seed %d" % seed)


# 64 or more heads with enough tokens (at least 4 64-token tiles per
# workgroup slot: 4 * CUs / ceil(H / 64) tiles) run the 64-heads-per-workgroup
# kernel.  Sizes just above that threshold cover padding (80 = 64 + 16),
# several head sets, ragged and empty requests, many short requests (many
# query switches) and requests spanning many segments.
def _h64_tokens(H):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 64 * (4 * cus // ((H + 63) // 64)) + 64


@pytest.mark.parametrize("H,shape", [
    (64, "two_long"),
    (80, "ragged"),
    (128, "ragged"),
    (128, "many_short"),
    (256, "two_long"),
])
def test_high_head_counts(dev, H, shape):
    need = _h64_tokens(H)
    if shape == "two_long":
        lengths = [need // 2 + 37, 1, 0, need // 2 + 5]
    elif shape == "ragged":
        lengths = [need // 3, 63, 0, 65, need // 3 + 1, need // 3 + 200]
    else:
        lengths = [300 + (7 * i) % 64 for i in range(need // 300 + 2)]
    assert sum(lengths) >= need
    w = workloads.small(len(lengths), H, lengths, seed=H + len(lengths), device=dev)
    e = _check_full(w, "H=%d %s" % (H, shape))
    print("H=%d %s tokens=%d" % (H, shape, sum(lengths)), e)


def test_high_head_counts_half_tile_edges(dev):
    """The 64-head kernel works in half-tiles of 32 tokens: requests that end
    inside, at or just past a half-tile or tile boundary (so that a tile's
    second half is empty or a request switch follows its first half),
    hundreds of query switches, at two head sets."""
    H = 128
    pattern = [1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 0]
    need = _h64_tokens(H)
    lengths = pattern * (need // sum(pattern) + 1)
    w = workloads.small(len(lengths), H, lengths, seed=31, device=dev)
    e = _check_full(w, "H=%d half-tile edges" % H)
    print("H=%d requests=%d tokens=%d" % (H, len(lengths), sum(lengths)), e)


@pytest.mark.parametrize("kind", ["16-head", "64-head"])
def test_split_count_invariance(dev, kind):
    """The result does not depend on the split-K partition beyond rounding:
    the same call cut into at most 1 (no merge), 2 and 7 segments and into
    the library's own count each matches the oracle, and a bound above the
    library's own count changes nothing."""
    if kind == "16-head":
        w = workloads.small(5, 16, [3000, 50, 9000, 1, 700], seed=5, device=dev, scale=1.3)
    else:
        need = _h64_tokens(128)
        w = workloads.small(3, 128, [need // 2 + 300, 90, need // 2 + 77], seed=6, device=dev)
    ref = oracle.mla_decode_ref(*oracle_args(w))
    outs = {}
    for S in (1, 2, 7, None, 10 ** 6):
        out = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale, segments=S)
        torch.cuda.synchronize()
        e = assert_attention_close(out, ref, "%s segments=%s" % (kind, S))
        print(kind, "segments", S, e)
        outs[S] = out
    assert torch.equal(outs[None], outs[10 ** 6])


@pytest.mark.parametrize("sm_scale", [-0.07, 0.0, 1e-30])
@pytest.mark.parametrize("H", [16, 128])
def test_sm_scale_sign_and_zero(dev, H, sm_scale):
    """The ABI accepts any finite sm_scale.  A negative one flips every
    score, zero makes the attention a plain mean of the visible values, a
    tiny one nearly so; the 64-head kernel takes its maxima on unscaled sums
    and handles a non-positive scale through the query (negated or zeroed)."""
    n = _h64_tokens(H) if H >= 64 else 3000
    w = workloads.small(3, H, [n // 2 + 17, 40, n // 2 + 3], seed=41, device=dev,
                        sm_scale=sm_scale)
    e = _check_full(w, "H=%d sm_scale=%g" % (H, sm_scale))
    print("H=%d sm_scale=%g" % (H, sm_scale), e)


@pytest.mark.parametrize("H", [16, 128])
def test_trailing_empty_requests(dev, H):
    """Long requests followed by 150 empty ones (more than a 64-entry window
    of the request list past the last tile): the tile cursors stop at the
    segment's last tile instead of walking the empty tail."""
    n = _h64_tokens(H) if H >= 64 else 5000
    lengths = [n // 2 + 11, 70, n // 2 + 5] + [0] * 150
    w = workloads.small(len(lengths), H, lengths, seed=57, device=dev)
    e = _check_full(w, "H=%d trailing empty" % H)
    print("H=%d trailing empty requests" % H, e)


def test_all_requests_empty(dev):
    w = workloads.small(4, 16, [0, 0, 0, 0], num_slots=64, device=dev)
    out = _run(w)
    assert torch.count_nonzero(out.float()).item() == 0


def test_requests_span_many_segments(dev):
    # 3000 + 50 + 9000 tokens -> many segments per request, exercising the combine
    w = workloads.small(3, 16, [3000, 50, 9000], seed=11, device=dev, scale=1.7)
    e = _check_full(w, "multi-segment")
    print("multi-segment", e)


@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_layout(dev, page_size):
    w = workloads.small(5, 32, [700, 64, 65, 1, 2049], page_size=page_size, seed=page_size,
                        device=dev)
    _check_full(w, "page=%d" % page_size)


def test_large_scores_and_outliers(dev):
    # saturated +-448 values and a large q: near one-hot softmax
    w = workloads.small(2, 16, [300, 1000], seed=5, device=dev, q_sigma=4.0, outlier_frac=0.02)
    _check_full(w, "outliers")


def test_query_zero_gives_mean(dev):
    w = workloads.small(2, 16, [333, 20], seed=6, device=dev)
    w.q.zero_()
    _check_full(w, "q=0")


def test_nan_rows_do_not_leak_across_requests(dev):
    # request 1's rows contain NaN codes; request 0 (sharing a 128-token tile) must stay exact
    w = workloads.small(2, 16, [50, 40], seed=7, device=dev)
    idx1 = w.indices[50:90].long()
    w.pool[idx1, 5] = 0x7F
    out = _run(w)
    args = oracle_args(w)
    ref0 = oracle.mla_decode_ref(*args, requests=[0])
    assert_attention_close(out[0:1], ref0, "nan isolation")
    assert torch.isnan(out[1].float()).any()


def test_deterministic(dev):
    w = workloads.small(3, 16, [900, 17, 2000], seed=8, device=dev)
    a = _run(w)
    b = _run(w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_reuse_across_shapes(dev):
    # One workspace, filled with garbage first, reused by calls of different
    # shapes (split requests, head groups): the workspace is pure scratch,
    # every call must match the oracle.
    shapes = [(3, 32, [3000, 50, 9000]), (5, 16, [700, 1, 0, 2049, 130]), (2, 17, [4000, 4000]),
              (40, 16, [1500 + 37 * i for i in range(40)])]
    need = max(fm.mla_decode_fp8_workspace_bytes(len(L), H, sum(L), dev) for _, H, L in shapes)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)
    for rep in range(2):
        for i, (B, H, L) in enumerate(shapes):
            w = workloads.small(B, H, L, seed=100 + i, device=dev)
            out = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale,
                                    workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.mla_decode_ref(*oracle_args(w))
            assert_attention_close(out, ref, "reuse %d/%d" % (rep, i))


def test_workspace_shared_with_other_entry_points(dev):
    # One garbage-filled workspace shared by the FP8 decode, the BF16 decode
    # and the extend path (one query token per request, which is decode),
    # called in turn twice: each call overwrites what the others left.
    w = workloads.small(6, 16, [2100, 900, 4000, 64, 3000, 1200], seed=31, device=dev)
    need = max(fm.mla_decode_fp8_workspace_bytes(w.B, w.H, w.total_tokens, dev),
               fm.mla_decode_bf16_workspace_bytes(w.B, w.H, w.total_tokens, dev),
               fm.mla_extend_fp8_workspace_bytes(w.B, w.H, w.B, dev))
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)
    ref = oracle.mla_decode_ref(*oracle_args(w))
    rows16 = fm.cast_pool_fp8_bf16(w.pool)
    qo = torch.arange(w.B + 1, dtype=torch.int32, device=dev)
    for rep in range(2):
        a = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale, workspace=ws)
        b = fm.mla_decode_bf16(w.q, rows16, w.indptr, w.indices, w.scale, w.sm_scale, workspace=ws)
        c = fm.mla_extend_fp8(w.q.reshape(w.B, w.H, -1), w.pool, qo, w.indptr, w.indices, w.scale,
                              w.sm_scale, causal=False, workspace=ws)
        torch.cuda.synchronize()
        for name, out in (("fp8", a), ("bf16", b), ("extend", c)):
            assert_attention_close(out, ref, "shared workspace %s %d" % (name, rep))


def test_slot_relocation_invariance(dev):
    w = workloads.small(2, 16, [400, 300], seed=9, device=dev)
    a = _run(w)
    g = torch.Generator().manual_seed(0)
    perm = torch.randperm(w.num_slots, generator=g).to(dev)
    moved = torch.empty_like(w.pool)
    moved[perm] = w.pool
    w2 = workloads.Workload(w.name, w.seed, w.B, w.H, w.page_size, w.num_slots, w.lengths, moved,
                            w.indptr, perm[w.indices.long()].to(torch.int32).contiguous(), w.q,
                            w.scale, w.sm_scale)
    b = _run(w2)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _full_call(w, label):
    """The whole call against the oracle, every request and head; the literal
    absolute errors are printed beside the relative ones."""
    print("case:", label, "B=%d H=%d tokens=%d" % (w.B, w.H, w.total_tokens), flush=True)
    out = _run(w)
    ref = oracle.mla_decode_ref(*oracle_args(w))
    e = assert_attention_close(out, ref, label)
    print(label, e, flush=True)
    return e


@pytest.mark.parametrize("replica", [0, 1, 2, 3])
def test_config2_batch40_full(dev, replica):
    """Every request of each of the four replicas the benchmark rotates."""
    _full_call(workloads.config(2, replica, device=dev), "config2 replica %d" % replica)


def test_config3_layer_full(dev):
    w = workloads.config(3, device=dev)
    _check_full(w, "config3")


def test_config4_long_context_full(dev):
    _full_call(workloads.config(4, device=dev), "config4")


def test_config5_serving_mix_full(dev):
    _full_call(workloads.config(5, device=dev), "config5")


def test_workspace_size_does_not_grow_with_tokens(dev):
    """The split-K scratch is two partial pieces per segment and head row plus
    8 bytes per request: one size per (batch, heads), whatever the tokens."""
    for B, H in [(1, 16), (40, 16), (8, 128), (256, 16), (3, 100), (2, 64)]:
        sizes = {fm.mla_decode_fp8_workspace_bytes(B, H, n, dev) for n in [1, 1000, 10 ** 6, 10 ** 9]}
        assert len(sizes) == 1, (B, H, sizes)


def test_prepared_call_reuses_buffers(dev):
    """The prepared path re-issues the same call on the same buffers: new
    contents written into them between calls give the new results."""
    w = workloads.small(4, 16, [900, 1, 3000, 128], seed=71, device=dev)
    call = fm.prepare_mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale)
    a = call().clone()
    torch.cuda.synchronize()
    assert_attention_close(a, oracle.mla_decode_ref(*oracle_args(w)), "prepared 1")
    w.q.copy_(workloads.random_q(w.B, w.H, seed=72, device=dev))
    b = call()
    torch.cuda.synchronize()
    assert b.data_ptr() == call.result.data_ptr()
    assert_attention_close(b, oracle.mla_decode_ref(*oracle_args(w)), "prepared 2")
    assert not torch.equal(a, b)


@pytest.mark.parametrize("n", [1, 64, 128, 129, 256, 257, 400])
def test_single_request_small_plans(dev, n):
    """One request of up to a few tiles: the plan knows its tile count, and
    with a single segment no combine kernel is launched."""
    for H in (16, 64):
        w = workloads.small(1, H, [n], seed=n + H, device=dev)
        _check_full(w, "B=1 n=%d H=%d" % (n, H))
