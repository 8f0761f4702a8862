"""GPU parity of the extend (prefill) attention mla_extend_fp8 against the
float64 oracle: several query tokens per request, causal or not, ragged
token counts, head counts on both sides of 64, blocks spanning segments,
tokens that see nothing, and the named extend workloads (every row)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, bf16_bits

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _args(w):
    return (bf16_bits(w.q), w.pool.cpu().numpy(), w.qo_indptr.cpu().numpy(),
            w.kv_indptr.cpu().numpy(), w.kv_indices.cpu().numpy(), w.scale, w.sm_scale)


def _run(w, dev, **kw):
    out = fm.mla_extend_fp8(w.q.to(dev), w.pool.to(dev), w.qo_indptr.to(dev), w.kv_indptr.to(dev),
                            w.kv_indices.to(dev), w.scale, w.sm_scale, causal=w.causal, **kw)
    torch.cuda.synchronize()
    return out


def _check(w, dev, label="", rows=None):
    print("case:", label, w.name, "q_lens", w.q_lens.tolist()[:8], "kv_lens", w.kv_lens.tolist()[:8],
          flush=True)
    got = _run(w, dev)
    ref = oracle.mla_extend_ref(*_args(w), causal=w.causal, rows=rows)
    g = got if rows is None else got[torch.as_tensor(rows, device=got.device)]
    return assert_attention_close(g, ref, label)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("H", [16, 8, 32, 48, 64, 128])
def test_head_counts(dev, H, causal):
    w = workloads.extend(3, H, [5, 1, 9], [40, 200, 3], seed=H, causal=causal, scale=1.5)
    _check(w, dev, "H=%d causal=%s" % (H, causal))


@pytest.mark.parametrize("sm_scale", [-0.07, 0.0])
@pytest.mark.parametrize("H", [16, 64])
def test_sm_scale_sign_and_zero(dev, H, sm_scale):
    """Any finite sm_scale: negative flips the scores, zero gives the mean of
    each token's visible values (the kernel negates or zeroes the query)."""
    w = workloads.extend(3, H, [5, 1, 9], [40, 200, 3], seed=H + 3, causal=True,
                         sm_scale=sm_scale, scale=1.2)
    _check(w, dev, "H=%d sm_scale=%g" % (H, sm_scale))


@pytest.mark.parametrize("q_lens,history", [
    ([1], [0]),                          # one token, no history
    ([2, 3, 4, 5], [0, 1, 63, 64]),      # ragged blocks around the 4-token block size
    ([7, 0, 13], [100, 50, 129]),        # a request without query tokens
    ([64], [0]),                         # prefill from scratch
    ([33, 17], [500, 1000]),
])
def test_ragged_blocks(dev, q_lens, history):
    w = workloads.extend(len(q_lens), 16, q_lens, history, seed=len(q_lens) + sum(q_lens))
    _check(w, dev, "ragged %s/%s" % (q_lens, history))


@pytest.mark.parametrize("q_lens", [
    [12] * 64,               # 64 requests, 256 list entries: the split kernel lays out the list
    [12] * 63 + [13],        # 257 entries: the pre-pass kernel does
    [1] * 65,                # 65 requests: the pre-pass kernel does
    [0, 9, 0, 30, 1, 0, 17, 3] * 8,  # 64 requests, empty ones, 144 list entries in three chunks
])
def test_list_in_kernel_and_prepass(dev, q_lens):
    """Calls of at most 64 requests and 256 virtual requests have their list
    built inside the split kernel, larger ones by the pre-pass kernel: both
    sides of both limits against the oracle."""
    rng = np.random.default_rng(len(q_lens) + sum(q_lens))
    history = rng.integers(0, 300, size=len(q_lens))
    w = workloads.extend(len(q_lens), 16, q_lens, history, seed=len(q_lens), causal=True)
    _check(w, dev, "list B=%d total_q=%d" % (len(q_lens), sum(q_lens)))


def test_one_token_per_request_matches_decode(dev):
    w = workloads.extend(6, 16, [1] * 6, [300, 1, 2000, 77, 64, 640], seed=11, scale=0.75)
    got = _run(w, dev)
    ref = oracle.mla_extend_ref(*_args(w))
    assert_attention_close(got, ref, "q_len 1")
    dec = fm.mla_decode_fp8(w.q.to(dev), w.pool.to(dev), w.kv_indptr.to(dev), w.kv_indices.to(dev),
                            w.scale, w.sm_scale)
    torch.cuda.synchronize()
    assert_attention_close(dec, ref, "decode")


def test_blocks_span_many_segments(dev):
    """Enough tokens that virtual requests are cut across several segments,
    so their partials go through the combine."""
    w = workloads.extend(2, 16, [8, 6], [6000, 9000], seed=12)
    _check(w, dev, "multi-segment")
    w = workloads.extend(1, 128, [3], [7000], seed=13)
    _check(w, dev, "multi-segment H=128")


def test_tokens_that_see_nothing_get_zero_rows(dev):
    # kv_len < q_len: the first tokens of request 0 see no cache token
    w = workloads.extend(2, 16, [6, 2], [0, 5], seed=14)
    kv = w.kv_lens.copy()
    kv[0] = 3
    w.kv_lens = kv
    ind = np.concatenate([[0], np.cumsum(kv)])
    w.kv_indptr = torch.from_numpy(ind.astype(np.int32))
    w.kv_indices = w.kv_indices[: int(ind[-1])].contiguous()
    e = _check(w, dev, "kv_len < q_len")
    got = _run(w, dev).float().cpu()
    assert torch.all(got[0:3] == 0)


def test_no_cache_tokens_at_all(dev):
    w = workloads.extend(2, 16, [3, 2], [0, 0], seed=15)
    w.kv_lens = np.zeros(2, dtype=np.int64)
    w.kv_indptr = torch.zeros(3, dtype=torch.int32)
    w.kv_indices = torch.zeros(0, dtype=torch.int32)
    got = _run(w, dev)
    assert torch.all(got.float() == 0)


def test_workspace_garbage_and_reuse(dev):
    shapes = [([4, 9], [700, 30], 16), ([1, 1, 1], [5000, 2, 9], 16), ([12], [3000], 64)]
    ws = torch.empty(1 << 27, dtype=torch.uint8, device=dev).random_(0, 256)
    for rep in range(2):
        for k, (ql, hist, H) in enumerate(shapes):
            w = workloads.extend(len(ql), H, ql, hist, seed=20 + k)
            need = fm.mla_extend_fp8_workspace_bytes(w.B, H, w.total_q)
            assert need <= ws.numel()
            got = fm.mla_extend_fp8(w.q.to(dev), w.pool.to(dev), w.qo_indptr.to(dev),
                                    w.kv_indptr.to(dev), w.kv_indices.to(dev), w.scale, w.sm_scale,
                                    workspace=ws)
            torch.cuda.synchronize()
            assert_attention_close(got, oracle.mla_extend_ref(*_args(w)), "reuse %d/%d" % (rep, k))


def test_deterministic(dev):
    w = workloads.extend(2, 32, [9, 4], [3000, 800], seed=30)
    a = _run(w, dev)
    b = _run(w, dev)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", list(workloads.EXTEND_NAMES))
def test_named_extend_workloads_full(dev, name):
    """Every query row of the named extend workloads the benchmark times."""
    w = workloads.extend_config(name, device="cpu")
    e = _check(w, dev, name)
    print(name, e, flush=True)


def test_prefill_past_2_29_visible_pairs(dev):
    """A causal prefill of 32,768 tokens at 64 heads: 536,887,296 (token,
    visible token) pairs, past 2^29, which an earlier layout of the block CSR
    could not address.  The whole call runs; the oracle checks the rows that
    see the most tokens (the last ones), a row from each quarter, and the
    first."""
    n = 32768
    w = workloads.extend(1, 64, [n], [0], seed=77)
    assert w.visible_tokens() > 1 << 29
    rows = np.array([0, n // 4, n // 2, 3 * n // 4, n - 2, n - 1])
    e = _check(w, dev, "prefill 32k H=64", rows=rows)
    print("prefill 32k", e, flush=True)


@pytest.mark.parametrize("H", [256, 96])
def test_more_than_64_heads(dev, H):
    """Several 64-head sets per token block (H = 256: four; H = 96: two, the
    second half empty)."""
    w = workloads.extend(2, H, [3, 2], [150, 70], seed=H + 1)
    _check(w, dev, "H=%d" % H)


@pytest.mark.parametrize("causal", [True, False])
def test_paged_layout(dev, causal):
    """Slots laid out in 64-slot pages (runs of consecutive slots from scattered
    page bases, last page partial), as in the long-context workload."""
    w = workloads.extend(3, 16, [9, 4, 17], [200, 63, 500], page_size=64, seed=41, causal=causal)
    _check(w, dev, "paged causal=%s" % causal)


def test_large_scores_and_outliers(dev):
    """Queries 4x N(0,1) over a pool with 1% +-448 outliers: near one-hot softmax."""
    w = workloads.extend(2, 32, [5, 8], [300, 90], seed=43, q_sigma=4.0, outlier_frac=0.01,
                         scale=2.0)
    _check(w, dev, "outliers")
