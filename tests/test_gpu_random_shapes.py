"""GPU parity over randomly drawn (fixed-seed) shapes: decode and extend
against the float64 oracle, every output row checked.  Each case draws its
batch, head count, ragged lengths (empty requests included), page size,
per-tensor scale, query spread and outliers, so that combinations the
hand-written cases do not pair up are covered too; the decode cases with
many tokens at 64 or more heads run the 64-heads-per-workgroup kernel."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, bf16_bits, oracle_args

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")

HEADS = [1, 3, 16, 17, 31, 48, 64, 65, 100, 128, 200]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _decode_case(seed, cus):
    rng = np.random.default_rng(5100 + seed)
    big = seed % 4 == 0  # enough tokens at 64+ heads for the 64-heads-per-workgroup kernel
    H = int(rng.choice([64, 65, 100, 128, 200])) if big else int(rng.choice(HEADS))
    B = int(rng.integers(1, 48))
    if big:
        need = 64 * (4 * cus // ((H + 63) // 64)) + 64  # tokens that select that kernel
        lengths = rng.integers(need // B + 1, 2 * need // B + 2, size=B)
    else:
        lengths = rng.integers(0, max(2, 120000 // (B * H)), size=B)
        lengths[rng.random(B) < 0.15] = 0
    if lengths.sum() == 0:
        lengths[0] = 1
    page = int(rng.choice([1, 1, 16, 64]))
    return dict(B=B, H=H, lengths=lengths.tolist(), page_size=page, seed=seed,
                scale=float(rng.uniform(0.5, 2.0)), q_sigma=float(rng.choice([1.0, 3.0])),
                outlier_frac=float(rng.choice([0.0, 0.01])))


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(dev, seed):
    c = _decode_case(seed, torch.cuda.get_device_properties(0).multi_processor_count)
    print("case: decode seed", seed, {k: v for k, v in c.items() if k != "lengths"},
          "tokens", sum(c["lengths"]), flush=True)
    w = workloads.small(c["B"], c["H"], c["lengths"], page_size=c["page_size"], seed=c["seed"],
                        scale=c["scale"], q_sigma=c["q_sigma"], outlier_frac=c["outlier_frac"],
                        device=dev)
    out = fm.mla_decode_fp8(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale)
    torch.cuda.synchronize()
    ref = oracle.mla_decode_ref(*oracle_args(w))
    assert_attention_close(out, ref, "random decode %d" % seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_extend(dev, seed):
    rng = np.random.default_rng(6100 + seed)
    H = int(rng.choice([8, 16, 32, 48, 64, 100]))
    B = int(rng.integers(1, 9))
    q_lens = rng.integers(1, 40, size=B)
    history = rng.integers(0, 3000, size=B)
    history[rng.random(B) < 0.2] = 0
    causal = bool(seed % 4 != 3)
    page = int(rng.choice([1, 16]))
    print("case: extend seed", seed, "H", H, "B", B, "causal", causal, "page", page, flush=True)
    w = workloads.extend(B, H, q_lens, history, page_size=page, seed=seed, causal=causal,
                         scale=float(rng.uniform(0.5, 2.0)), q_sigma=float(rng.choice([1.0, 3.0])),
                         outlier_frac=float(rng.choice([0.0, 0.01])))
    out = fm.mla_extend_fp8(w.q.to(dev), w.pool.to(dev), w.qo_indptr.to(dev),
                            w.kv_indptr.to(dev), w.kv_indices.to(dev), w.scale, w.sm_scale,
                            causal=causal)
    torch.cuda.synchronize()
    ref = oracle.mla_extend_ref(bf16_bits(w.q), w.pool.cpu().numpy(), w.qo_indptr.cpu().numpy(),
                                w.kv_indptr.cpu().numpy(), w.kv_indices.cpu().numpy(), w.scale,
                                w.sm_scale, causal=causal)
    assert_attention_close(out, ref, "random extend %d" % seed)
