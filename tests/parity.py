"""Shared helpers for GPU parity tests: tensor <-> numpy marshalling and the
attention tolerance."""
import numpy as np
import torch

# Tolerance for BF16 attention outputs against the float64 oracle, per
# element, relative to max(1, |reference|): max <= 2e-2 and mean <= 2e-3.
# Where |reference| <= 1 this is the plain absolute bound; above 1 it scales
# with the value, since BF16's own rounding step (half an ulp, 2^-9 relative)
# already exceeds 2e-2 in absolute terms once |out| >= 8.
MAX_TOL = 2e-2
MEAN_TOL = 2e-3


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_args(w):
    return (bf16_bits(w.q), w.pool.cpu().numpy(), w.indptr.cpu().numpy(),
            w.indices.cpu().numpy(), w.scale, w.sm_scale)


def attention_errors(got_bf16: torch.Tensor, ref: np.ndarray):
    got = got_bf16.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    absd = np.abs(got - ref)
    rel = absd / np.maximum(1.0, np.abs(ref))
    return {
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "mean_rel": float(rel.mean()) if rel.size else 0.0,
        "max_abs": float(absd.max()) if absd.size else 0.0,
        "mean_abs": float(absd.mean()) if absd.size else 0.0,
        "n_ge8": int((np.abs(ref) >= 8).sum()),
        "finite": bool(np.all(np.isfinite(got))),
    }


def assert_attention_close(got_bf16, ref, label=""):
    e = attention_errors(got_bf16, ref)
    assert e["finite"], (label, e)
    assert e["max_rel"] <= MAX_TOL and e["mean_rel"] <= MEAN_TOL, (label, e)
    return e
