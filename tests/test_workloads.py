"""Host-side checks of the seeded input generator (no GPU, no method arithmetic)."""
import numpy as np
import torch

import workloads


def test_config1_shape_and_determinism():
    a = workloads.config(1)
    b = workloads.config(1)
    assert a.pool.shape == (1024, 576) and a.pool.dtype == torch.uint8
    assert a.q.shape == (1, 16, 576) and a.q.dtype == torch.bfloat16
    assert a.indptr.tolist() == [0, 64]
    assert len(set(a.indices.tolist())) == 64
    assert torch.equal(a.pool, b.pool) and torch.equal(a.q, b.q) and torch.equal(a.indices, b.indices)


def test_page1_slots_disjoint():
    rng = np.random.default_rng(3)
    s = workloads.assign_slots([5, 9, 1], 40, 1, rng)
    assert len(s) == 15 and len(set(s.tolist())) == 15 and s.max() < 40


def test_paged_layout():
    rng = np.random.default_rng(4)
    lengths = [130, 64, 1]
    s = workloads.assign_slots(lengths, 64 * 16, 64, rng)
    assert len(s) == 195 and len(set(s.tolist())) == 195
    r0 = s[:130]
    # within a page the slots are consecutive and the page base is 64-aligned
    for p in range(3):
        seg = r0[64 * p: 64 * (p + 1)]
        assert seg[0] % 64 == 0
        assert np.array_equal(seg, seg[0] + np.arange(len(seg)))


def test_values_are_finite_e4m3_and_clipped():
    w = workloads.small(2, 16, [3, 70], outlier_frac=0.05, seed=2)
    vals = w.pool.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(vals).all()
    assert vals.abs().max().item() == 448.0
