"""Invariants of the decode kernel's work split, on a Python model of its
integer formulas (no GPU).

Every request's tokens are cut into 128-token tiles; tile j of request b sits
at weighted position x = P_b + 2 + 4j (P_b: total weight 4*tiles + 2 of the
non-empty requests before b), and segment s of nseg = min(launched, W // 6)
takes the tiles with x in [ceil(s W / nseg), ceil((s+1) W / nseg)).  The
combine kernel relies on: the segments partition the tile list, none is empty,
and a request's tiles fall in the consecutive segments
floor(x_first nseg / W) .. floor(x_last nseg / W).
"""
import numpy as np
import pytest

TILE, TILE_W, START_W = 128, 4, 2


def split(lengths, launched):
    nt = [(int(L) + TILE - 1) // TILE for L in lengths]
    w = [TILE_W * n + START_W if n else 0 for n in nt]
    W = sum(w)
    if W == 0:
        return nt, None, None, 0
    nseg = min(launched, W // (TILE_W + START_W))
    P = np.concatenate([[0], np.cumsum(w)[:-1]]).astype(np.int64)
    TB = np.concatenate([[0], np.cumsum(nt)[:-1]]).astype(np.int64)
    T = sum(nt)

    def first_at(X):  # global index of the first tile at weighted position >= X
        for b, n in enumerate(nt):
            if n and P[b] + START_W + TILE_W * (n - 1) >= X:
                rel = X - P[b] - START_W
                return int(TB[b]) + (0 if rel <= 0 else -(-rel // TILE_W))
        return T

    owner = np.full(T, -1)
    for s in range(nseg):
        t0 = first_at(-(-s * W // nseg))
        t1 = first_at(-(-(s + 1) * W // nseg))
        assert (owner[t0:t1] == -1).all()
        owner[t0:t1] = s
    return nt, (P, TB), owner, nseg


def check(lengths, launched):
    nt, (P, TB), owner, nseg = split(lengths, launched)
    W = int(sum(TILE_W * n + START_W for n in nt if n))
    assert (owner >= 0).all(), "a tile belongs to no segment"
    assert set(owner.tolist()) == set(range(nseg)), "an empty segment"
    assert (np.diff(owner) >= 0).all(), "segments are not contiguous"
    for b, n in enumerate(nt):
        if not n:
            continue
        xs = P[b] + START_W + TILE_W * np.arange(n)
        assert ((xs * nseg) // W == owner[TB[b]:TB[b] + n]).all()
        s0, s1 = (xs[0] * nseg) // W, (xs[-1] * nseg) // W
        assert sorted(set(owner[TB[b]:TB[b] + n].tolist())) == list(range(s0, s1 + 1))
    return np.bincount(owner, minlength=nseg)


@pytest.mark.parametrize("seed", range(40))
def test_random_batches(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 90))
    lengths = rng.integers(0, 4000, size=B) * (rng.random(B) > 0.15)
    check(lengths, int(rng.integers(1, 300)))


def test_batch40_balance():
    rng = np.random.default_rng(2000)
    lengths = rng.integers(1024, 8192, size=40, endpoint=True)
    counts = check(lengths, 256)
    # 256 segments of ~5.2 tiles: none carries more than one tile above the mean
    assert counts.max() <= int(np.ceil(counts.mean())) + 1


def test_tiny_and_empty():
    check([1], 256)
    check([0, 0, 5, 0], 256)
    check([1] * 40, 256)
    assert split([0, 0], 256)[3] == 0


def test_double_division_is_exact_floor():
    """The kernels compute floor(a / b) (segment of a weighted position, and
    a segment's bounds) as floor of one correctly rounded double division,
    claimed exact for 0 <= a < 2^53, 0 < b < 2^31.  Python floats are IEEE
    doubles with correctly rounded division: check the claim on random and
    adversarial operands (a one below, at and one above a multiple of b)."""
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(20000):
        b = int(rng.integers(1, 2**31))
        k = int(rng.integers(0, (2**53 - 2) // b))
        for a in (k * b - 1, k * b, k * b + 1, int(rng.integers(0, 2**53))):
            if 0 <= a < 2**53:
                cases.append((a, b))
    cases += [(2**53 - 1, 1), (2**53 - 1, 2**31 - 1), (2**53 - 2, 3), (0, 5), (2**31 - 1, 2**31 - 1)]
    for a, b in cases:
        assert int(float(a) / float(b) // 1) == a // b, (a, b)
