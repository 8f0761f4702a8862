"""The explicit vmcnt waits of the two cast kernels, on a Python model of
their issue order (no GPU).

Both kernels copy their input into per-wave LDS slots with global->LDS copies
and wait for a chunk with ``s_waitcnt vmcnt(N)``: "at most N memory operations
of this wave outstanding".  Operations complete in issue order, and stores
count too, so N must not exceed the number of operations issued after the
last one the chunk needs.  The kernels compute that number with closed forms;
here the same forms are checked against a literal list of the issued
operations, for every chunk of every per-wave chunk count up to 40, and the
immediate the kernel picks is checked to be at most the count.
"""
import pytest

# cast_pool_kernel: 2 slots, 2 copy ops (1 KB each) and 4 stores per 2 KB chunk
CAST_S, CAST_OPS = 2, 2
CAST_IMMEDIATES = [10, 8, 6, 4, 2, 1, 0]
# gather_cast_kernel: 3 slots, 9 row copies, 18 stores per 16-row chunk, one id copy per chunk
GATHER_S, GATHER_G, GATHER_R = 3, 9, 18
GATHER_IMMEDIATES = [48, 40, 32, 27, 24, 18, 12, 9, 4, 1, 0]


def cast_younger(k, K):
    """cast_wait_chunk's count (closed form as in cast.hip)."""
    S, OPS = CAST_S, CAST_OPS
    P0 = min(K, S)
    m = max(0, k - max(0, K - S))
    return OPS * (P0 - 1 - k) + 3 * OPS * k - OPS * m if k < S else 3 * OPS * (S - 1) + 2 * OPS - OPS * m


def cast_issue_order(K):
    """Operations in issue order: prologue copies of chunks 0..min(K,S)-1, then per
    iteration k the copies of chunk k + S (if any) and 2 * OPS stores."""
    S, OPS = CAST_S, CAST_OPS
    order = [("copy", d, o) for d in range(min(K, S)) for o in range(OPS)]
    waits = {}
    for k in range(K):
        waits[k] = len(order)  # operations issued when iteration k waits
        if k + S < K:
            order += [("copy", k + S, o) for o in range(OPS)]
        order += [("store", k, h) for h in range(2 * OPS)]
    return order, waits


def gather_younger(k, K):
    """gather_wait_chunk's count (closed forms as in cast.hip)."""
    S, G, R = GATHER_S, GATHER_G, GATHER_R
    A, P0 = min(K, S + 1), min(K, S)
    T0 = A + G * P0
    KS, KS1 = max(0, K - S), max(0, K - S - 1)

    def ops_before(i):
        return R * i + G * min(i, KS) + min(i, KS1)

    Tk = T0 + ops_before(k)
    if k < P0:
        last_row_copy = A + G * k + G - 1
    else:
        j = k - S
        last_row_copy = T0 + ops_before(j) + (1 if j + S + 1 < K else 0) + G - 1
    younger = Tk - last_row_copy - 1
    if k + S < K:
        id_copy = S if k == 0 else T0 + ops_before(k - 1)
        younger = min(younger, Tk - id_copy - 1)
    return younger


def gather_issue_order(K):
    """Prologue: id copies of chunks 0..A-1, a drain, row copies of chunks 0..P0-1;
    iteration k: [ids of chunk k + S + 1] [rows of chunk k + S] [R stores]."""
    S, G, R = GATHER_S, GATHER_G, GATHER_R
    A, P0 = min(K, S + 1), min(K, S)
    order = [("ids", c) for c in range(A)]
    order += [("rows", c, g) for c in range(P0) for g in range(G)]
    waits = {}
    for k in range(K):
        waits[k] = len(order)
        if k + S < K:
            if k + S + 1 < K:
                order.append(("ids", k + S + 1))
            order += [("rows", k + S, g) for g in range(G)]
        order += [("store", k, h) for h in range(R)]
    return order, waits


def _pick(immediates, younger):
    return next(n for n in immediates if n <= younger)


@pytest.mark.parametrize("K", range(0, 41))
def test_cast_wait_counts(K):
    order, waits = cast_issue_order(K)
    for k in range(K):
        needed = order.index(("copy", k, CAST_OPS - 1))
        exact = waits[k] - needed - 1
        assert cast_younger(k, K) == exact
        assert _pick(CAST_IMMEDIATES, exact) <= exact


@pytest.mark.parametrize("K", range(0, 41))
def test_gather_wait_counts(K):
    order, waits = gather_issue_order(K)
    for k in range(K):
        needed = [order.index(("rows", k, GATHER_G - 1))]
        if k + GATHER_S < K:  # the ids of the chunk whose rows this iteration copies
            needed.append(order.index(("ids", k + GATHER_S)))
        exact = waits[k] - max(needed) - 1
        assert gather_younger(k, K) == exact
        assert _pick(GATHER_IMMEDIATES, exact) <= exact


def test_gather_id_slots_outlive_their_reads():
    # ids of chunk c sit in id slot c % (S + 2); they are read when chunk c's rows
    # are copied (iteration c - S, or the prologue) and overwritten by the id copy
    # of chunk c + S + 2, issued in iteration c + 1: always later
    S = GATHER_S
    for c in range(60):
        read_at = c - S if c >= S else -1
        overwritten_at = (c + S + 2) - S - 1
        assert overwritten_at > read_at


def test_model_matches_the_kernel_source():
    # the constants and wait immediates above are those of cast.hip
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "fp8_paged_mla_amd", "csrc",
                            "cast.hip")).read()

    def const(name):
        return int(re.search(r"constexpr int %s = (\d+);" % name, src).group(1))

    assert const("CAST_SLOTS") == CAST_S
    assert const("CAST_CHUNK") // 1024 == CAST_OPS
    assert const("GATHER_SLOTS") == GATHER_S
    assert const("GATHER_ROWS") * 576 // 1024 == GATHER_G
    assert const("GATHER_ROWS") * 576 * 2 // 1024 == GATHER_R

    def immediates(fn):
        body = src.split("void %s(" % fn, 1)[1].split("\n}\n", 1)[0]
        return [int(x) for x in re.findall(r"wait_vm<(\d+)>", body)]

    assert immediates("cast_wait_chunk") == CAST_IMMEDIATES
    assert immediates("gather_wait_chunk") == GATHER_IMMEDIATES
