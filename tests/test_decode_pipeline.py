"""The explicit vmcnt waits of the 16-head FP8 decode kernel (mla_split_kernel),
on a Python model of one wave's issue order (no GPU).

A wave issues index loads, query copies, row copies (global -> LDS) and
stores, and waits with ``s_waitcnt vmcnt(N)``: "at most N
of this wave's memory operations outstanding".  Operations retire in issue
order, so such a wait proves complete every operation older than the N
youngest.  Each wait of the kernel is modelled with the count the kernel
passes, and the operations the code after it consumes are checked to be
among the proven ones, for every tile count up to 12, every pattern of
request ends and both wave classes (waves 0-1 own the query rows and copy
their next rows late after a query switch).  A last check ties the model to
the kernel source: the copy-op counts and the wait expressions it models.
"""
import itertools
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_paged_mla_amd", "csrc", "mla_decode.hip")

ROW_SLOTS = 37                                  # 36 data chunks + 1 pad per LDS row
DMA_OPS = (16 * ROW_SLOTS + 63) // 64           # 10 row-copy ops per wave per tile
QCOPY_OPS = 3
WAIT_UPTO_CASES = {1, 10, 11}               # immediates wait_vm_upto has; others wait for 0


class Wave:
    def __init__(self):
        self.ops = []

    def issue(self, kind, tile, n=1):
        self.ops += [(kind, tile)] * n

    def wait(self, n, needed, upto=False):
        if upto and n not in WAIT_UPTO_CASES:
            n = 0
        proven = len(self.ops) - n  # operations [0, proven) have retired
        for op in needed:
            last = len(self.ops) - 1 - self.ops[::-1].index(op)  # its last copy op
            assert last < proven, "waiting for %s with vmcnt(%d) after %s" % (op, n, self.ops)


def run_wave(T, ends, w):
    """One wave of a segment with T tiles; ends = tiles that end a request."""
    v = Wave()
    v.issue("idx", 0)
    v.issue("idx", 1)
    v.issue("q", 0, QCOPY_OPS)
    v.wait(QCOPY_OPS, [("idx", 0), ("idx", 1)])
    v.issue("rows", 0, DMA_OPS)
    v.issue("idx", 2)
    v.wait(1 + DMA_OPS, [("q", 0)])
    if T > 1:
        v.issue("rows", 1, DMA_OPS)
    v.wait(1 + DMA_OPS if T > 1 else 1, [("rows", 0)], upto=True)
    for k in range(T):
        # scores of tile k read rows(k): proven by the previous tile's last wait;
        # the rows of tile k+2 need its index
        v.wait(DMA_OPS if k + 1 < T else 0, [("idx", k + 2)] if k + 2 < T else [], upto=True)
        v.issue("idx", k + 3)
        new_q = k in ends and k + 1 < T
        if new_q:
            v.issue("q", k + 1, QCOPY_OPS)
        rows_now = k + 2 < T and (not new_q or w >= 2)
        if rows_now:
            v.issue("rows", k + 2, DMA_OPS)
        if k + 1 < T:
            n = (0 if new_q else 1) + (DMA_OPS if rows_now else 0)
            need = [("rows", k + 1)] + ([("q", k + 1)] if new_q else [])
            v.wait(n, need, upto=True)
        if new_q and w < 2 and k + 2 < T:
            v.issue("rows", k + 2, DMA_OPS)
        if k in ends or k + 1 == T:
            v.issue("store", k, 5)  # output or partial: 4 row stores (+ lse)
    v.wait(0, [op for op in v.ops])
    return v


def test_every_wait_proves_what_follows():
    for T in range(1, 13):
        for mask in range(1 << T):
            ends = {k for k in range(T) if mask >> k & 1}
            for w in (0, 5):
                run_wave(T, ends, w)


def test_rows_are_issued_after_their_index_and_before_use():
    for T, w in itertools.product(range(1, 9), (1, 3)):
        for mask in range(1 << T):
            v = run_wave(T, {k for k in range(T) if mask >> k & 1}, w)
            for t in range(T):
                assert v.ops.index(("idx", t)) < v.ops.index(("rows", t))


def test_source_matches_model():
    src = open(SRC).read()
    assert "constexpr int ROW_SLOTS = KV_CHUNKS + 1;" in src
    assert "constexpr int DMA_OPS = (16 * ROW_SLOTS + 63) / 64;" in src
    assert "constexpr int QCOPY_OPS = 3;" in src
    cases = {int(c) for c in re.findall(r"case (\d+): wait_vm<\1>\(\); break;", src)}
    assert cases == WAIT_UPTO_CASES
    body = src[src.index("void mla_split_kernel("):src.index("struct CombineParams")]
    for expr in ("wait_vm<QCOPY_OPS>();",
                 "wait_vm<1 + DMA_OPS>();",
                 "wait_vm_upto(ntiles > 1 ? 1 + DMA_OPS : 1);",
                 "wait_vm_upto(k + 1 < ntiles ? DMA_OPS : 0);",
                 "wait_vm_upto((new_q ? 0 : 1) + (rows_now ? DMA_OPS : 0));",
                 "const bool rows_now = k + 2 < ntiles && (!new_q || w >= 2);",
                 "if (w < 2 && k + 2 < ntiles) issue_tile(k + 2, ix_cur);"):
        assert expr in body, expr
