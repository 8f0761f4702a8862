"""The load schedule of the role-specialised 64-head FP8 decode kernel
(mla_split_h64_kernel), on a Python model of its waves (no GPU).

The kernel's time is cut into half-tile intervals, each ended by one
workgroup barrier.  Score waves compute the scores of half-tile h in interval
h, value waves the P.V of half-tile h - 1.  The value waves also copy the
rows of each tile (global -> LDS, an eighth each) into slot tile % 3 and the
slot ids of each tile into their own LDS ring entry tile % 4; score waves
only load a query per request.  A wave waits with "at most N of my loads
outstanding"; loads retire in issue order, so such a wait proves every load
older than the N youngest.

For every tile count up to 10 and every pattern of request ends, the model
replays both roles' issue order and waits and checks:
  * the rows of a tile are proven by the copying waves before the barrier
    that precedes the first interval (of either role) reading them;
  * a slot is refilled only after the barrier that ends the last interval
    reading its previous tile, and a ring entry only after the row copies that
    read its previous ids were issued;
  * a tile's ids are proven before its row copies are addressed, a query
    before the scores that use it;
  * every wait count is one of the immediates the kernel's wait helper has
    (otherwise it would round down and wait longer than needed).
A last check ties the model to the kernel source.
"""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_paged_mla_amd", "csrc", "mla_decode_h64.hip")

DMA_OPS = 5        # row-copy ops per value wave per tile (8 rows x 37 chunks of 16 B)
QSTEPS = 18        # query loads per request (score waves)
NSLOTS = 3
ID_SLOTS = 4


def wait_immediates():
    src = open(SRC).read()
    return {int(n) for n in re.findall(r"wait_vm<(\d+)>\(\);", src)}


class Wave:
    """One wave's loads: a list of (kind, tile) per issued op."""

    def __init__(self, immediates):
        self.ops = []
        self.proven = 0          # ops [0, proven) have retired
        self.imm = immediates
        self.counts = []

    def issue(self, kind, tile, n=1):
        self.ops += [(kind, tile)] * n
        return len(self.ops) - 1

    def wait_done(self, op):
        """The kernel's wait_done(op): at most len - 1 - op outstanding."""
        n = len(self.ops) - 1 - op
        self.counts.append(n)
        usable = max(i for i in self.imm if i <= n)
        self.proven = max(self.proven, len(self.ops) - usable)

    def done(self, kind, tile):
        idx = [i for i, o in enumerate(self.ops) if o == (kind, tile)]
        return bool(idx) and idx[-1] < self.proven


def simulate(T, ends, imm):
    """Both roles over a segment of T tiles; ends = tiles that end a request.
    Returns {role: (wave, events)}, an event being (interval, kind, tile)
    with interval -1 for the prologue."""
    roles = {}
    # score wave: its query, then one more per request that starts in the segment
    v = Wave(imm)
    events = []
    q_pending = (v.issue("q", 0, QSTEPS), 0)
    v.wait_done(q_pending[0])
    assert v.done("q", 0)
    q_pending = None
    for h in range(2 * T + 1):
        m = h >> 1
        if h < 2 * T:
            if q_pending is not None:
                v.wait_done(q_pending[0])
                assert v.done("q", q_pending[1])
                q_pending = None
            events.append((h, "read", m))
            if h & 1 and m in ends and m + 1 < T:
                q_pending = (v.issue("q", m + 1, QSTEPS), m + 1)
    roles["score"] = (v, events)
    # value wave: the copies
    v = Wave(imm)
    events = []
    for j in range(4):
        v.issue("ids", j)
    v.wait_done(len(v.ops) - 3)  # ids of tile 1 (those of tiles 2, 3 younger)
    assert all(v.done("ids", j) for j in range(2))
    for j in range(2):
        if j < T:
            events.append((-1, "ring_read", j))
            v.issue("rows", j, DMA_OPS)
            events.append((-1, "copy", j))
    v.wait_done([i for i, o in enumerate(v.ops) if o == ("rows", 0)][-1])
    events.append((-1, "proven", [j for j in range(T) if v.done("rows", j)]))
    for h in range(2 * T + 1):
        m = h >> 1
        if h & 1:  # start of an odd interval: the copies
            if m + 2 < T:
                v.wait_done([i for i, o in enumerate(v.ops) if o == ("ids", m + 2)][-1])
                assert v.done("ids", m + 2)
                events.append((h, "ring_read", m + 2))
                v.issue("rows", m + 2, DMA_OPS)
                events.append((h, "copy", m + 2))
            events.append((h, "ring_write", m + 4))
            v.issue("ids", m + 4)
        if h >= 1:
            events.append((h, "read", (h - 1) >> 1))
        if h & 1:  # end of an odd interval: the wait
            if m + 1 < T:
                v.wait_done([i for i, o in enumerate(v.ops) if o == ("rows", m + 1)][-1])
            events.append((h, "proven", [j for j in range(T) if v.done("rows", j)]))
    roles["value"] = (v, events)
    return roles


def check(T, ends, imm):
    roles = simulate(T, ends, imm)
    # proven-before-barrier: tile m is read in interval h only if the copying
    # waves had proven its rows before the barrier ending interval h - 1 (or
    # the prologue's, h - 1 == -1)
    acc, proven_by = set(), {}  # barrier index -> tiles proven by then
    for h, ev, x in roles["value"][1]:
        if ev == "proven":
            acc |= set(x)
            proven_by[h] = set(acc)
    last_read = {}
    for role, (_, events) in roles.items():
        for h, ev, x in events:
            if ev != "read":
                continue
            last_read[x] = max(last_read.get(x, -2), h)
            before = [b for b in proven_by if b <= h - 1]
            assert before and x in proven_by[max(before)], \
                "T=%d ends=%s: %s reads tile %d in interval %d before it was proven" % (
                    T, sorted(ends), role, x, h)
    # slot refill after the last read of its previous tile (strictly earlier
    # interval: a barrier separates them); ring entry after its previous ids
    # were read to address row copies
    for role, (_, events) in roles.items():
        for i, (h, ev, x) in enumerate(events):
            if ev == "copy" and x >= NSLOTS:
                prev = x - NSLOTS
                assert last_read.get(prev, -2) < h, (T, sorted(ends), "slot", x, h)
            if ev == "ring_write" and x >= ID_SLOTS:
                prev = x - ID_SLOTS
                if prev < T:
                    reads = [k for k, (_, e2, y) in enumerate(events) if e2 == "ring_read" and y == prev]
                    assert reads and reads[0] < i, (T, sorted(ends), "ring", x)
    return roles


def test_schedule_every_tile_count_and_request_pattern():
    imm = wait_immediates()
    for T in range(1, 11):
        for mask in range(1 << T):
            ends = {k for k in range(T) if mask >> k & 1}
            check(T, ends, imm)


def test_wait_counts_are_exact_immediates():
    """No wait of the schedule rounds down to a stricter immediate."""
    imm = wait_immediates()
    seen = set()
    for T in range(1, 11):
        for mask in range(1 << T):
            ends = {k for k in range(T) if mask >> k & 1}
            for v, _ in check(T, ends, imm).values():
                seen |= set(v.counts)
    missing = sorted(n for n in seen if n not in imm and n < 63)
    assert not missing, missing


def test_source_matches_model():
    src = open(SRC).read()
    assert "constexpr int NSLOTS = 3;" in src
    assert "constexpr int ID_SLOTS = 4;" in src
    assert "constexpr int DMA_OPS = (ROWS_PER_COPIER * ROW_SLOTS + 63) / 64;  // 5" in src
    assert "constexpr int ROWS_PER_COPIER = TILE / COPIERS;   // 8" in src
    assert "constexpr int COPIERS = 8;" in src
    assert "constexpr int QSTEPS = 2 * KSTEPS;                // 18" in src
    for expr in ("if (m + 2 < ntiles) {\n        wait_done(id_a);  // ids of tile m + 2\n        r_new = copy_rows(m + 2);",
                 "id_new = copy_ids(m + 4);\n    };",
                 "if (h & 1) issue_copies(h >> 1);\n      if (h >= 1) {",
                 "if (h & 1) wait_copies();\n      __syncthreads();",
                 "int q_op = count_ops(QSTEPS);\n    wait_done(q_op);",
                 "if (last_of_request && m + 1 < ntiles) {"):
        assert expr in src, expr
