"""Paired kernel-trace ledger: name rules that put every GPU kernel of a trace in
a category, per-category totals, the diff of two runs of the same workload, and
the balance of costs against savings.

This is the attribution method of "When a Faster Kernel Doesn't Speed Up
Serving" (ROCm blog): *Step 1* (paired trace diff: compare a run against a
baseline under the same workload, category by category, weighting each change
by its share of total GPU time), *Step 2* (semantic analysis: every grouping is
an explicit, repeatable rule on kernel names, with the FP8 <-> BF16 dtype casts
as categories of their own, CastFromFP8 for the read path and CastToFP8 for the
write path) and *The Ledger* (positive diffs are costs the change introduced,
negative diffs are savings; their sum is the net delta).

The rules below are written for the kernels of this library, of PyTorch-ROCm
and of the serving stacks the pages profile (the example names of the pages'
category table); anything they do not match is ``Others``.

    python -m fp8_paged_mla_amd.ledger RUN BASE [--labels FP8 BF16]

Each trace is a rocprofv3 ``*_kernel_trace.csv`` (one row per dispatch) or
``*_kernel_stats.csv`` (one row per kernel name), or a chrome-trace ``.json``
as the torch profiler exports it (events of category "kernel").
"""
import argparse
import csv
import re
import sys
from collections import OrderedDict

OTHERS = "Others"

# (category, pattern) -- the first pattern that matches the kernel name wins,
# so the dtype-cast and KV-write rules come before the generic copy and
# elementwise ones.
RULES = [
    # FP8 -> BF16 (read path): this library's cast kernels, and any kernel
    # launched by an aten::copy_ into a BF16 tensor from an FP8 one (torch's
    # copy kernel is named after its output dtype only, so the launching op and
    # its input types, which the torch profiler records, decide).
    ("CastFromFP8", r"cast_pool_kernel|gather_cast_kernel"
                    r"|<- aten::copy_\((c10::)?BFloat16, (c10::)?Float8_e4m3fn"),
    # BF16 -> FP8 (write path): torch's copy kernel into an FP8 tensor, or any
    # kernel of an aten::copy_ into an FP8 tensor from a BF16 one.
    ("CastToFP8", r"float8_copy_kernel"
                  r"|<- aten::copy_\((c10::)?Float8_e4m3fn, (c10::)?BFloat16"),
    # KV-cache writes that are not dtype casts: index writes into the cache,
    # the serving stacks' cache-store kernels, and this library's fused
    # quantise-and-scatter (it writes FP8 directly, so no cast kernel remains).
    ("KVCacheWrite", r"scatter_cast_kernel|index_put|set_kv_buffer|set_mla_kv"
                     r"|store_kvcache|reshape_and_cache|concat_and_cache"),
    ("MLA", r"\bmla_|::mla_|^mla_|_mla_"),
    ("MoEGEMM", r"moe_gemm|fused_moe|ck_moe|MoeGemm"),
    ("MoESorting", r"moe_sorting|moe_align|MoeSorting"),
    ("GEMM", r"^Cijk_|\bCijk_|wvSpltK|gemm|Gemm|GEMM"),
    ("Comm (NCCL)", r"nccl|rccl|cross_device_reduce|all_reduce|allreduce|AllReduce"),
    ("RMSNorm", r"[Rr]ms_?[Nn]orm"),
    ("Quant", r"(?<![a-z])quant|_quant|Quant"),
    ("TopK", r"topk|TopK|top_k"),
    ("ActMul", r"act_and_mul|silu_and_mul|gelu_and_mul|ActMul"),
    ("ReduceOP", r"reduce_kernel|ReduceOp|reduce_"),
    ("Elementwise", r"elementwise|copy_kernel|copyBuffer|fillBuffer|FillFunctor"),
]
_COMPILED = [(c, re.compile(p)) for c, p in RULES]


def categorize(name: str) -> str:
    """Category of one kernel name (first matching rule, else Others)."""
    for cat, pat in _COMPILED:
        if pat.search(name):
            return cat
    return OTHERS


class Totals:
    """Per-category dispatch count and GPU time (ms) of one run."""

    def __init__(self, rows=None):
        self.rows = OrderedDict()  # category -> [count, ms]
        for cat, count, ms in rows or []:
            self.add(cat, count, ms)

    def add(self, cat, count, ms):
        r = self.rows.setdefault(cat, [0, 0.0])
        r[0] += count
        r[1] += ms

    def total_ms(self) -> float:
        return sum(ms for _, ms in self.rows.values())

    def get(self, cat):
        return tuple(self.rows.get(cat, (0, 0.0)))


def totals_from_kernels(kernels) -> Totals:
    """kernels: iterable of (name, count, total_ms)."""
    t = Totals()
    for name, count, ms in kernels:
        t.add(categorize(name), count, ms)
    return t


def read_rocprof_csv(path):
    """(name, count, total_ms) per kernel name from a rocprofv3 kernel-trace or
    kernel-stats CSV."""
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    per = OrderedDict()
    if rows and "Kernel_Name" in rows[0]:
        for r in rows:
            ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            c = per.setdefault(r["Kernel_Name"], [0, 0.0])
            c[0] += 1
            c[1] += ns / 1e6
    elif rows and "Name" in rows[0]:
        for r in rows:
            c = per.setdefault(r["Name"], [0, 0.0])
            c[0] += int(r["Calls"])
            c[1] += float(r["TotalDurationNs"]) / 1e6
    else:
        raise ValueError("%s: not a rocprofv3 kernel trace or kernel stats CSV" % path)
    return [(n, c, ms) for n, (c, ms) in per.items()]


def read_chrome_trace(path):
    """(name, count, total_ms) per kernel from a chrome-trace JSON (the torch
    profiler's export): events of category "kernel", durations in microseconds.
    A kernel whose launching operator is in the trace (same "External id") is
    named ``"<kernel>  <- <op>(<input types>)"`` when the trace recorded input
    types (``record_shapes=True``), else ``"<kernel>  <- <op>"``."""
    import json
    with open(path) as f:
        data = json.load(f)
    events = data.get("traceEvents", data) if isinstance(data, dict) else data
    ops = {}
    for e in events:
        if isinstance(e, dict) and e.get("cat") == "cpu_op":
            a = e.get("args", {})
            if "External id" in a:
                types = a.get("Input type")
                ops[a["External id"]] = e["name"] + (
                    "(%s)" % ", ".join(str(t) for t in types) if types else "")
    per = OrderedDict()
    for e in events:
        if isinstance(e, dict) and str(e.get("cat", "")).lower() == "kernel" and "dur" in e:
            op = ops.get(e.get("args", {}).get("External id"))
            name = e["name"] + ("  <- " + op if op else "")
            c = per.setdefault(name, [0, 0.0])
            c[0] += 1
            c[1] += float(e["dur"]) / 1e3
    return [(n, c, ms) for n, (c, ms) in per.items()]


def read_kernel_events(path):
    """Kernels of a trace file: chrome-trace JSON, or a rocprofv3 CSV."""
    if path.endswith(".json"):
        return read_chrome_trace(path)
    return read_rocprof_csv(path)


def paired_diff(run: Totals, base: Totals):
    """Rows (category, run_count, run_ms, run_pct, base_count, base_ms, base_pct,
    diff_ms), largest run time first, over every category either run has."""
    tr, tb = run.total_ms(), base.total_ms()
    cats = list(OrderedDict.fromkeys(list(run.rows) + list(base.rows)))
    out = []
    for c in cats:
        rc, rm = run.get(c)
        bc, bm = base.get(c)
        out.append((c, rc, rm, 100.0 * rm / tr if tr else 0.0,
                    bc, bm, 100.0 * bm / tb if tb else 0.0, rm - bm))
    out.sort(key=lambda r: (-r[2], -r[5], r[0]))
    return out


def ledger(diffs, list_at_least=500.0, always_list=("MLA",)):
    """Balance of per-category diffs {category: diff_ms}.

    Returns (costs, savings, cost_total, saving_total, net): costs are the
    positive diffs, largest first; savings the negative ones, largest first,
    where savings smaller than ``list_at_least`` (and not in ``always_list``)
    are merged into one line ("n smaller categories")."""
    costs = sorted(((c, d) for c, d in diffs.items() if d > 0), key=lambda x: -x[1])
    neg = sorted(((c, d) for c, d in diffs.items() if d < 0), key=lambda x: x[1])
    listed = [(c, d) for c, d in neg if -d >= list_at_least or c in always_list]
    small = [(c, d) for c, d in neg if not (-d >= list_at_least or c in always_list)]
    savings = [x for x in listed if x[0] not in always_list]
    if small:
        savings.append(("%d smaller categories (%s)" % (len(small), ", ".join(c for c, _ in small)),
                        sum(d for _, d in small)))
    savings += [x for x in listed if x[0] in always_list]
    cost_total = sum(d for _, d in costs)
    saving_total = sum(d for _, d in neg)
    return costs, savings, cost_total, saving_total, cost_total + saving_total


def share_weighted_impact(local_speedup: float, share: float) -> float:
    """End-to-end fraction saved by a per-kernel speedup: the speedup (fraction of
    the kernel's time saved) times the kernel's share of total GPU time."""
    return local_speedup * share


def format_report(run: Totals, base: Totals, labels=("run", "base")) -> str:
    rows = paired_diff(run, base)
    a, b = labels
    lines = ["%-14s %10s %12s %8s %10s %12s %8s %12s" % (
        "Category", a + " n", a + " ms", a + " %", b + " n", b + " ms", b + " %",
        "Diff ms")]
    for c, rc, rm, rp, bc, bm, bp, d in rows:
        lines.append("%-14s %10d %12.3f %7.2f%% %10d %12.3f %7.2f%% %+12.3f"
                     % (c, rc, rm, rp, bc, bm, bp, d))
    tr, tb = run.total_ms(), base.total_ms()
    lines.append("%-14s %10s %12.3f %8s %10s %12.3f %8s %+12.3f"
                 % ("Total", "", tr, "100%", "", tb, "100%", tr - tb))
    # savings below 0.04% of the baseline's total are merged into one line; on
    # the pages' traces that is ~490 ms, which merges exactly their seven
    # smaller categories
    costs, savings, ct, st, net = ledger({r[0]: r[7] for r in rows}, list_at_least=4e-4 * tb)
    lines.append("")
    lines.append("Ledger (%s - %s, ms):" % (a, b))
    lines.append("  costs:")
    for c, d in costs:
        lines.append("    +%-40s %+12.3f" % (c, d))
    lines.append("    %-41s %+12.3f" % ("subtotal", ct))
    lines.append("  savings:")
    for c, d in savings:
        lines.append("    -%-40s %+12.3f" % (c, d))
    lines.append("    %-41s %+12.3f" % ("subtotal", st))
    lines.append("  net %+.3f ms (%+.2f%% of %s)" % (net, 100.0 * net / tb if tb else 0.0, b))
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("run")
    ap.add_argument("base")
    ap.add_argument("--labels", nargs=2, default=("run", "base"))
    args = ap.parse_args(argv)
    run = totals_from_kernels(read_kernel_events(args.run))
    base = totals_from_kernels(read_kernel_events(args.base))
    print(format_report(run, base, tuple(args.labels)))


if __name__ == "__main__":
    sys.exit(main())
