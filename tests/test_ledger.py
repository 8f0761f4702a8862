"""The paired-trace ledger (host code): category rules, per-category totals,
diff and balance, pinned to the category table and ledger the pages print
("When a Faster Kernel Doesn't Speed Up Serving", Step 1, Step 2, The Ledger)."""
import csv
import os

import pytest

from fp8_paged_mla_amd import ledger as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages_table():
    rows = []
    with open(os.path.join(GOLDEN, "pages_category_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, fc, fm, fp, bc, bm, bp, d = line.rstrip("\n").split("\t")
            rows.append((c, int(fc), float(fm), float(fp), int(bc), float(bm), float(bp), int(d)))
    return rows


def _runs():
    t = _pages_table()
    fp8 = L.Totals([(r[0], r[1], r[2]) for r in t])
    bf16 = L.Totals([(r[0], r[4], r[5]) for r in t])
    return t, fp8, bf16


def test_totals_and_shares_match_the_pages():
    t, fp8, bf16 = _runs()
    assert fp8.total_ms() == 1215200
    assert abs(bf16.total_ms() - 1214240) <= 1          # printed rows are rounded
    rows = {r[0]: r for r in L.paired_diff(fp8, bf16)}
    for c, fc, fm, fp, bc, bm, bp, d in t:
        got = rows[c]
        assert got[1] == fc and got[4] == bc
        assert round(got[3], 2) == fp, c
        assert round(got[6], 2) == bp, c


def test_diffs_match_the_pages_within_rounding():
    t, fp8, bf16 = _runs()
    rows = {r[0]: r for r in L.paired_diff(fp8, bf16)}
    exact = 0
    for c, *_, printed in t:
        assert abs(rows[c][7] - printed) <= 1, c
        exact += rows[c][7] == printed
    assert exact == 13                                  # KVCacheWrite and MLA round differently
    order = [r[0] for r in L.paired_diff(fp8, bf16)]
    assert order == [r[0] for r in t]                   # the page sorts by FP8 time


def test_ledger_reproduces_the_pages_balance():
    t, _, _ = _runs()
    costs, savings, ct, st, net = L.ledger({r[0]: r[7] for r in t})
    assert costs == [("CastFromFP8", 6392), ("CastToFP8", 2202)]
    assert ct == 8594 and st == -7633 and net == 961
    names = [c for c, _ in savings]
    assert names[:5] == ["Others", "GEMM", "Comm (NCCL)", "Elementwise", "MoEGEMM"]
    assert names[5].startswith("7 smaller categories")
    assert set(names[5].split("(")[1].rstrip(")").split(", ")) == {
        "RMSNorm", "MoESorting", "KVCacheWrite", "ReduceOP", "TopK", "ActMul", "Quant"}
    assert savings[5][1] == -568
    assert savings[6] == ("MLA", -94)
    assert round(100 * net / 1214240, 2) == 0.08


def test_share_weighted_impact_of_the_mla_speedup():
    speedup = 1 - 0.125 / 0.190
    assert round(100 * speedup) == 34
    assert round(100 * 190 / 1215200, 4) == 0.0156
    assert round(100 * 94 / 1214240, 4) == 0.0077
    assert round(100 * L.share_weighted_impact(0.34, 0.0002), 3) == 0.007


@pytest.mark.parametrize("name,cat", [
    # example kernels of the pages' category table
    ("moe_gemm1_0", "MoEGEMM"), ("moe_gemm2_0", "MoEGEMM"),
    ("aiter::mla_a8w8_qh16_qseqlen1_gqaratio16", "MLA"),
    ("mla_dec_stage1_bf16_a16w16_subQ16_mqa16", "MLA"),
    ("Cijk_Alik_Bljk_BBS_BH_MT128x128x64", "GEMM"), ("wvSpltK_hf_", "GEMM"),
    ("bf16gemm_fp32bf16_tn_96x64", "GEMM"),
    ("cross_device_reduce_2stage<__hip_bfloat16, 8>", "Comm (NCCL)"),
    ("ncclDevKernel_Generic", "Comm (NCCL)"),
    ("Rmsnorm2dFwd<...>", "RMSNorm"),
    # this library's kernels
    ("void fp8mla::(anonymous namespace)::cast_pool_kernel(...)", "CastFromFP8"),
    ("void fp8mla::(anonymous namespace)::gather_cast_kernel(...)", "CastFromFP8"),
    ("void fp8mla::(anonymous namespace)::scatter_cast_kernel<false>(...)", "KVCacheWrite"),
    ("void fp8mla::(anonymous namespace)::mla_split_kernel(fp8mla::decode::SplitParams)", "MLA"),
    ("void fp8mla::(anonymous namespace)::mla_combine_kernel(...)", "MLA"),
    ("void fp8mla::(anonymous namespace)::mla_split_bf16_kernel(...)", "MLA"),
    # PyTorch-ROCm kernels seen in this library's traces
    ("void at::native::vectorized_elementwise_kernel<8, at::native::float8_copy_kernel_cuda"
     "(at::TensorIteratorBase&)::{lambda(c10::BFloat16)#1}, std::array<char*, 2ul> >(...)",
     "CastToFP8"),
    ("void at::native::index_elementwise_kernel<128, 4, at::native::gpu_index_kernel<at::native::"
     "index_put_kernel_impl<at::native::OpaqueType<1> >(...)", "KVCacheWrite"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda"
     "(at::TensorIteratorBase&)::{lambda(float)#1}, std::array<char*, 2ul> >(...)", "Elementwise"),
    ("__amd_rocclr_copyBuffer", "Elementwise"),
    ("some_unknown_kernel", "Others"),
])
def test_rules(name, cat):
    assert L.categorize(name) == cat


def test_rules_are_deterministic_and_cover_every_kernel():
    names = ["mla_x", "Cijk_y", "foo", "float8_copy_kernel", "index_put"]
    assert [L.categorize(n) for n in names] == [L.categorize(n) for n in names]
    t = L.totals_from_kernels([(n, 2, 1.5) for n in names])
    assert sum(c for c, _ in t.rows.values()) == 10 and t.total_ms() == 7.5


def test_reads_both_rocprof_csv_forms(tmp_path):
    trace = tmp_path / "kt_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerow(["KERNEL_DISPATCH", "mla_split_kernel", 1000, 31000])
        w.writerow(["KERNEL_DISPATCH", "mla_split_kernel", 50000, 80000])
        w.writerow(["KERNEL_DISPATCH", "cast_pool_kernel", 0, 172000])
    stats = tmp_path / "kt_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs"])
        w.writerow(["mla_split_kernel", 2, 60000, 30000])
        w.writerow(["cast_pool_kernel", 1, 172000, 172000])
    a = L.totals_from_kernels(L.read_rocprof_csv(str(trace)))
    b = L.totals_from_kernels(L.read_rocprof_csv(str(stats)))
    assert a.rows == b.rows == {"MLA": [2, 0.06], "CastFromFP8": [1, 0.172]}
    text = L.format_report(a, L.Totals([("MLA", 2, 0.1)]), ("fp8", "bf16"))
    assert "CastFromFP8" in text and "net" in text


def test_cli(tmp_path, capsys):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs"])
        w.writerow(["mla_split_kernel", 3, 90000])
    L.main([str(p), str(p), "--labels", "A", "B"])
    out = capsys.readouterr().out
    assert "net +0.000 ms" in out


def test_chrome_trace_op_types_decide_the_copy_direction(tmp_path):
    """torch names its FP8 -> BF16 copy kernel after the BF16 output only; the
    launching aten::copy_ and its input types (dst, src) decide the category."""
    import json
    copy_kernel = ("void at::native::elementwise_kernel_manual_unroll<128, 4, at::native::"
                   "gpu_kernel_impl<at::native::direct_copy_kernel_cuda(at::TensorIteratorBase&)"
                   "::{lambda()#3}::operator()() const::{lambda()#12}::operator()() const::"
                   "{lambda(c10::BFloat16)#1}>(...)")
    p = tmp_path / "t.json"
    json.dump({"traceEvents": [
        {"ph": "X", "cat": "cpu_op", "name": "aten::copy_",
         "args": {"External id": 4, "Input type": ["c10::BFloat16", "c10::Float8_e4m3fn", "Scalar"]}},
        {"ph": "X", "cat": "cpu_op", "name": "aten::copy_",
         "args": {"External id": 9, "Input type": ["c10::BFloat16", "c10::BFloat16", "Scalar"]}},
        {"ph": "X", "cat": "kernel", "name": copy_kernel, "dur": 687.0, "args": {"External id": 4}},
        {"ph": "X", "cat": "kernel", "name": copy_kernel, "dur": 10.0, "args": {"External id": 9}},
        {"ph": "X", "cat": "kernel", "name": copy_kernel, "dur": 1.0, "args": {"External id": 77}},
    ]}, open(p, "w"))
    t = L.totals_from_kernels(L.read_kernel_events(str(p)))
    assert t.rows == {"CastFromFP8": [1, 0.687], "Elementwise": [2, 0.011]}


def test_reads_chrome_trace(tmp_path):
    import json
    p = tmp_path / "t.json"
    json.dump({"traceEvents": [
        {"ph": "X", "cat": "kernel", "name": "mla_split_kernel", "dur": 30.0},
        {"ph": "X", "cat": "kernel", "name": "mla_split_kernel", "dur": 31.0},
        {"ph": "X", "cat": "cpu_op", "name": "aten::copy_", "dur": 99.0},
        {"ph": "X", "cat": "kernel", "name": "float8_copy_kernel_cuda", "dur": 5.0},
    ]}, open(p, "w"))
    t = L.totals_from_kernels(L.read_kernel_events(str(p)))
    assert t.rows == {"MLA": [2, 0.061], "CastToFP8": [1, 0.005]}


def test_report_merges_the_same_small_savings_as_the_pages():
    _, fp8, bf16 = _runs()
    text = L.format_report(fp8, bf16, ("FP8", "BF16"))
    assert "7 smaller categories" in text
    assert "+CastFromFP8" in text and "+CastToFP8" in text
    assert "net +959.000 ms (+0.08% of BF16)" in text   # from the rounded printed rows
