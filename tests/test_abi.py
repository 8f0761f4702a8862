"""The C ABI loads, exports every symbol the header declares, and rejects bad
arguments on the host before touching any device (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mla.h")
PROBE_HEADER = os.path.join(ROOT, "include", "fp8mla_probe.h")

fm = pytest.importorskip("fp8_paged_mla_amd")


def _lib():
    path = os.environ.get("FP8MLA_TEST_LIB")
    if path:  # another build of the same ABI (the sanitized one: test_abi_sanitized.py)
        return fm._bind(ctypes.CDLL(path))
    try:
        return fm.library()
    except RuntimeError as e:  # not built
        pytest.fail(str(e))


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)


def _status(name):
    text = open(HEADER).read()
    return int(re.search(r"#define %s \((-?\d+)\)|#define %s (-?\d+)" % (name, name), text)
               .group(1) or 0)


def test_header_declares_the_three_calls():
    names = set(_declared_functions())
    assert {"mla_decode_fp8", "gather_cast_fp8_bf16", "cast_pool_fp8_bf16"} <= names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = _lib()
    assert lib.fp8mla_abi_version() == 1
    for code in range(0, -7, -1):
        s = fm.status_string(code)
        assert s and s != "unknown status"
    assert fm.status_string(12345) == "unknown status"


P16 = 4096           # fake, 16-byte aligned, never dereferenced
P8 = 4096 + 8        # fake, misaligned
NULL = None

ERR_NULL = -1
ERR_SHAPE = -2
ERR_ALIGN = -3
ERR_SCALAR = -5


def test_header_status_values():
    assert _status("FP8MLA_ERR_NULL_PTR") == ERR_NULL
    assert _status("FP8MLA_ERR_BAD_SHAPE") == ERR_SHAPE
    assert _status("FP8MLA_ERR_MISALIGNED") == ERR_ALIGN
    assert _status("FP8MLA_ERR_BAD_SCALAR") == ERR_SCALAR


def test_cast_pool_validation():
    lib = _lib()
    assert lib.cast_pool_fp8_bf16(P16, -1, P16, NULL) == ERR_SHAPE
    assert lib.cast_pool_fp8_bf16(P16, 1 << 33, P16, NULL) == ERR_SHAPE
    assert lib.cast_pool_fp8_bf16(P16, 0, P16, NULL) == 0          # empty pool: no-op
    assert lib.cast_pool_fp8_bf16(NULL, 4, P16, NULL) == ERR_NULL
    assert lib.cast_pool_fp8_bf16(P16, 4, NULL, NULL) == ERR_NULL
    assert lib.cast_pool_fp8_bf16(P8, 4, P16, NULL) == ERR_ALIGN
    assert lib.cast_pool_fp8_bf16(P16, 4, P8, NULL) == ERR_ALIGN


def test_gather_cast_validation():
    lib = _lib()
    assert lib.gather_cast_fp8_bf16(P16, 10, P16, -1, P16, NULL) == ERR_SHAPE
    assert lib.gather_cast_fp8_bf16(P16, 10, P16, 0, P16, NULL) == 0   # n = 0: no-op
    assert lib.gather_cast_fp8_bf16(P16, 0, P16, 3, P16, NULL) == ERR_SHAPE
    assert lib.gather_cast_fp8_bf16(NULL, 10, P16, 3, P16, NULL) == ERR_NULL
    assert lib.gather_cast_fp8_bf16(P16, 10, NULL, 3, P16, NULL) == ERR_NULL
    assert lib.gather_cast_fp8_bf16(P16, 10, P16, 3, NULL, NULL) == ERR_NULL
    assert lib.gather_cast_fp8_bf16(P16, 10, P16 + 2, 3, P16, NULL) == ERR_ALIGN
    assert lib.gather_cast_fp8_bf16(P16, 10, P16, 3, P8, NULL) == ERR_ALIGN


def test_scatter_cast_validation():
    lib = _lib()

    def sc(**kw):
        a = dict(src=P16, n=3, stride=576, slots=P16, pool=P16, num_slots=10, inv=1.0, sat=0,
                 stream=NULL)
        a.update(kw)
        return lib.scatter_cast_bf16_fp8(a["src"], a["n"], a["stride"], a["slots"], a["pool"],
                                         a["num_slots"], a["inv"], a["sat"], a["stream"])

    assert sc(n=-1) == ERR_SHAPE
    assert sc(n=1 << 31) == ERR_SHAPE
    assert sc(num_slots=-1) == ERR_SHAPE
    assert sc(num_slots=0) == ERR_SHAPE
    assert sc(stride=575) == ERR_SHAPE
    assert sc(stride=580) == ERR_SHAPE            # not a multiple of 8 elements
    assert sc(inv=0.0) == ERR_SCALAR
    assert sc(inv=-2.0) == ERR_SCALAR
    assert sc(inv=math.inf) == ERR_SCALAR
    assert sc(inv=math.nan) == ERR_SCALAR
    assert sc(n=0) == 0                           # no-op, nothing launched
    assert sc(n=0, src=NULL, slots=NULL, pool=NULL, num_slots=0) == 0
    assert sc(src=NULL) == ERR_NULL
    assert sc(slots=NULL) == ERR_NULL
    assert sc(pool=NULL) == ERR_NULL
    assert sc(src=P8) == ERR_ALIGN
    assert sc(pool=P8) == ERR_ALIGN
    assert sc(slots=P16 + 2) == ERR_ALIGN


def _decode(lib, **kw):
    a = dict(q=P16, pool=P16, slots=100, indptr=P16, indices=P16, total=10, B=2, H=16,
             scale=1.0, sm=0.07, out=P16, ws=P16, ws_bytes=1 << 20, stream=NULL)
    a.update(kw)
    return lib.mla_decode_fp8(a["q"], a["pool"], a["slots"], a["indptr"], a["indices"],
                              a["total"], a["B"], a["H"], a["scale"], a["sm"], a["out"],
                              a["ws"], a["ws_bytes"], a["stream"])


def test_mla_decode_validation():
    lib = _lib()
    assert _decode(lib, B=0) == ERR_SHAPE
    assert _decode(lib, B=(1 << 24) + 1) == ERR_SHAPE  # FP8MLA_MAX_BATCH: the split's weights stay in int
    assert _decode(lib, H=0) == ERR_SHAPE
    assert _decode(lib, H=257) == ERR_SHAPE
    assert _decode(lib, total=-1) == ERR_SHAPE
    assert _decode(lib, total=1 << 31) == ERR_SHAPE
    assert _decode(lib, slots=0) == ERR_SHAPE
    assert _decode(lib, slots=-5) == ERR_SHAPE
    assert _decode(lib, scale=0.0) == ERR_SCALAR
    assert _decode(lib, scale=-1.0) == ERR_SCALAR
    assert _decode(lib, scale=math.nan) == ERR_SCALAR
    assert _decode(lib, sm=math.inf) == ERR_SCALAR
    assert _decode(lib, q=NULL) == ERR_NULL
    assert _decode(lib, out=NULL) == ERR_NULL
    assert _decode(lib, indptr=NULL) == ERR_NULL
    assert _decode(lib, pool=NULL) == ERR_NULL
    assert _decode(lib, indices=NULL) == ERR_NULL
    assert _decode(lib, ws=NULL) == ERR_NULL
    assert _decode(lib, q=P8) == ERR_ALIGN
    assert _decode(lib, out=P8) == ERR_ALIGN
    assert _decode(lib, pool=P8) == ERR_ALIGN
    assert _decode(lib, ws=P8) == ERR_ALIGN
    assert _decode(lib, indptr=P16 + 2) == ERR_ALIGN


def test_mla_decode_segments_validation():
    """The bounded-split call shares mla_decode_fp8's checks and rejects a
    segment bound below 1 before any device call."""
    lib = _lib()

    def call(S, **kw):
        a = dict(q=P16, pool=P16, slots=100, indptr=P16, indices=P16, total=10, B=2, H=16,
                 scale=1.0, sm=0.07, out=P16, ws=P16, ws_bytes=1 << 20, stream=NULL)
        a.update(kw)
        return lib.mla_decode_fp8_segments(a["q"], a["pool"], a["slots"], a["indptr"],
                                           a["indices"], a["total"], a["B"], a["H"], a["scale"],
                                           a["sm"], a["out"], a["ws"], a["ws_bytes"], S,
                                           a["stream"])

    assert call(0) == ERR_SHAPE
    assert call(-3) == ERR_SHAPE
    assert call(7, B=0) == ERR_SHAPE
    assert call(7, scale=0.0) == ERR_SCALAR
    assert call(7, q=NULL) == ERR_NULL
    assert call(7, ws=NULL) == ERR_NULL
    assert call(7, out=P8) == ERR_ALIGN


def test_mla_decode_bf16_validation():
    lib = _lib()
    lib.mla_decode_bf16.argtypes = lib.mla_decode_fp8.argtypes
    lib.mla_decode_bf16.restype = ctypes.c_int

    def dec(**kw):
        a = dict(q=P16, kv=P16, rows=100, indptr=P16, indices=P16, total=10, B=2, H=16,
                 scale=1.0, sm=0.07, out=P16, ws=P16, ws_bytes=1 << 20, stream=NULL)
        a.update(kw)
        return lib.mla_decode_bf16(a["q"], a["kv"], a["rows"], a["indptr"], a["indices"],
                                   a["total"], a["B"], a["H"], a["scale"], a["sm"], a["out"],
                                   a["ws"], a["ws_bytes"], a["stream"])

    assert dec(B=0) == ERR_SHAPE
    assert dec(B=(1 << 24) + 1) == ERR_SHAPE
    assert dec(H=257) == ERR_SHAPE
    assert dec(rows=0) == ERR_SHAPE
    assert dec(total=-1) == ERR_SHAPE
    assert dec(scale=0.0) == ERR_SCALAR
    assert dec(sm=math.nan) == ERR_SCALAR
    assert dec(kv=NULL) == ERR_NULL
    assert dec(ws=NULL) == ERR_NULL
    assert dec(kv=P8) == ERR_ALIGN
    assert dec(out=P8) == ERR_ALIGN


def test_workspace_query_rejects_bad_sizes():
    lib = _lib()
    assert lib.mla_decode_fp8_workspace_bytes(0, 16, 10) == 0
    assert lib.mla_decode_fp8_workspace_bytes((1 << 24) + 1, 16, 10) == 0
    assert lib.mla_decode_fp8_workspace_bytes(1, 0, 10) == 0
    assert lib.mla_decode_fp8_workspace_bytes(1, 300, 10) == 0
    assert lib.mla_decode_fp8_workspace_bytes(1, 16, -1) == 0
    assert lib.mla_decode_fp8_workspace_bytes(4, 16, 0) == 0       # nothing to split


def test_binding_rejects_cpu_tensors():
    import torch
    pool = torch.zeros((4, 576), dtype=torch.uint8)
    with pytest.raises(ValueError):
        fm.cast_pool_fp8_bf16(pool)
    with pytest.raises(ValueError):
        fm.scatter_cast_bf16_fp8(torch.zeros((2, 576), dtype=torch.bfloat16),
                                 torch.zeros(2, dtype=torch.int32), pool)


def test_mla_extend_validation():
    lib = _lib()

    def ext(**kw):
        a = dict(q=P16, pool=P16, slots=100, qo=P16, kv=P16, idx=P16, tq=10, tkv=40, B=2, H=16,
                 scale=1.0, sm=0.07, causal=1, out=P16, ws=P16, ws_bytes=1 << 30, stream=NULL)
        a.update(kw)
        return lib.mla_extend_fp8(a["q"], a["pool"], a["slots"], a["qo"], a["kv"], a["idx"],
                                  a["tq"], a["tkv"], a["B"], a["H"], a["scale"], a["sm"],
                                  a["causal"], a["out"], a["ws"], a["ws_bytes"], a["stream"])

    assert ext(B=0) == ERR_SHAPE
    assert ext(H=0) == ERR_SHAPE
    assert ext(H=257) == ERR_SHAPE
    assert ext(tq=-1) == ERR_SHAPE
    assert ext(tq=1 << 23) == ERR_SHAPE                # query rows pack into 23 bits
    assert ext(tkv=-1) == ERR_SHAPE
    assert ext(tq=(1 << 23) - 1, H=257) == ERR_SHAPE
    assert ext(tkv=1 << 31) == ERR_SHAPE
    assert ext(slots=0) == ERR_SHAPE
    assert ext(scale=0.0) == ERR_SCALAR
    assert ext(sm=math.nan) == ERR_SCALAR
    assert ext(tq=0) == 0                              # no query rows: no-op
    assert ext(q=NULL) == ERR_NULL
    assert ext(qo=NULL) == ERR_NULL
    assert ext(kv=NULL) == ERR_NULL
    assert ext(out=NULL) == ERR_NULL
    assert ext(ws=NULL) == ERR_NULL
    assert ext(pool=NULL) == ERR_NULL
    assert ext(idx=NULL) == ERR_NULL
    assert ext(q=P8) == ERR_ALIGN
    assert ext(out=P8) == ERR_ALIGN
    assert ext(qo=P16 + 2) == ERR_ALIGN
    assert ext(ws=P8) == ERR_ALIGN
    assert lib.mla_extend_fp8_workspace_bytes(0, 16, 10) == 0
    assert lib.mla_extend_fp8_workspace_bytes(1, 16, 0) == 0
    assert lib.mla_extend_fp8_workspace_bytes(1, 300, 10) == 0


def test_mla_extend_size_bound():
    """Calls whose tile bound, (NB + 1) * ceil(total_kv / 64) + batch + NB with
    NB = ceil(total_q / T), exceeds 2^28 are rejected on the host with
    BAD_SHAPE (never accepted and left unwritten); calls inside the bound get
    past every size check (here they fail later, for want of a device)."""
    lib = _lib()

    def ext(tq, tkv, B, H):
        return lib.mla_extend_fp8(P16, P16, 1 << 22, P16, P16, P16, tq, tkv, B, H, 1.0, 0.07, 1,
                                  P16, P16, 1 << 40, NULL)

    def bound(tq, tkv, B, H):
        rows = -(-H // 16) * 16
        T = 64 // rows if rows <= 64 else 1
        nb = -(-tq // T)
        return (nb + 1) * -(-tkv // 64) + B + nb

    cases = [
        (32768, 32768, 1, 128, True),        # 32k causal prefill, 128 heads
        (65536, 65536, 1, 64, True),         # 64k prefill, 64 heads
        (131072, 131072, 1, 128, False),     # 128k prefill at T = 1: bound just past 2^28
        (131072, 131072, 1, 16, True),       # the same at 16 heads (T = 4)
        (1024, 256 * 32768, 256, 16, True),  # 4 speculative tokens x 256 requests of 32k
        (1 << 22, 1 << 24, 1, 64, False),
        (1, 1, 1 << 25, 16, False),          # more virtual requests than 2^25
    ]
    for tq, tkv, B, H, ok in cases:
        assert (bound(tq, tkv, B, H) <= 1 << 28) == ok or B >= 1 << 25, (tq, tkv, B, H)
        st = ext(tq, tkv, B, H)
        if ok:
            assert st != ERR_SHAPE, (tq, tkv, B, H, st)
        else:
            assert st == ERR_SHAPE, (tq, tkv, B, H, st)


def test_mla_decode_noalloc_validation():
    """The allocation-free decode takes the same checks as mla_decode_fp8 (no
    workspace argument) and rejects batches past its scratch's limit, all on
    the host before any device call."""
    lib = _lib()
    text = open(HEADER).read()
    max_batch = int(re.search(r"#define FP8MLA_NOALLOC_MAX_BATCH (\d+)", text).group(1))
    scratch = re.search(r"#define FP8MLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert int(scratch.group(1)) << int(scratch.group(2)) <= 64 << 20  # a modest, stated size

    def dec(**kw):
        a = dict(q=P16, pool=P16, slots=100, indptr=P16, idx=P16, total=10, B=2, H=16, scale=1.0,
                 sm=0.07, out=P16, stream=NULL)
        a.update(kw)
        return lib.mla_decode_fp8_noalloc(a["q"], a["pool"], a["slots"], a["indptr"], a["idx"],
                                          a["total"], a["B"], a["H"], a["scale"], a["sm"],
                                          a["out"], a["stream"])

    assert dec(B=0) == ERR_SHAPE
    assert dec(B=max_batch + 1) == ERR_SHAPE
    assert dec(H=0) == ERR_SHAPE
    assert dec(H=257) == ERR_SHAPE
    assert dec(total=-1) == ERR_SHAPE
    assert dec(slots=0) == ERR_SHAPE
    assert dec(scale=-1.0) == ERR_SCALAR
    assert dec(sm=math.inf) == ERR_SCALAR
    assert dec(q=NULL) == ERR_NULL
    assert dec(out=NULL) == ERR_NULL
    assert dec(pool=NULL) == ERR_NULL
    assert dec(idx=NULL) == ERR_NULL
    assert dec(q=P8) == ERR_ALIGN
    assert dec(out=P8) == ERR_ALIGN
    assert dec(indptr=P16 + 2) == ERR_ALIGN


def test_probe_header_symbols_exported_and_validated():
    """The HBM probes' header: every declared call is exported, and bad
    arguments are rejected on the host."""
    lib = _lib()
    names = _declared_functions(PROBE_HEADER)
    assert set(names) == {"fp8mla_probe_read", "fp8mla_probe_copy_1to2", "fp8mla_probe_write",
                          "fp8mla_probe_gather_rows"}
    for n in names:
        assert hasattr(lib, n), n
    from fp8_paged_mla_amd import probe
    L = probe._lib(lib)
    assert L.fp8mla_probe_read(P16, 0, 256, 8, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_read(P16, 1000, 256, 8, P16, NULL) == ERR_SHAPE   # not a multiple of 16
    assert L.fp8mla_probe_read(P16, 1024, 0, 8, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_read(P16, 1024, 256, 5, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_read(NULL, 1024, 256, 8, P16, NULL) == ERR_NULL
    assert L.fp8mla_probe_read(P8, 1024, 256, 8, P16, NULL) == ERR_ALIGN
    assert L.fp8mla_probe_copy_1to2(P16, 1024, NULL, 256, 8, NULL) == ERR_NULL
    assert L.fp8mla_probe_copy_1to2(P16, 1040, P16, 256, 8, NULL) == ERR_SHAPE  # not whole KB
    assert L.fp8mla_probe_copy_1to2(P16, 1024, P8, 256, 8, NULL) == ERR_ALIGN
    assert L.fp8mla_probe_write(P16, 0, 256, 8, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_write(NULL, 1024, 256, 8, NULL) == ERR_NULL
    assert L.fp8mla_probe_write(P8, 1024, 256, 8, NULL) == ERR_ALIGN
    assert L.fp8mla_probe_gather_rows(P16, 0, P16, 16, 256, 2, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_gather_rows(P16, 100, P16, 17, 256, 2, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_gather_rows(P16, 100, P16, 16, 256, 3, P16, NULL) == ERR_SHAPE
    assert L.fp8mla_probe_gather_rows(P16, 100, NULL, 16, 256, 2, P16, NULL) == ERR_NULL
    assert L.fp8mla_probe_gather_rows(P16, 100, P16 + 2, 16, 256, 2, P16, NULL) == ERR_ALIGN


def test_index_check_validation_and_debug_status():
    """fp8mla_check_indices rejects bad arguments on the host; the release
    build has no accumulated check status, the debug build exports the same
    ABI."""
    lib = _lib()
    ck = lib.fp8mla_check_indices
    assert ck(P16, 0, 10, P16, 100, P16, NULL) == ERR_SHAPE       # batch 0 with an indptr
    assert ck(P16, 2, -1, P16, 100, P16, NULL) == ERR_SHAPE       # negative total
    assert ck(P16, 2, 10, P16, 0, P16, NULL) == ERR_SHAPE         # indices but no pool
    assert ck(P16, 2, 10, P16, 100, NULL, NULL) == ERR_NULL       # no status
    assert ck(P16 + 2, 2, 10, P16, 100, P16, NULL) == ERR_ALIGN
    assert ck(P16, 2, 10, P16 + 1, 100, P16, NULL) == ERR_ALIGN
    assert ck(P16, 2, 10, P16, 100, P16 + 2, NULL) == ERR_ALIGN
    out = (ctypes.c_int32 * 4)()
    not_debug = _status("FP8MLA_ERR_NOT_DEBUG")
    assert not_debug == -7
    assert lib.fp8mla_debug_status(ctypes.cast(out, ctypes.c_void_p), 0) == not_debug
    assert "debug" in fm.status_string(not_debug)
    dbg = fm.library(debug=True)
    for name in _declared_functions():
        assert hasattr(dbg, name), name
    assert dbg.fp8mla_debug_status(None, 0) == ERR_NULL
