"""The allocation-free decode entry point (mla_decode_fp8_noalloc) called
through the C ABI: its output matches mla_decode_fp8's (same kernels, its
split-K scratch in the library's static per-device array instead of a caller
workspace) bit for bit, and the oracle within the attention tolerance, on
calls in a row whose second is smaller than the first."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, oracle_args

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _noalloc(lib, w, out, stream):
    return lib.mla_decode_fp8_noalloc(
        ctypes.c_void_p(w.q.data_ptr()), ctypes.c_void_p(w.pool.data_ptr()),
        ctypes.c_int64(w.pool.shape[0]), ctypes.c_void_p(w.indptr.data_ptr()),
        ctypes.c_void_p(w.indices.data_ptr()), ctypes.c_int64(w.indices.numel()),
        ctypes.c_int32(w.B), ctypes.c_int32(w.H), ctypes.c_float(w.scale),
        ctypes.c_float(w.sm_scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))


def _with_workspace(lib, w, out, stream):
    need = lib.mla_decode_fp8_workspace_bytes(w.B, w.H, w.indices.numel())
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=out.device)
    st = lib.mla_decode_fp8(
        ctypes.c_void_p(w.q.data_ptr()), ctypes.c_void_p(w.pool.data_ptr()),
        ctypes.c_int64(w.pool.shape[0]), ctypes.c_void_p(w.indptr.data_ptr()),
        ctypes.c_void_p(w.indices.data_ptr()), ctypes.c_int64(w.indices.numel()),
        ctypes.c_int32(w.B), ctypes.c_int32(w.H), ctypes.c_float(w.scale),
        ctypes.c_float(w.sm_scale), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
        ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream))
    return st, ws


@pytest.mark.parametrize("H", [16, 128])
def test_noalloc_matches_workspace_entry_point(dev, H):
    lib = fm.library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    # a larger call, then a smaller one: the second must not see the first's scratch
    cases = [workloads.small(12, H, [3000, 50, 9000, 1, 0, 640, 2049, 77, 5000, 128, 129, 7],
                             seed=500 + H, device=dev, scale=1.25),
             workloads.small(3, H, [700, 65, 1], seed=600 + H, device=dev, outlier_frac=0.01)]
    for i, w in enumerate(cases):
        print("case: noalloc H=%d call %d B=%d tokens=%d" % (H, i, w.B, w.total_tokens), flush=True)
        a = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        b = torch.full((w.B, w.H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        assert _noalloc(lib, w, a, stream) == 0
        st, ws = _with_workspace(lib, w, b, stream)
        assert st == 0
        torch.cuda.synchronize(dev)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "call %d differs" % i
        assert_attention_close(a, oracle.mla_decode_ref(*oracle_args(w)), "noalloc H=%d call %d" % (H, i))


def test_noalloc_after_other_entry_points(dev):
    """Between two allocation-free calls, the workspace entry points and the
    extend path run with garbage-filled workspaces; the second allocation-free
    call still matches."""
    lib = fm.library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    w = workloads.config(2, 1, device=dev)
    out1 = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev)
    assert _noalloc(lib, w, out1, stream) == 0
    v = workloads.small(5, 64, [4000, 1, 300, 0, 12000], seed=9, device=dev)
    ws = torch.randint(0, 256, (fm.mla_decode_fp8_workspace_bytes(v.B, v.H, v.total_tokens, dev),),
                       dtype=torch.uint8, device=dev)
    fm.mla_decode_fp8(v.q, v.pool, v.indptr, v.indices, v.scale, v.sm_scale, workspace=ws)
    out2 = torch.empty((v.B, v.H, 512), dtype=torch.bfloat16, device=dev)
    assert _noalloc(lib, v, out2, stream) == 0
    ref_out = fm.mla_decode_fp8(v.q, v.pool, v.indptr, v.indices, v.scale, v.sm_scale)
    out3 = torch.empty_like(out1)
    assert _noalloc(lib, w, out3, stream) == 0
    torch.cuda.synchronize(dev)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), ref_out.view(torch.int16))
    assert_attention_close(out1, oracle.mla_decode_ref(*oracle_args(w)), "noalloc config2 replica 1")


def test_noalloc_python_binding(dev):
    w = workloads.small(2, 32, [1000, 3], seed=4, device=dev)
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev)
    got = fm.mla_decode_fp8_noalloc(w.q, w.pool, w.indptr, w.indices, w.scale, w.sm_scale, out)
    torch.cuda.synchronize(dev)
    assert got.data_ptr() == out.data_ptr()
    assert_attention_close(out, oracle.mla_decode_ref(*oracle_args(w)), "noalloc binding")
