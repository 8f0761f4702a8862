"""On-device checks of the index contract (fp8mla_check_indices, and the
debug build that runs them inside every reading call).  Each broken layout
is planted in a copy of a valid one and must raise exactly its flag, with the
first bad position; the reading calls themselves clamp such entries, so a
debug-built decode with one bad slot id still matches the oracle on every
other request."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import assert_attention_close, oracle_args

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("fp8_paged_mla_amd")

NONE = 2 ** 31 - 1


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _status(st):
    torch.cuda.synchronize()
    return st.cpu().tolist()


def test_valid_layouts_pass(dev):
    for cfg in (1, 2, 5):
        w = workloads.config(cfg, device=dev)
        print("case: check config %d" % cfg, flush=True)
        st = fm.check_indices(w.indptr, w.indices, w.num_slots)
        assert _status(st) == [0, NONE, NONE, 0], cfg


def test_planted_violations(dev):
    w = workloads.small(6, 16, [300, 0, 70, 1000, 5, 64], seed=3, device=dev)
    ip, ix = w.indptr.clone(), w.indices.clone()
    print("case: planted index violations", flush=True)
    # indptr[0] != 0
    bad = ip.clone()
    bad[0] = 1
    assert _status(fm.check_indices(bad, ix, w.num_slots))[0] == fm.CHECK_INDPTR_START
    # a decrease between requests 3 and 4
    bad = ip.clone()
    bad[4] = bad[3] - 1
    s = _status(fm.check_indices(bad, ix, w.num_slots))
    assert s[0] == fm.CHECK_INDPTR_ORDER and s[1] == 3
    # indptr[B] != total
    s = _status(fm.check_indices(ip, ix, w.num_slots, total=int(ip[-1]) - 1))
    assert s[0] == fm.CHECK_INDPTR_END
    # slot ids: one past the pool, one negative, one far past
    badx = ix.clone()
    pos = [17, 401, 1300]
    badx[pos[0]] = w.num_slots
    badx[pos[1]] = -5
    badx[pos[2]] = 2 ** 31 - 1
    s = _status(fm.check_indices(ip, badx, w.num_slots))
    assert s == [fm.CHECK_SLOT_RANGE, NONE, pos[0], 3]
    # indices only (a gather list), and indptr only (a query CSR)
    s = _status(fm.check_indices(None, badx, w.num_slots))
    assert s == [fm.CHECK_SLOT_RANGE, NONE, pos[0], 3]
    assert _status(fm.check_indices(ip, None, 0, total=int(ip[-1]))) == [0, NONE, NONE, 0]
    # a status buffer holding an earlier result is reset by the next check
    st = fm.check_indices(ip, badx, w.num_slots)
    fm.check_indices(ip, ix, w.num_slots, status=st)
    assert _status(st) == [0, NONE, NONE, 0]


def test_debug_build_decode_reports_bad_slot(dev):
    """The debug build's decode, given one out-of-range slot id in request 2,
    records it in the device's check status; the other requests' rows match
    the oracle (the read path clamps the bad id, so nothing faults)."""
    dbg = fm.library(debug=True)
    fm.debug_status(reset=True)
    w = workloads.small(5, 16, [700, 64, 300, 1, 2049], seed=8, device=dev)
    bad_pos = int(w.indptr[2]) + 17
    idx = w.indices.clone()
    idx[bad_pos] = w.num_slots + 1000
    out = torch.empty((w.B, w.H, 512), dtype=torch.bfloat16, device=dev)
    need = dbg.mla_decode_fp8_workspace_bytes(w.B, w.H, idx.numel())
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    print("case: debug-build decode with a bad slot id", flush=True)
    st = dbg.mla_decode_fp8(w.q.data_ptr(), w.pool.data_ptr(), w.pool.shape[0], w.indptr.data_ptr(),
                            idx.data_ptr(), idx.numel(), w.B, w.H, w.scale, w.sm_scale,
                            out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0
    s = fm.debug_status(reset=True)
    assert s == [fm.CHECK_SLOT_RANGE, NONE, bad_pos, 1]
    assert fm.debug_status() == [0, NONE, NONE, 0]  # cleared
    good = [0, 1, 3, 4]
    ref = oracle.mla_decode_ref(*oracle_args(w), requests=good)
    assert_attention_close(out[good], ref, "debug decode, valid requests")
    # the same call on valid indices leaves the status clear
    st = dbg.mla_decode_fp8(w.q.data_ptr(), w.pool.data_ptr(), w.pool.shape[0], w.indptr.data_ptr(),
                            w.indices.data_ptr(), w.indices.numel(), w.B, w.H, w.scale, w.sm_scale,
                            out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0
    assert fm.debug_status(reset=True) == [0, NONE, NONE, 0]


def test_debug_build_extend_and_gather(dev):
    """Extend checks both CSRs (a query CSR that ends past total_q is
    flagged); gather checks its slot list."""
    dbg = fm.library(debug=True)
    fm.debug_status(reset=True)
    e = workloads.extend(2, 16, [3, 5], [40, 7], seed=6)
    q, pool = e.q.to(dev), e.pool.to(dev)
    qo, kv, ki = e.qo_indptr.to(dev), e.kv_indptr.to(dev), e.kv_indices.to(dev)
    out = torch.empty((e.total_q, e.H, 512), dtype=torch.bfloat16, device=dev)
    need = dbg.mla_extend_fp8_workspace_bytes(e.B, e.H, e.total_q)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    print("case: debug-build extend and gather", flush=True)
    args = (q.data_ptr(), pool.data_ptr(), pool.shape[0], qo.data_ptr(), kv.data_ptr(),
            ki.data_ptr(), e.total_q, ki.numel(), e.B, e.H, e.scale, e.sm_scale, 1,
            out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert dbg.mla_extend_fp8(*args) == 0
    assert fm.debug_status(reset=True) == [0, NONE, NONE, 0]
    # total_q one larger than qo_indptr's last entry: the query CSR's end is wrong
    big_out = torch.empty((e.total_q + 1, e.H, 512), dtype=torch.bfloat16, device=dev)
    q1 = torch.cat([q, q[:1]]).contiguous()
    need1 = dbg.mla_extend_fp8_workspace_bytes(e.B, e.H, e.total_q + 1)
    ws1 = torch.empty(max(need1, 256), dtype=torch.uint8, device=dev)
    args1 = (q1.data_ptr(), pool.data_ptr(), pool.shape[0], qo.data_ptr(), kv.data_ptr(),
             ki.data_ptr(), e.total_q + 1, ki.numel(), e.B, e.H, e.scale, e.sm_scale, 1,
             big_out.data_ptr(), ws1.data_ptr(), ws1.numel(), stream)
    assert dbg.mla_extend_fp8(*args1) == 0
    assert fm.debug_status(reset=True)[0] == fm.CHECK_INDPTR_END
    # gather with a negative slot id at position 5
    idx = ki.clone()
    idx[5] = -1
    g = torch.empty((idx.numel(), 576), dtype=torch.bfloat16, device=dev)
    assert dbg.gather_cast_fp8_bf16(pool.data_ptr(), pool.shape[0], idx.data_ptr(), idx.numel(),
                                    g.data_ptr(), stream) == 0
    assert fm.debug_status(reset=True) == [fm.CHECK_SLOT_RANGE, NONE, 5, 1]
