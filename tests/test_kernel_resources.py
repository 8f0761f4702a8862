"""Register, scratch and LDS budgets of every kernel, read from the code
object metadata that hipcc writes for gfx950 (device code compiled to
assembly here, no GPU).

The pipelines rely on these budgets:
  * no kernel may use scratch: a spilled register reloaded inside a tile loop
    brings a vmcnt(0) with it, which drains the explicit copy pipelines (their
    waits count this wave's own loads);
  * the 16-head split kernel keeps two waves per SIMD (512 threads, at most
    256 registers) and the 64-row kernel three (768 threads, at most 168), with
    one workgroup per CU: both hold their tiles in LDS slots sized for that;
  * every kernel's static LDS fits one CU's 160 KiB.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest
import yaml

from fp8_paged_mla_amd import build as fb

HIP_SOURCES = [s for s in fb.SOURCES if s.endswith(".hip")]
LDS_PER_CU = 160 * 1024


def _have_hipcc():
    try:
        fb.hipcc()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc not installed")


def _kernels_of(src, tmpdir):
    out = os.path.join(tmpdir, src + ".s")
    cmd = ([fb.hipcc()] + fb.COMMON_FLAGS + fb.HIP_FLAGS +
           ["--cuda-device-only", "-S", os.path.join(fb.CSRC, src), "-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = open(out).read()
    meta = re.search(r"\.amdgpu_metadata\n(---\n.*?\n\.\.\.)\n", text, re.S)
    assert meta, src
    return yaml.safe_load(meta.group(1))["amdhsa.kernels"]


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("isa"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        per_src = list(ex.map(lambda s: _kernels_of(s, tmp), HIP_SOURCES))
    shutil.rmtree(tmp, ignore_errors=True)
    return {k[".name"]: (src, k) for src, ks in zip(HIP_SOURCES, per_src) for k in ks}


def test_every_source_has_kernels(kernels):
    assert {src for src, _ in kernels.values()} == set(HIP_SOURCES)


def test_no_scratch_no_spills(kernels):
    for name, (src, k) in kernels.items():
        assert k[".private_segment_fixed_size"] == 0, (src, name)
        assert k[".vgpr_spill_count"] == 0 and k[".sgpr_spill_count"] == 0, (src, name)
        assert not k[".uses_dynamic_stack"], (src, name)


def test_lds_fits_a_cu(kernels):
    for name, (src, k) in kernels.items():
        assert k[".group_segment_fixed_size"] <= LDS_PER_CU, (src, name)


def _waves_per_simd(k):
    return -(-k[".max_flat_workgroup_size"] // 256)  # 64-lane waves over 4 SIMDs


def _regs(k):
    # architectural VGPRs are allocated in granules of 8, accumulation
    # registers after them
    return -(-k[".vgpr_count"] // 8) * 8 + k[".agpr_count"]


@pytest.mark.parametrize("kernel,threads,max_regs", [
    ("mla_split_kernel", 512, 256),
    ("mla_split_h64_kernel", 768, 168),
])
def test_split_kernels_keep_their_occupancy(kernels, kernel, threads, max_regs):
    found = [k for name, (_, k) in kernels.items() if "%d%s" % (len(kernel), kernel) in name]
    assert len(found) == 2  # both instances (row-copy policy / extend)
    for k in found:
        assert k[".max_flat_workgroup_size"] == threads
        assert _regs(k) <= max_regs
        assert _waves_per_simd(k) * _regs(k) <= 512  # one workgroup per CU fits
