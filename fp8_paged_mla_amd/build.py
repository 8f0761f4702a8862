"""Build libfp8mla.so (and its debug build libfp8mla_debug.so) in-tree with
hipcc for gfx950.

    python -m fp8_paged_mla_amd.build [-v]

Each HIP/C++ translation unit is compiled in parallel into ``_build/`` at the
repository root, then linked into ``fp8_paged_mla_amd/libfp8mla.so``.  The
debug build differs only in the C ABI unit (``api.cpp`` compiled with
``FP8MLA_DEBUG_CHECKS``: every reading call first checks the index contract
on the device) and is linked into ``fp8_paged_mla_amd/libfp8mla_debug.so``.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfp8mla.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libfp8mla_debug.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "cast.hip", "scatter_cast.hip", "mla_decode.hip", "mla_decode_h64.hip",
           "mla_decode_bf16.hip", "mla_extend.hip", "index_check.hip", "hbm_probe.hip"]

COMMON_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-I" + os.path.join(ROOT, "include"),
]
# HIP device code: gfx950 only; packed-FP32 VALU forms disabled.
HIP_FLAGS = [
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libfp8mla.so)")


def _compile(job, verbose: bool) -> str:
    src, obj_name, extra = job
    obj = os.path.join(BUILD_DIR, obj_name)
    cmd = [hipcc()] + COMMON_FLAGS + HIP_FLAGS + list(extra)
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, msg))
    if verbose and msg.strip():
        print(msg)
    return obj


def _link(objs, path, verbose: bool) -> str:
    tmp = path + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("linking %s failed:\n%s%s" % (os.path.basename(path), res.stdout,
                                                         res.stderr))
    os.replace(tmp, path)
    return path


# A third library, built on request only (``build_sanitized``): the C ABI's
# host code under AddressSanitizer and UndefinedBehaviorSanitizer, every
# finding fatal, linked with the release build's other objects.  Each flag
# applies to the host pass only (device code cannot be sanitized here).  The
# runtime is not linked into a shared library: a process loading it must
# preload SANITIZER_RUNTIME.
SANITIZED_LIB_PATH = os.path.join(BUILD_DIR, "libfp8mla_sanitized.so")
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=all "
                  "-Xarch_host -fno-omit-frame-pointer").split()


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), or '' if none is installed."""
    cc = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin",
                      "clang")
    for c in (cc, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if c and os.path.exists(c):
            res = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True)
            path = res.stdout.strip()
            if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
            rt = subprocess.run([c, "-print-resource-dir"], capture_output=True, text=True)
            path = os.path.join(rt.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
            if rt.returncode == 0 and os.path.exists(path):
                return path
    return ""


def build_sanitized(verbose: bool = False) -> str:
    """Build the release objects and a sanitized C-ABI object, link
    SANITIZED_LIB_PATH and return it."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, os.path.basename(s) + ".o", ()) for s in SOURCES[1:]]
    jobs.append(("api.cpp", "api_sanitized.cpp.o", tuple(SANITIZE_FLAGS)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j, verbose), jobs))
    return _link([objs[-1]] + objs[:-1], SANITIZED_LIB_PATH, verbose)


def build(verbose: bool = False) -> str:
    """Compile every source and link both shared libraries; returns the
    release library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, os.path.basename(s) + ".o", ()) for s in SOURCES]
    jobs.append(("api.cpp", "api_debug.cpp.o", ("-DFP8MLA_DEBUG_CHECKS",)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j, verbose), jobs))
    release, debug_api = objs[:-1], objs[-1]
    _link(release, LIB_PATH, verbose)
    _link([debug_api] + release[1:], DEBUG_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    if "--sanitized" in sys.argv[1:]:
        print(build_sanitized(verbose="-v" in sys.argv[1:]))
    else:
        print(build(verbose="-v" in sys.argv[1:]))
