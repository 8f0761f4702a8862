"""Python binding of libfp8mla.so: MLA decode over a paged FP8-E4M3FN latent KV
cache, the full-pool and gather-then-cast FP8->BF16 casts, and the BF16->FP8
write path into the cache, for MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libfp8mla.so``; PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

The extend (prefill) attention ``mla_extend_fp8`` serves several new query
tokens per request with a causal mask.

The operations follow three public write-ups on FP8 KV caches for MLA models:
"The KV Cache Cast Bottleneck" (the full-pool ``.to()`` cast of a
``[495552, 1, 576]`` Float8_e4m3fn pool and the native-FP8 attention that
replaces it), "The Gather-Then-Cast Pivot" (gathering only the active rows
before casting) and "When a Faster Kernel Doesn't Speed Up Serving" (the
CastFromFP8 history cast on the extend path and the CastToFP8 write of new KV
rows into the FP8 cache).
"""
import ctypes
import os

import torch

from .build import DEBUG_LIB_PATH, LIB_PATH

KV_WIDTH = 576
V_WIDTH = 512
MAX_HEADS = 256

__all__ = [
    "FP8MLAError",
    "library",
    "cast_pool_fp8_bf16",
    "gather_cast_fp8_bf16",
    "scatter_cast_bf16_fp8",
    "mla_decode_fp8",
    "mla_decode_fp8_workspace_bytes",
    "mla_decode_fp8_noalloc",
    "prepare_mla_decode_fp8",
    "PreparedCall",
    "mla_decode_bf16",
    "mla_extend_fp8",
    "mla_extend_fp8_workspace_bytes",
    "mla_decode_bf16_workspace_bytes",
    "status_string",
    "check_indices",
    "debug_status",
    "CHECK_INDPTR_START",
    "CHECK_INDPTR_ORDER",
    "CHECK_INDPTR_END",
    "CHECK_SLOT_RANGE",
    "KV_WIDTH",
    "V_WIDTH",
]


# flags of check_indices / debug_status (fp8mla.h FP8MLA_CHECK_*)
CHECK_INDPTR_START = 1
CHECK_INDPTR_ORDER = 2
CHECK_INDPTR_END = 4
CHECK_SLOT_RANGE = 8


class FP8MLAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed with status %d: %s" % (where, code, status_string(code)))


_LIB = None
_DEBUG_LIB = None


def library(debug: bool = None) -> ctypes.CDLL:
    """The loaded libfp8mla.so (raises if it has not been built).

    ``debug=True`` loads the debug build libfp8mla_debug.so instead (same
    ABI; every reading call checks the index contract on the device first, see
    debug_status); by default the debug build is used when the environment
    sets FP8MLA_DEBUG=1."""
    global _LIB, _DEBUG_LIB
    if debug is None:
        debug = os.environ.get("FP8MLA_DEBUG", "0") == "1"
    if debug and _DEBUG_LIB is not None:
        return _DEBUG_LIB
    if not debug and _LIB is not None:
        return _LIB
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            "%s is not built (%s missing); run `python -m fp8_paged_mla_amd.build`"
            % (os.path.basename(path), path))
    lib = _bind(ctypes.CDLL(path))
    if debug:
        _DEBUG_LIB = lib
    else:
        _LIB = lib
    return lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.cast_pool_fp8_bf16.argtypes = [vp, i64, vp, vp]
    lib.cast_pool_fp8_bf16.restype = ctypes.c_int
    lib.gather_cast_fp8_bf16.argtypes = [vp, i64, vp, i64, vp, vp]
    lib.gather_cast_fp8_bf16.restype = ctypes.c_int
    lib.scatter_cast_bf16_fp8.argtypes = [vp, i64, i64, vp, vp, i64, f32, i32, vp]
    lib.scatter_cast_bf16_fp8.restype = ctypes.c_int
    lib.mla_decode_fp8.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, f32, f32, vp, vp, sz, vp]
    lib.mla_decode_fp8.restype = ctypes.c_int
    lib.mla_decode_fp8_segments.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, f32, f32, vp, vp,
                                            sz, i32, vp]
    lib.mla_decode_fp8_segments.restype = ctypes.c_int
    lib.mla_decode_fp8_noalloc.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, f32, f32, vp, vp]
    lib.mla_decode_fp8_noalloc.restype = ctypes.c_int
    lib.mla_decode_fp8_workspace_bytes.argtypes = [i32, i32, i64]
    lib.mla_decode_fp8_workspace_bytes.restype = sz
    lib.mla_extend_fp8.argtypes = [vp, vp, i64, vp, vp, vp, i64, i64, i32, i32, f32, f32, i32,
                                   vp, vp, sz, vp]
    lib.mla_extend_fp8.restype = ctypes.c_int
    lib.mla_extend_fp8_workspace_bytes.argtypes = [i32, i32, i64]
    lib.mla_extend_fp8_workspace_bytes.restype = sz
    lib.mla_decode_bf16.argtypes = [vp, vp, i64, vp, vp, i64, i32, i32, f32, f32, vp, vp, sz, vp]
    lib.mla_decode_bf16.restype = ctypes.c_int
    lib.mla_decode_bf16_workspace_bytes.argtypes = [i32, i32, i64]
    lib.mla_decode_bf16_workspace_bytes.restype = sz
    lib.fp8mla_check_indices.argtypes = [vp, i32, i64, vp, i64, vp, vp]
    lib.fp8mla_check_indices.restype = ctypes.c_int
    lib.fp8mla_debug_status.argtypes = [vp, i32]
    lib.fp8mla_debug_status.restype = ctypes.c_int
    lib.fp8mla_status_string.argtypes = [ctypes.c_int]
    lib.fp8mla_status_string.restype = ctypes.c_char_p
    lib.fp8mla_abi_version.argtypes = []
    lib.fp8mla_abi_version.restype = ctypes.c_int
    return lib


def status_string(code: int) -> str:
    return library().fp8mla_status_string(int(code)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FP8MLAError(status, where)


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _as_bytes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError("%s must be float8_e4m3fn or uint8 (E4M3FN bytes), got %s" % (name, t.dtype))
    return t


def _require(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _pool_rows(pool: torch.Tensor) -> torch.Tensor:
    """Accept [num_slots, 576] or the pages' [num_slots, 1, 576] view."""
    pool = _as_bytes(pool, "pool")
    if pool.dim() == 3 and pool.shape[1] == 1:
        pool = pool.view(pool.shape[0], pool.shape[2])
    if pool.dim() != 2 or pool.shape[1] != KV_WIDTH:
        raise ValueError("pool must be [num_slots, 576] (or [num_slots, 1, 576]), got %s"
                         % (tuple(pool.shape),))
    return pool


def cast_pool_fp8_bf16(pool: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """BF16 copy of a whole FP8 pool: ``out[i, j] = bf16(e4m3fn(pool[i, j]))``."""
    pool = _pool_rows(pool)
    _require(pool, "pool")
    dev = pool.device
    if out is None:
        out = torch.empty(pool.shape, dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != tuple(pool.shape):
        raise ValueError("out must be %s" % (tuple(pool.shape),))
    with torch.cuda.device(dev):
        _check(library().cast_pool_fp8_bf16(pool.data_ptr(), pool.shape[0], out.data_ptr(),
                                            _stream_handle(dev)), "cast_pool_fp8_bf16")
    return out


def gather_cast_fp8_bf16(pool: torch.Tensor, indices: torch.Tensor,
                         out: torch.Tensor = None) -> torch.Tensor:
    """Compact BF16 rows of the slots named by ``indices``: ``out[r] = bf16(pool[indices[r]])``."""
    pool = _pool_rows(pool)
    _require(pool, "pool")
    dev = pool.device
    _require(indices, "indices", torch.int32, dev)
    if indices.dim() != 1:
        raise ValueError("indices must be 1-D")
    n = indices.shape[0]
    if out is None:
        out = torch.empty((n, KV_WIDTH), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (n, KV_WIDTH):
        raise ValueError("out must be [%d, 576]" % n)
    with torch.cuda.device(dev):
        _check(library().gather_cast_fp8_bf16(pool.data_ptr(), pool.shape[0], indices.data_ptr(), n,
                                              out.data_ptr(), _stream_handle(dev)),
               "gather_cast_fp8_bf16")
    return out


def scatter_cast_bf16_fp8(src: torch.Tensor, slots: torch.Tensor, pool: torch.Tensor,
                          inv_scale: float = 1.0, saturate: bool = False) -> torch.Tensor:
    """Write path: ``pool[slots[r], :] = e4m3fn(float32(src[r, :]) * inv_scale)``, in place.

    src [n, 576] (or [n, 1, 576]) bf16 whose rows may be strided (last dim
    contiguous, row stride a multiple of 8); slots [n] int32, distinct; pool
    [num_slots, 576] E4M3FN bytes.  Rows whose slot is outside the pool are
    skipped.  ``saturate`` clamps overflow to +-448 instead of giving NaN.
    Returns ``pool``.
    """
    pool_rows = _pool_rows(pool)
    _require(pool_rows, "pool")
    dev = pool_rows.device
    if not isinstance(src, torch.Tensor) or src.device != dev or src.dtype != torch.bfloat16:
        raise TypeError("src must be a bfloat16 tensor on %s" % dev)
    if src.dim() == 3 and src.shape[1] == 1:
        src = src[:, 0, :]
    if src.dim() != 2 or src.shape[1] != KV_WIDTH:
        raise ValueError("src must be [n, 576] (or [n, 1, 576]), got %s" % (tuple(src.shape),))
    n = src.shape[0]
    row_stride = src.stride(0) if n > 1 else max(src.stride(0), KV_WIDTH)
    if src.stride(1) != 1:
        raise ValueError("src rows must be contiguous")
    _require(slots, "slots", torch.int32, dev)
    if slots.dim() != 1 or slots.shape[0] != n:
        raise ValueError("slots must be [%d]" % n)
    with torch.cuda.device(dev):
        _check(library().scatter_cast_bf16_fp8(src.data_ptr(), n, row_stride, slots.data_ptr(),
                                               pool_rows.data_ptr(), pool_rows.shape[0],
                                               float(inv_scale), 1 if saturate else 0,
                                               _stream_handle(dev)),
               "scatter_cast_bf16_fp8")
    return pool


def mla_extend_fp8_workspace_bytes(batch: int, num_heads: int, total_q: int, device=None) -> int:
    """Bytes of workspace mla_extend_fp8 needs (scratch; no initialisation)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        return int(library().mla_extend_fp8_workspace_bytes(int(batch), int(num_heads), int(total_q)))


def mla_extend_fp8(q: torch.Tensor, kv_pool: torch.Tensor, qo_indptr: torch.Tensor,
                   kv_indptr: torch.Tensor, kv_indices: torch.Tensor, scale: float,
                   sm_scale: float, causal: bool = True, out: torch.Tensor = None,
                   workspace: torch.Tensor = None) -> torch.Tensor:
    """Extend (prefill) attention reading the FP8 pool directly.

    q [total_q, H, 576] bf16 (request b's new tokens are rows
    qo_indptr[b]:qo_indptr[b+1]); kv_pool [num_slots, 576] E4M3FN;
    qo_indptr, kv_indptr [B+1] int32; kv_indices int32 slot ids (the last
    q_len_b entries of request b's list are its new tokens).  With ``causal``
    token i of request b sees the first kv_len_b - q_len_b + i + 1 tokens.
    Returns out [total_q, H, 512] bf16.
    """
    kv_pool = _pool_rows(kv_pool)
    _require(q, "q", torch.bfloat16)
    dev = q.device
    _require(kv_pool, "kv_pool", None, dev)
    _require(qo_indptr, "qo_indptr", torch.int32, dev)
    _require(kv_indptr, "kv_indptr", torch.int32, dev)
    _require(kv_indices, "kv_indices", torch.int32, dev)
    if q.dim() != 3 or q.shape[2] != KV_WIDTH:
        raise ValueError("q must be [total_q, H, 576], got %s" % (tuple(q.shape),))
    total_q, H = q.shape[0], q.shape[1]
    if qo_indptr.dim() != 1 or kv_indptr.dim() != 1 or qo_indptr.shape != kv_indptr.shape:
        raise ValueError("qo_indptr and kv_indptr must both be [B+1]")
    B = qo_indptr.shape[0] - 1
    if B < 1:
        raise ValueError("need at least one request")
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    if out is None:
        out = torch.empty((total_q, H, V_WIDTH), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (total_q, H, V_WIDTH):
        raise ValueError("out must be [%d, %d, 512]" % (total_q, H))
    need = mla_extend_fp8_workspace_bytes(B, H, total_q, dev)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _require(workspace, "workspace", torch.uint8, dev)
    with torch.cuda.device(dev):
        _check(library().mla_extend_fp8(q.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                                        qo_indptr.data_ptr(), kv_indptr.data_ptr(),
                                        kv_indices.data_ptr(), total_q, kv_indices.shape[0], B, H,
                                        float(scale), float(sm_scale), 1 if causal else 0,
                                        out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                        _stream_handle(dev)),
               "mla_extend_fp8")
    return out


def mla_decode_fp8_workspace_bytes(batch: int, num_heads: int, total_tokens: int,
                                   device=None) -> int:
    """Bytes of workspace mla_decode_fp8 needs (scratch; no initialisation)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        return int(library().mla_decode_fp8_workspace_bytes(int(batch), int(num_heads),
                                                            int(total_tokens)))


def mla_decode_fp8(q: torch.Tensor, kv_pool: torch.Tensor, kv_indptr: torch.Tensor,
                   kv_indices: torch.Tensor, scale: float, sm_scale: float,
                   out: torch.Tensor = None, workspace: torch.Tensor = None,
                   segments: int = None) -> torch.Tensor:
    """Fused MLA decode reading the FP8 pool directly.

    q [B, H, 576] bf16; kv_pool [num_slots, 576] E4M3FN; kv_indptr [B+1] int32;
    kv_indices [kv_indptr[B]] int32 slot ids; returns out [B, H, 512] bf16.
    ``segments`` bounds the split-K partition (mla_decode_fp8_segments);
    None keeps the library's own.
    """
    kv_pool = _pool_rows(kv_pool)
    _require(q, "q", torch.bfloat16)
    dev = q.device
    _require(kv_pool, "kv_pool", None, dev)
    _require(kv_indptr, "kv_indptr", torch.int32, dev)
    _require(kv_indices, "kv_indices", torch.int32, dev)
    if q.dim() != 3 or q.shape[2] != KV_WIDTH:
        raise ValueError("q must be [B, H, 576], got %s" % (tuple(q.shape),))
    B, H = q.shape[0], q.shape[1]
    if kv_indptr.dim() != 1 or kv_indptr.shape[0] != B + 1:
        raise ValueError("kv_indptr must be [B+1]")
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    total = kv_indices.shape[0]
    if out is None:
        out = torch.empty((B, H, V_WIDTH), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (B, H, V_WIDTH):
        raise ValueError("out must be [%d, %d, 512]" % (B, H))
    lib = library()
    with torch.cuda.device(dev):
        need = int(lib.mla_decode_fp8_workspace_bytes(B, H, total))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _require(workspace, "workspace", torch.uint8, dev)
        ws_bytes = workspace.numel()
        if segments is None:
            _check(lib.mla_decode_fp8(q.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                                      kv_indptr.data_ptr(), kv_indices.data_ptr(), total, B, H,
                                      float(scale), float(sm_scale), out.data_ptr(),
                                      workspace.data_ptr(), ws_bytes, _stream_handle(dev)),
                   "mla_decode_fp8")
        else:
            _check(lib.mla_decode_fp8_segments(q.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                                               kv_indptr.data_ptr(), kv_indices.data_ptr(), total,
                                               B, H, float(scale), float(sm_scale),
                                               out.data_ptr(), workspace.data_ptr(), ws_bytes,
                                               int(segments), _stream_handle(dev)),
                   "mla_decode_fp8_segments")
    return out


def mla_decode_fp8_noalloc(q: torch.Tensor, kv_pool: torch.Tensor, kv_indptr: torch.Tensor,
                           kv_indices: torch.Tensor, scale: float, sm_scale: float,
                           out: torch.Tensor) -> torch.Tensor:
    """mla_decode_fp8 without a workspace (its split-K scratch is a static
    array inside the library, one per GPU): for callers that cannot allocate.
    The caller passes ``out`` [B, H, 512] bf16; nothing is allocated.  Calls
    that may overlap on one GPU share that scratch and must not be issued."""
    kv_pool = _pool_rows(kv_pool)
    _require(q, "q", torch.bfloat16)
    dev = q.device
    _require(kv_pool, "kv_pool", None, dev)
    _require(kv_indptr, "kv_indptr", torch.int32, dev)
    _require(kv_indices, "kv_indices", torch.int32, dev)
    _require(out, "out", torch.bfloat16, dev)
    if q.dim() != 3 or q.shape[2] != KV_WIDTH:
        raise ValueError("q must be [B, H, 576], got %s" % (tuple(q.shape),))
    B, H = q.shape[0], q.shape[1]
    if kv_indptr.dim() != 1 or kv_indptr.shape[0] != B + 1:
        raise ValueError("kv_indptr must be [B+1]")
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    if tuple(out.shape) != (B, H, V_WIDTH):
        raise ValueError("out must be [%d, %d, 512]" % (B, H))
    with torch.cuda.device(dev):
        _check(library().mla_decode_fp8_noalloc(q.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                                                kv_indptr.data_ptr(), kv_indices.data_ptr(),
                                                kv_indices.shape[0], B, H, float(scale),
                                                float(sm_scale), out.data_ptr(), _stream_handle(dev)),
               "mla_decode_fp8_noalloc")
    return out


class PreparedCall:
    """One library call whose arguments were checked and marshalled once.

    Calling it re-issues the same C-ABI call on the same buffers (whose
    contents may change between calls) and stream, with no per-call Python
    argument handling: for serving loops and small calls, where the
    binding's own checks would otherwise cost more host time than the GPU
    spends.  The library still validates every call on the host.  The
    tensors are kept alive by the object."""

    def __init__(self, fn, args, keep, result, where):
        self._fn = fn
        self._args = args
        self._keep = keep
        self.result = result
        self._where = where

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise FP8MLAError(st, self._where)
        return self.result


def prepare_mla_decode_fp8(q: torch.Tensor, kv_pool: torch.Tensor, kv_indptr: torch.Tensor,
                           kv_indices: torch.Tensor, scale: float, sm_scale: float,
                           out: torch.Tensor = None, workspace: torch.Tensor = None,
                           stream=None, segments: int = None) -> PreparedCall:
    """mla_decode_fp8 with its arguments checked and marshalled once; returns
    a callable that enqueues the call (on ``stream``, default the current
    stream at preparation) and returns ``out``.  ``segments`` bounds the
    split-K partition (mla_decode_fp8_segments)."""
    kv_pool = _pool_rows(kv_pool)
    _require(q, "q", torch.bfloat16)
    dev = q.device
    _require(kv_pool, "kv_pool", None, dev)
    _require(kv_indptr, "kv_indptr", torch.int32, dev)
    _require(kv_indices, "kv_indices", torch.int32, dev)
    if q.dim() != 3 or q.shape[2] != KV_WIDTH:
        raise ValueError("q must be [B, H, 576], got %s" % (tuple(q.shape),))
    B, H = q.shape[0], q.shape[1]
    if kv_indptr.dim() != 1 or kv_indptr.shape[0] != B + 1:
        raise ValueError("kv_indptr must be [B+1]")
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    total = kv_indices.shape[0]
    if out is None:
        out = torch.empty((B, H, V_WIDTH), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (B, H, V_WIDTH):
        raise ValueError("out must be [%d, %d, 512]" % (B, H))
    lib = library()
    with torch.cuda.device(dev):
        need = int(lib.mla_decode_fp8_workspace_bytes(B, H, total))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _require(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError("workspace needs %d bytes" % need)
        handle = _stream_handle(dev) if stream is None else stream.cuda_stream
    c = ctypes
    args = (c.c_void_p(q.data_ptr()), c.c_void_p(kv_pool.data_ptr()), c.c_int64(kv_pool.shape[0]),
            c.c_void_p(kv_indptr.data_ptr()), c.c_void_p(kv_indices.data_ptr()), c.c_int64(total),
            c.c_int32(B), c.c_int32(H), c.c_float(float(scale)), c.c_float(float(sm_scale)),
            c.c_void_p(out.data_ptr()), c.c_void_p(workspace.data_ptr()),
            c.c_size_t(workspace.numel()), c.c_void_p(handle))
    keep = (q, kv_pool, kv_indptr, kv_indices, out, workspace)
    if segments is not None:
        args = args[:-1] + (c.c_int32(int(segments)), args[-1])
        return PreparedCall(lib.mla_decode_fp8_segments, args, keep, out, "mla_decode_fp8_segments")
    return PreparedCall(lib.mla_decode_fp8, args, keep, out, "mla_decode_fp8")


def mla_decode_bf16_workspace_bytes(batch: int, num_heads: int, total_tokens: int,
                                    device=None) -> int:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        return int(library().mla_decode_bf16_workspace_bytes(int(batch), int(num_heads),
                                                             int(total_tokens)))


def mla_decode_bf16(q: torch.Tensor, kv: torch.Tensor, kv_indptr: torch.Tensor,
                    kv_indices: torch.Tensor, scale: float, sm_scale: float,
                    out: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """The same decode over BF16 latent rows (benchmark-only: the attention of
    the cast-then-attend fallback paths).

    q [B, H, 576] bf16; kv [num_rows, 576] bf16 (e.g. a cast pool or a
    gathered buffer); kv_indptr [B+1] int32; kv_indices int32 row ids.
    """
    if kv.dim() == 3 and kv.shape[1] == 1:
        kv = kv.view(kv.shape[0], kv.shape[2])
    _require(q, "q", torch.bfloat16)
    dev = q.device
    _require(kv, "kv", torch.bfloat16, dev)
    _require(kv_indptr, "kv_indptr", torch.int32, dev)
    _require(kv_indices, "kv_indices", torch.int32, dev)
    if kv.dim() != 2 or kv.shape[1] != KV_WIDTH:
        raise ValueError("kv must be [num_rows, 576], got %s" % (tuple(kv.shape),))
    if q.dim() != 3 or q.shape[2] != KV_WIDTH:
        raise ValueError("q must be [B, H, 576], got %s" % (tuple(q.shape),))
    B, H = q.shape[0], q.shape[1]
    if kv_indptr.dim() != 1 or kv_indptr.shape[0] != B + 1:
        raise ValueError("kv_indptr must be [B+1]")
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    total = kv_indices.shape[0]
    if out is None:
        out = torch.empty((B, H, V_WIDTH), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != (B, H, V_WIDTH):
        raise ValueError("out must be [%d, %d, 512]" % (B, H))
    lib = library()
    with torch.cuda.device(dev):
        need = int(lib.mla_decode_bf16_workspace_bytes(B, H, total))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _require(workspace, "workspace", torch.uint8, dev)
        _check(lib.mla_decode_bf16(q.data_ptr(), kv.data_ptr(), kv.shape[0], kv_indptr.data_ptr(),
                                   kv_indices.data_ptr(), total, B, H, float(scale), float(sm_scale),
                                   out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream_handle(dev)), "mla_decode_bf16")
    return out


def check_indices(indptr: torch.Tensor = None, indices: torch.Tensor = None, num_slots: int = 0,
                  total: int = None, status: torch.Tensor = None) -> torch.Tensor:
    """On-device check of an index layout (fp8mla_check_indices): indptr
    [B+1] int32 starts at 0, never decreases and ends at ``total`` (default
    len(indices)); every slot id lies in [0, num_slots).  Either array may be
    None.  Returns the device int32 [4] status: FP8MLA_CHECK_* flags (0 = the
    contract holds), first bad request, first bad slot position (INT32_MAX
    when none), number of bad slot ids."""
    ref = indptr if indptr is not None else indices
    if ref is None:
        raise ValueError("give indptr, indices or both")
    dev = ref.device
    B = 0
    if indptr is not None:
        _require(indptr, "indptr", torch.int32, dev)
        if indptr.dim() != 1 or indptr.shape[0] < 2:
            raise ValueError("indptr must be [B+1] with B >= 1")
        B = indptr.shape[0] - 1
    if indices is not None:
        _require(indices, "indices", torch.int32, dev)
        if indices.dim() != 1:
            raise ValueError("indices must be 1-D")
    if total is None:
        if indices is None:
            raise ValueError("total is needed without indices")
        total = indices.shape[0]
    if indices is not None and indices.shape[0] < total:
        raise ValueError("indices holds fewer than total entries")
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=dev)
    _require(status, "status", torch.int32, dev)
    with torch.cuda.device(dev):
        _check(library().fp8mla_check_indices(
            indptr.data_ptr() if indptr is not None else None, B, int(total),
            indices.data_ptr() if indices is not None else None, int(num_slots),
            status.data_ptr(), _stream_handle(dev)), "fp8mla_check_indices")
    return status


def debug_status(reset: bool = False, device=None) -> list:
    """The debug build's accumulated index-check status on ``device`` (waits
    for the device to finish): [flags, first bad request, first bad slot
    position, bad slot count].  Raises on the release build."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    out = (ctypes.c_int32 * 4)()
    with torch.cuda.device(dev):
        _check(library(debug=True).fp8mla_debug_status(ctypes.cast(out, ctypes.c_void_p),
                                                       1 if reset else 0), "fp8mla_debug_status")
    return [int(v) for v in out]
