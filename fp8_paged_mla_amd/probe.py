"""Python binding of the HBM ceiling probes of libfp8mla.so (benchmark-only;
see include/fp8mla_probe.h).  Argument marshalling only."""
import ctypes

import torch

from . import _check, _require, _stream_handle, library

KV_WIDTH = 576


def _lib(lib=None):
    """The library (default the loaded release or debug build) with the probe
    calls' argument types set."""
    lib = library() if lib is None else lib
    if not getattr(lib, "_probe_argtypes_set", False):
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.fp8mla_probe_read.argtypes = [vp, i64, i32, i32, vp, vp]
        lib.fp8mla_probe_read.restype = ctypes.c_int
        lib.fp8mla_probe_copy_1to2.argtypes = [vp, i64, vp, i32, i32, vp]
        lib.fp8mla_probe_copy_1to2.restype = ctypes.c_int
        lib.fp8mla_probe_write.argtypes = [vp, i64, i32, i32, vp]
        lib.fp8mla_probe_write.restype = ctypes.c_int
        lib.fp8mla_probe_gather_rows.argtypes = [vp, i64, vp, i64, i32, i32, vp, vp]
        lib.fp8mla_probe_gather_rows.restype = ctypes.c_int
        lib._probe_argtypes_set = True
    return lib


def probe_read(src: torch.Tensor, grid: int, unroll: int, sink: torch.Tensor) -> None:
    """Sequential read of every byte of ``src`` (a contiguous GPU tensor)."""
    _require(src, "src")
    _require(sink, "sink", torch.int32, src.device)
    if sink.numel() < grid:
        raise ValueError("sink needs %d entries" % grid)
    nbytes = src.numel() * src.element_size()
    _check(_lib().fp8mla_probe_read(src.data_ptr(), nbytes, grid, unroll, sink.data_ptr(),
                                    _stream_handle(src.device)), "fp8mla_probe_read")


def probe_copy_1to2(src: torch.Tensor, dst: torch.Tensor, grid: int, unroll: int) -> None:
    """Each 16-byte chunk of ``src`` written twice into ``dst`` (twice the bytes)."""
    _require(src, "src")
    _require(dst, "dst", None, src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < 2 * nbytes:
        raise ValueError("dst must hold twice the bytes of src")
    _check(_lib().fp8mla_probe_copy_1to2(src.data_ptr(), nbytes, dst.data_ptr(), grid, unroll,
                                         _stream_handle(src.device)), "fp8mla_probe_copy_1to2")


def probe_write(dst: torch.Tensor, grid: int, unroll: int) -> None:
    """Sequential writes over every byte of ``dst``."""
    _require(dst, "dst")
    nbytes = dst.numel() * dst.element_size()
    _check(_lib().fp8mla_probe_write(dst.data_ptr(), nbytes, grid, unroll,
                                     _stream_handle(dst.device)), "fp8mla_probe_write")


def probe_gather_rows(pool: torch.Tensor, indices: torch.Tensor, grid: int, chunks_in_flight: int,
                      sink: torch.Tensor) -> None:
    """The 576-byte rows pool[indices[r]] gathered into LDS, no arithmetic."""
    _require(pool, "pool", torch.uint8)
    _require(indices, "indices", torch.int32, pool.device)
    _require(sink, "sink", torch.int32, pool.device)
    if pool.dim() != 2 or pool.shape[1] != KV_WIDTH:
        raise ValueError("pool must be [num_slots, 576] uint8")
    if sink.numel() < 8 * grid:
        raise ValueError("sink needs %d entries" % (8 * grid))
    _check(_lib().fp8mla_probe_gather_rows(pool.data_ptr(), pool.shape[0], indices.data_ptr(),
                                           indices.numel(), grid, chunks_in_flight, sink.data_ptr(),
                                           _stream_handle(pool.device)), "fp8mla_probe_gather_rows")
