"""Binding of the benchmark's measurement probes (libtv_probe.so, include/tv_probe.h).

Not part of the verify step: a plain HBM read stream (contiguous or in the KV cache's
pattern) and a shader-clock counter, the two ceilings the attention kernel's bandwidth is
set against. Argument marshalling only; raises if the library is missing.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import PROBE_LIB_PATH

_lib = None
_lock = threading.Lock()

EXPORTS = ("tv_probe_stream_read", "tv_probe_clock")


def lib():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(PROBE_LIB_PATH):
                raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                                   "`python -m draft_tree_verification_tv_amd.build`")
            L = ctypes.CDLL(PROBE_LIB_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
            L.tv_probe_stream_read.restype = i32
            L.tv_probe_stream_read.argtypes = [vp, i64, i32, i64, i32, i64, vp, vp]
            L.tv_probe_clock.restype = i32
            L.tv_probe_clock.argtypes = [vp, ctypes.c_uint64, vp]
            _lib = L
    return _lib


def _stream(stream):
    return (stream or torch.cuda.current_stream()).cuda_stream


def stream_read_grid(rows, cols, rows_per_wg):
    return -(-rows // rows_per_wg) * cols


def stream_read(buf: torch.Tensor, rows: int, row_bytes: int, row_stride: int, cols: int, rows_per_wg: int,
                sink: torch.Tensor, stream=None):
    """Read rows x cols blocks of row_bytes bytes (block (r, c) at r * row_stride +
    c * row_bytes) from the device buffer ``buf``; sink is a uint32 device tensor with one
    entry per workgroup (``stream_read_grid``)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    need = (rows - 1) * row_stride + cols * row_bytes
    if need > buf.numel() * buf.element_size():
        raise ValueError(f"buf holds {buf.numel() * buf.element_size()} bytes, the pattern reads up to {need}")
    if sink.dtype != torch.int32 or not sink.is_cuda or sink.numel() < stream_read_grid(rows, cols, rows_per_wg):
        raise ValueError("sink must be an int32 device tensor with one entry per workgroup")
    st = lib().tv_probe_stream_read(buf.data_ptr(), rows, row_bytes, row_stride, cols, rows_per_wg,
                                    sink.data_ptr(), _stream(stream))
    if st != 0:
        raise RuntimeError(f"tv_probe_stream_read failed with status {st}")


def clock(out: torch.Tensor, ticks: int, stream=None):
    """One wave spins for ``ticks`` real-time ticks; out (int64 [2]) receives the shader
    cycles and real-time ticks elapsed."""
    if out.dtype != torch.int64 or not out.is_cuda or out.numel() < 2:
        raise ValueError("out must be an int64 device tensor of two entries")
    st = lib().tv_probe_clock(out.data_ptr(), int(ticks), _stream(stream))
    if st != 0:
        raise RuntimeError(f"tv_probe_clock failed with status {st}")
