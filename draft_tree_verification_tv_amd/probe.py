"""Binding of the benchmark's measurement probes (libtv_probe.so, include/tv_probe.h).

Not part of the verify step: a plain HBM read stream (contiguous or in the KV cache's
pattern) and a shader-clock counter, the two ceilings the attention kernel's bandwidth is
set against; an MFMA/VALU co-issue timer on one CU; and a whole-chip run of MFMA streams
with LDS reads and VALU work beside them. Argument marshalling only; raises if the library
is missing.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import PROBE_LIB_PATH

_lib = None
_lock = threading.Lock()

EXPORTS = ("tv_probe_stream_read", "tv_probe_clock", "tv_probe_coissue", "tv_probe_mix")

COISSUE_MODES = ("MFMA only (8 per iteration)", "VALU only (64 FMA)", "MFMA + 8 FMA each",
                 "MFMA + 4 exp2 + 4 FMA each", "exp2 only (64)", "MFMA + 2 exp2 + 6 FMA each")


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
            L.tv_probe_coissue.restype = i32
            L.tv_probe_coissue.argtypes = [i32, i32, i32, vp, vp, vp, vp]
            L.tv_probe_mix.restype = i32
            L.tv_probe_mix.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
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


def coissue(mode: int, threads: int, iters: int = 2000):
    """Shader-clock cycles per iteration of instruction mix ``mode`` (COISSUE_MODES), the
    mean over the workgroup's waves (one workgroup of ``threads`` threads, so 64 gives one
    wave alone on a SIMD and 512 two waves on every SIMD of a CU)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    src = (torch.arange(1024, device=dev, dtype=torch.float32) % 17) * 1e-3
    out = torch.empty(512, dtype=torch.float32, device=dev)
    cyc = torch.zeros(8, dtype=torch.int64, device=dev)
    for _ in range(2):  # the first launch loads the code
        st = lib().tv_probe_coissue(int(mode), int(threads), int(iters), src.data_ptr(), out.data_ptr(),
                                    cyc.data_ptr(), _stream(None))
        if st != 0:
            raise RuntimeError(f"tv_probe_coissue failed with status {st}")
        torch.cuda.synchronize()
    waves = threads // 64
    return float(cyc[:waves].double().mean()) / iters


MIX_CASES = ((0, 0, "MFMA only"), (1, 0, "MFMA + 1 KB LDS reads each"), (0, 1, "MFMA + exp2 + 4 FMA each"),
             (1, 1, "MFMA + 1 KB LDS + exp2 + 4 FMA each"), (2, 1, "MFMA + 0.5 KB LDS + exp2 + 4 FMA each"),
             (5, 0, "MFMA + K fragment (swizzled 128-bit)"), (4, 0, "MFMA + V^T fragment (2 transposed reads)"),
             (3, 0, "MFMA + K / V^T fragments alternating"), (3, 1, "MFMA + K / V^T + exp2 + 4 FMA each"),
             (6, 1, "64-row wave: K,-,V^T,- + exp2 + 4 FMA each"), (7, 1, "64-row wave: K,K,V^T,- + exp2 + 4 FMA"))


def mix(lds_step: int, valu: int, threads: int, iters: int = 20000):
    """Whole-chip bf16 MFMA throughput (TFLOP/s, from HIP events) and the shader clock (GHz)
    of the instruction mix (lds_step, valu) with threads / 128 waves per SIMD, one
    workgroup per CU."""
    dev = torch.device("cuda", torch.cuda.current_device())
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    src = (torch.arange(1024, device=dev, dtype=torch.float32) % 17) * 1e-3
    out = torch.empty(cus * threads, dtype=torch.float32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(2):  # the first launch loads the code and lets the clock settle
        e0.record(stream)
        st = lib().tv_probe_mix(int(lds_step), int(valu), int(threads), cus, int(iters), src.data_ptr(),
                                out.data_ptr(), clk.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        if st != 0:
            raise RuntimeError(f"tv_probe_mix failed with status {st}")
        torch.cuda.synchronize()
        best = e0.elapsed_time(e1) * 1e-3
    cyc, ticks = (int(v) for v in clk.cpu())
    flops = 2.0 * 32 * 32 * 16 * 8 * iters * cus * (threads // 64)
    return flops / best / 1e12, cyc / ticks * 0.1  # the real-time counter runs at 100 MHz


def main():
    """Print the co-issue and mix tables: python -m draft_tree_verification_tv_amd.probe"""
    torch.cuda.init()
    for threads in (64, 512):
        for mode, name in enumerate(COISSUE_MODES):
            c = coissue(mode, threads)
            print(f"{name:30s} waves/workgroup={threads // 64}  cycles/iteration={c:7.1f}", flush=True)
    for threads in (512, 256):
        for lds_step, valu, name in MIX_CASES:
            tf, ghz = mix(lds_step, valu, threads)
            print(f"every CU, {threads // 256} wave(s)/SIMD: {name:40s} {tf:7.1f} TFLOP/s  clock {ghz:.3f} GHz",
                  flush=True)


if __name__ == "__main__":
    main()
