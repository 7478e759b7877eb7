"""Python binding of libtv (ctypes): argument marshalling only.

Every computation runs in the HIP kernels of ``libtv.so``; torch provides device memory
and the current stream. There is no fallback: if the library is missing or a call fails,
an exception is raised.

Function names match the C ABI in ``include/tv.h`` without the ``tv_`` prefix.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

from .build import LIB_PATH

TV_OK, TV_ERR_INVALID_ARG, TV_ERR_BAD_TREE, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE, TV_ERR_HIP = range(6)
TV_BF16, TV_F32 = 0, 1
MAX_NODES = 256
HEAD_DIM = 128

EXPORTS = ("tv_abi_version", "tv_status_string", "tv_validate_tree_host", "tv_tree_prep",
           "tv_tree_attn_workspace_size", "tv_tree_attn", "tv_argmax_workspace_size",
           "tv_argmax", "tv_accept", "tv_argmax_accept", "tv_sample_accept", "tv_kv_commit",
           "tv_kv_quantize_fp8", "tv_tree_attn_fp8", "tv_tree_attn_noalloc", "tv_kv_quantize_mx4",
           "tv_tree_attn_mx4")
NOALLOC_SCRATCH_BYTES = 32 << 20


class TVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None
_lock = threading.Lock()
_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float


def lib():
    """Load libtv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_tree_verification_tv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.tv_abi_version.restype = _i32
        L.tv_abi_version.argtypes = []
        L.tv_status_string.restype = ctypes.c_char_p
        L.tv_status_string.argtypes = [_i32]
        L.tv_validate_tree_host.restype = _i32
        L.tv_validate_tree_host.argtypes = [_vp, _i32]
        L.tv_tree_prep.restype = _i32
        L.tv_tree_prep.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp]
        L.tv_tree_attn_workspace_size.restype = _sz
        L.tv_tree_attn_workspace_size.argtypes = [_i32] * 6
        L.tv_tree_attn.restype = _i32
        L.tv_tree_attn.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, _i32,
                                   _f32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tv_argmax_workspace_size.restype = _sz
        L.tv_argmax_workspace_size.argtypes = [_i32, _i32]
        L.tv_argmax.restype = _i32
        L.tv_argmax.argtypes = [_vp, _i32, _i32, _i32, _i64, _vp, _vp, _sz, _vp]
        L.tv_accept.restype = _i32
        L.tv_accept.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.tv_argmax_accept.restype = _i32
        L.tv_argmax_accept.argtypes = [_vp, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                       _vp, _vp]
        L.tv_sample_accept.restype = _i32
        L.tv_sample_accept.argtypes = [_vp, _i32, _i32, _i32, _i64, _f32, ctypes.c_uint64, ctypes.c_uint64, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tv_kv_commit.restype = _i32
        L.tv_kv_commit.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
        L.tv_tree_attn_noalloc.restype = _i32
        L.tv_tree_attn_noalloc.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                           _vp, _vp, _vp, _vp]
        L.tv_tree_attn_fp8.restype = _i32
        L.tv_tree_attn_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                       _i32, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tv_kv_quantize_fp8.restype = _i32
        L.tv_kv_quantize_fp8.argtypes = [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _i64, _i64, _vp, _vp]
        L.tv_tree_attn_mx4.restype = _i32
        L.tv_tree_attn_mx4.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, _i32,
                                       _f32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tv_kv_quantize_mx4.restype = _i32
        L.tv_kv_quantize_mx4.argtypes = [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _i64, _i64, _vp, _vp]
        if L.tv_abi_version() != 1:
            raise RuntimeError("libtv ABI version mismatch")
        _lib = L
        return L


def _check(status: int, where: str):
    if status != TV_OK:
        raise TVError(status, where)


def _ptr(t):
    # The prototypes declare c_void_p, so ctypes takes the address as a plain int.
    return None if t is None else t.data_ptr()


# torch's raw current-stream query skips building a Stream object (a few µs per call,
# which matters for calls whose kernels take about 10 µs); the public route otherwise.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _need_buf(name, t, dtype, shape=None, min_numel=None, device=None):
    """A caller-supplied buffer the kernels index as a dense array: dtype, contiguity,
    device and either an exact shape or a minimum element count are checked before any
    launch, since a kernel would read or write past a smaller buffer."""
    _need_cuda(name, t, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")


def _opt_buf(name, t, dtype, shape=None, min_numel=None, device=None):
    if t is not None:
        _need_buf(name, t, dtype, shape=shape, min_numel=min_numel, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def _need_workspace(name, t, device):
    _need_cuda(name, t)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def abi_version() -> int:
    return lib().tv_abi_version()


def status_string(status: int) -> str:
    return lib().tv_status_string(status).decode()


def validate_tree_host(parent) -> int:
    """Host check of a parent array; returns a status code (0 = valid)."""
    p = torch.as_tensor(parent, dtype=torch.int32).contiguous().cpu()
    return lib().tv_validate_tree_host(ctypes.c_void_p(p.data_ptr()), p.numel())


def tree_prep(parent, dev_error=None, stream=None):
    """Ancestor bitmasks (int64 [N, 4], bit patterns of uint64 words) and depths int32 [N]."""
    _need_buf("parent", parent, torch.int32)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=parent.device)
    n = parent.numel()
    anc = torch.empty((n, 4), dtype=torch.int64, device=parent.device)
    depth = torch.empty(n, dtype=torch.int32, device=parent.device)
    _check(lib().tv_tree_prep(_ptr(parent), n, _ptr(anc), _ptr(depth), _ptr(dev_error), _stream(stream)),
           "tv_tree_prep")
    return anc, depth


def tree_attn_workspace_size(N, L, Hq, Hkv, D=HEAD_DIM, num_splits=0) -> int:
    return int(lib().tv_tree_attn_workspace_size(N, L, Hq, Hkv, D, num_splits))


def tree_attn(q, k, v, parent, L=None, scale=None, num_splits=0, out=None, lse=None,
              workspace=None, dev_error=None, stream=None):
    """Tree-masked attention. q bf16 [N, Hq, D]; k, v bf16 [>= L+N, Hkv, D] (last dim
    contiguous; any strides, e.g. a head-major [Hkv, T, D] cache viewed through
    permute(1, 0, 2)); parent int32 [N]. Returns out bf16 [N, Hq, D] (and fills ``lse``
    fp32 [N, Hq] when given)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k and v must share strides with a contiguous last dim")
    N, Hq, D = q.shape
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k and v must be on one device")
    Hkv = k.shape[1]
    if k.shape[1:] != (Hkv, D) or v.shape[1:] != (Hkv, D):
        raise ValueError(f"k and v must be [rows, Hkv, {D}] with one Hkv, got {tuple(k.shape)} and {tuple(v.shape)}")
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    if L is None:
        L = k.shape[0] - N
    if L < 0 or k.shape[0] < L + N or v.shape[0] < L + N:
        raise ValueError("k/v must hold L + N rows")
    _opt_buf("out", out, torch.bfloat16, shape=(N, Hq, D), device=dev)
    _opt_buf("lse", lse, torch.float32, shape=(N, Hq), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        ws_bytes = tree_attn_workspace_size(N, L, Hq, Hkv, D, num_splits)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _need_workspace("workspace", workspace, dev)
    _check(lib().tv_tree_attn(_ptr(q), _ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(parent), N, L, Hq,
                              Hkv, D, float(scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace),
                              _nbytes(workspace), _ptr(dev_error), _stream(stream)),
           "tv_tree_attn")
    return out


def tree_attn_noalloc(q, k, v, parent, L=None, scale=None, num_splits=0, out=None, lse=None, dev_error=None,
                      stream=None):
    """tree_attn through the allocation-free entry point: the split partials live in the
    library's static per-device buffer (NOALLOC_SCRATCH_BYTES), so the C call allocates
    nothing (pass ``out`` to allocate nothing here either). Calls that can overlap on one
    device race on that buffer."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, torch.bfloat16)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k and v must share strides with a contiguous last dim")
    N, Hq, D = q.shape
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k and v must be on one device")
    Hkv = k.shape[1]
    if k.shape[1:] != (Hkv, D) or v.shape[1:] != (Hkv, D):
        raise ValueError(f"k and v must be [rows, Hkv, {D}] with one Hkv, got {tuple(k.shape)} and {tuple(v.shape)}")
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    if L is None:
        L = k.shape[0] - N
    if L < 0 or k.shape[0] < L + N or v.shape[0] < L + N:
        raise ValueError("k/v must hold L + N rows")
    _opt_buf("out", out, torch.bfloat16, shape=(N, Hq, D), device=dev)
    _opt_buf("lse", lse, torch.float32, shape=(N, Hq), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    _check(lib().tv_tree_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(parent), N, L, Hq,
                                      Hkv, D, float(scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(dev_error),
                                      _stream(stream)),
           "tv_tree_attn_noalloc")
    return out


def tree_attn_fp8(q, k_codes, v_codes, k_exps, v_exps, parent, L=None, scale=None, num_splits=0, out=None,
                  lse=None, workspace=None, dev_error=None, stream=None):
    """Tree-masked attention over an FP8 cache: k_codes, v_codes uint8 [>= L+N, Hkv, D]
    (E4M3, last dim contiguous, shared strides); k_exps, v_exps int32 [>= L+N, Hkv]
    contiguous (row scales 2^e, as kv_quantize_fp8 writes them). Otherwise as tree_attn."""
    _need_cuda("q", q, torch.bfloat16)
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        _need_cuda(name, t, torch.uint8)
        if t.dim() != 3:
            raise ValueError(f"{name} must be 3-D")
    for name, t in (("k_exps", k_exps), ("v_exps", v_exps)):
        _need_cuda(name, t, torch.int32)
        if t.dim() != 2 or not t.is_contiguous() or t.shape[1] != k_codes.shape[1]:
            raise ValueError(f"{name} must be a contiguous [T, Hkv] tensor")
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [N, Hq, D] tensor")
    if k_codes.stride() != v_codes.stride() or k_codes.stride(2) != 1:
        raise ValueError("k_codes and v_codes must share strides with a contiguous last dim")
    N, Hq, D = q.shape
    dev = q.device
    for t in (k_codes, v_codes, k_exps, v_exps):
        if t.device != dev:
            raise ValueError("q, the codes and the exponents must be on one device")
    Hkv = k_codes.shape[1]
    if k_codes.shape[1:] != (Hkv, D) or v_codes.shape[1:] != (Hkv, D):
        raise ValueError(f"k_codes and v_codes must be [rows, Hkv, {D}] with one Hkv")
    if v_exps.shape[1] != Hkv:
        raise ValueError("v_exps must be a contiguous [T, Hkv] tensor")
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    if L is None:
        L = k_codes.shape[0] - N
    rows = L + N
    if L < 0 or min(k_codes.shape[0], v_codes.shape[0], k_exps.shape[0], v_exps.shape[0]) < rows:
        raise ValueError("codes and exponents must hold L + N rows")
    _opt_buf("out", out, torch.bfloat16, shape=(N, Hq, D), device=dev)
    _opt_buf("lse", lse, torch.float32, shape=(N, Hq), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        ws_bytes = tree_attn_workspace_size(N, L, Hq, Hkv, D, num_splits)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _need_workspace("workspace", workspace, dev)
    _check(lib().tv_tree_attn_fp8(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_exps), _ptr(v_exps),
                                  k_codes.stride(0), k_codes.stride(1), _ptr(parent), N, L, Hq, Hkv, D,
                                  float(scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace),
                                  _nbytes(workspace), _ptr(dev_error), _stream(stream)),
           "tv_tree_attn_fp8")
    return out


def tree_attn_mx4(q, k_codes, v_codes, k_exps, v_exps, parent, L=None, scale=None, num_splits=0, out=None,
                  lse=None, workspace=None, dev_error=None, stream=None):
    """Tree-masked attention over a 4-bit cache: k_codes, v_codes uint8 [>= L+N, Hkv, D / 2]
    (two E2M1 codes per byte, last dim contiguous, shared strides); k_exps, v_exps int8
    [>= L+N, Hkv, D / 32] contiguous (block scales 2^e, as kv_quantize_mx4 writes them).
    Otherwise as tree_attn."""
    _need_cuda("q", q, torch.bfloat16)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [N, Hq, D] tensor")
    N, Hq, D = q.shape
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        _need_cuda(name, t, torch.uint8)
        if t.dim() != 3:
            raise ValueError(f"{name} must be 3-D")
    if k_codes.stride() != v_codes.stride() or k_codes.stride(2) != 1:
        raise ValueError("k_codes and v_codes must share strides with a contiguous last dim")
    Hkv = k_codes.shape[1]
    if k_codes.shape[1:] != (Hkv, D // 2) or v_codes.shape[1:] != (Hkv, D // 2):
        raise ValueError(f"k_codes and v_codes must be [rows, Hkv, {D // 2}] with one Hkv")
    for name, t in (("k_exps", k_exps), ("v_exps", v_exps)):
        _need_cuda(name, t, torch.int8)
        if t.dim() != 3 or not t.is_contiguous() or t.shape[1:] != (Hkv, D // 32):
            raise ValueError(f"{name} must be a contiguous [T, Hkv, {D // 32}] tensor")
    dev = q.device
    for t in (k_codes, v_codes, k_exps, v_exps):
        if t.device != dev:
            raise ValueError("q, the codes and the exponents must be on one device")
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    if L is None:
        L = k_codes.shape[0] - N
    rows = L + N
    if L < 0 or min(k_codes.shape[0], v_codes.shape[0], k_exps.shape[0], v_exps.shape[0]) < rows:
        raise ValueError("codes and exponents must hold L + N rows")
    _opt_buf("out", out, torch.bfloat16, shape=(N, Hq, D), device=dev)
    _opt_buf("lse", lse, torch.float32, shape=(N, Hq), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        ws_bytes = tree_attn_workspace_size(N, L, Hq, Hkv, D, num_splits)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _need_workspace("workspace", workspace, dev)
    _check(lib().tv_tree_attn_mx4(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_exps), _ptr(v_exps),
                                  k_codes.stride(0), k_codes.stride(1), _ptr(parent), N, L, Hq, Hkv, D,
                                  float(scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace),
                                  _nbytes(workspace), _ptr(dev_error), _stream(stream)),
           "tv_tree_attn_mx4")
    return out


def _vocab(logits, V):
    """Row length to scan: the logits' second dimension unless a shorter V is given."""
    if V is None:
        return logits.shape[1]
    V = int(V)
    if V < 1 or V > logits.shape[1]:
        raise ValueError(f"V must lie in [1, {logits.shape[1]}] (the logits' row length), got {V}")
    return V


def _accept_out(out, N, dev):
    """The four acceptance outputs (accept_len [1], nodes [N], tokens [N], bonus [1] or
    None), allocated when ``out`` is None, checked otherwise."""
    if out is None:
        return (torch.empty(1, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev),
                torch.empty(N, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    if len(out) != 4:
        raise ValueError("out must be (accept_len, nodes, tokens, bonus)")
    ln, nodes, toks, bonus = out
    _need_buf("accept_len", ln, torch.int32, min_numel=1, device=dev)
    _need_buf("accept_nodes", nodes, torch.int32, min_numel=N, device=dev)
    _need_buf("accept_tokens", toks, torch.int32, min_numel=N, device=dev)
    _opt_buf("bonus", bonus, torch.int32, min_numel=1, device=dev)
    return out


def argmax_workspace_size(N, V) -> int:
    return int(lib().tv_argmax_workspace_size(N, V))


def argmax_workspace(N, V, device) -> torch.Tensor:
    """An argmax workspace (per-slice partial results; no initialisation needed)."""
    return torch.empty(max(argmax_workspace_size(N, V), 256), dtype=torch.uint8, device=device)


def argmax(logits, tok=None, workspace=None, V=None, stream=None):
    """Row argmax (lowest index on ties) of bf16 or fp32 logits [N, row_stride]."""
    _need_cuda("logits", logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bf16 or fp32")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with a contiguous last dim")
    N = logits.shape[0]
    V = _vocab(logits, V)
    dev = logits.device
    _opt_buf("tok", tok, torch.int32, shape=(N,), device=dev)
    if tok is None:
        tok = torch.empty(N, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = argmax_workspace(N, V, dev)
    _need_workspace("workspace", workspace, dev)
    dt = TV_F32 if logits.dtype == torch.float32 else TV_BF16
    _check(lib().tv_argmax(_ptr(logits), dt, N, V, logits.stride(0), _ptr(tok), _ptr(workspace),
                           _nbytes(workspace), _stream(stream)), "tv_argmax")
    return tok


def accept(parent, draft, tok, out=None, dev_error=None, stream=None):
    """Longest accepted path. Returns (accept_len [1], nodes [N], tokens [N], bonus [1])."""
    _need_buf("parent", parent, torch.int32)
    N = parent.numel()
    dev = parent.device
    _need_buf("draft", draft, torch.int32, shape=(N,), device=dev)
    _need_buf("tok", tok, torch.int32, shape=(N,), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    out = _accept_out(out, N, dev)
    ln, nodes, toks, bonus = out
    _check(lib().tv_accept(_ptr(parent), _ptr(draft), _ptr(tok), N, _ptr(ln), _ptr(nodes), _ptr(toks),
                           _ptr(bonus), _ptr(dev_error), _stream(stream)), "tv_accept")
    return ln, nodes, toks, bonus


def argmax_accept(logits, parent, draft, tok=None, out=None, workspace=None, V=None, dev_error=None,
                  stream=None):
    """Row argmax of the logits and the longest accepted path in one call.

    Returns (tok [N], (accept_len [1], nodes [N], tokens [N], bonus [1]))."""
    _need_cuda("logits", logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bf16 or fp32")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with a contiguous last dim")
    N = logits.shape[0]
    dev = logits.device
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    _need_buf("draft", draft, torch.int32, shape=(N,), device=dev)
    _opt_buf("tok", tok, torch.int32, shape=(N,), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    V = _vocab(logits, V)
    if tok is None:
        tok = torch.empty(N, dtype=torch.int32, device=dev)
    out = _accept_out(out, N, dev)
    if workspace is None:
        workspace = argmax_workspace(N, V, dev)
    _need_workspace("workspace", workspace, dev)
    ln, nodes, toks, bonus = out
    dt = TV_F32 if logits.dtype == torch.float32 else TV_BF16
    _check(lib().tv_argmax_accept(_ptr(logits), dt, N, V, logits.stride(0), _ptr(parent), _ptr(draft), _ptr(tok),
                                  _ptr(ln), _ptr(nodes), _ptr(toks), _ptr(bonus), _ptr(workspace),
                                  _nbytes(workspace), _ptr(dev_error), _stream(stream)), "tv_argmax_accept")
    return tok, out


def sample_accept(logits, parent, draft, temperature, seed, offset=0, tok=None, out=None, workspace=None, V=None,
                  dev_error=None, stream=None):
    """Sampled verification at temperature > 0: tok[i] is a sample from softmax(logits[i] / T)
    (Gumbel-max over Philox-4x32-10 keyed by seed, counter offset), then the longest
    accepted path. Returns (tok [N], (accept_len [1], nodes [N], tokens [N], bonus [1]))."""
    _need_cuda("logits", logits)
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bf16 or fp32")
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with a contiguous last dim")
    N = logits.shape[0]
    dev = logits.device
    _need_buf("parent", parent, torch.int32, shape=(N,), device=dev)
    _need_buf("draft", draft, torch.int32, shape=(N,), device=dev)
    _opt_buf("tok", tok, torch.int32, shape=(N,), device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    V = _vocab(logits, V)
    if tok is None:
        tok = torch.empty(N, dtype=torch.int32, device=dev)
    out = _accept_out(out, N, dev)
    if workspace is None:
        workspace = argmax_workspace(N, V, dev)
    _need_workspace("workspace", workspace, dev)
    ln, nodes, toks, bonus = out
    dt = TV_F32 if logits.dtype == torch.float32 else TV_BF16
    _check(lib().tv_sample_accept(_ptr(logits), dt, N, V, logits.stride(0), float(temperature), int(seed), int(offset),
                                  _ptr(parent), _ptr(draft), _ptr(tok), _ptr(ln), _ptr(nodes), _ptr(toks),
                                  _ptr(bonus), _ptr(workspace), _nbytes(workspace), _ptr(dev_error), _stream(stream)),
           "tv_sample_accept")
    return tok, out


def kv_commit(k, v, L, accept_len, accept_nodes, N=None, new_len=None, dev_error=None, stream=None):
    """Move the accepted nodes' K/V rows (cache rows L + node) to rows L + 0, 1, ... in path
    order, in place. k, v: [>= L+N, Hkv, D] 2-byte tensors sharing strides (last dim
    contiguous; rows disjoint in a token-major or a head-major layout); accept_len,
    accept_nodes: int32 device tensors as tv_accept writes them."""
    for name, t in (("k", k), ("v", v)):
        _need_cuda(name, t)
        if t.element_size() != 2 or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D tensor of 2-byte elements")
    if k.stride() != v.stride() or k.stride(2) != 1 or k.shape != v.shape:
        raise ValueError("k and v must share shape and strides with a contiguous last dim")
    dev = k.device
    if v.device != dev:
        raise ValueError("k and v must be on one device")
    _need_buf("accept_len", accept_len, torch.int32, min_numel=1, device=dev)
    _need_buf("accept_nodes", accept_nodes, torch.int32, device=dev)
    N = accept_nodes.numel() if N is None else int(N)
    if accept_nodes.numel() < N:
        raise ValueError(f"accept_nodes must hold at least N = {N} entries")
    _opt_buf("new_len", new_len, torch.int32, min_numel=1, device=dev)
    _opt_buf("dev_error", dev_error, torch.int32, min_numel=1, device=dev)
    if L < 0 or k.shape[0] < L + N:
        raise ValueError("k/v must hold L + N rows")
    _check(lib().tv_kv_commit(_ptr(k), _ptr(v), k.stride(0), k.stride(1), k.shape[1], k.shape[2], L, N,
                              _ptr(accept_len), _ptr(accept_nodes), _ptr(new_len), _ptr(dev_error), _stream(stream)),
           "tv_kv_commit")


def kv_quantize_fp8(x, codes=None, exps=None, stream=None):
    """Quantise a bf16 cache x [T, Hkv, D] (last dim contiguous) to E4M3 codes (uint8,
    same shape) and one power-of-two exponent per (token, head) row (int32 [T, Hkv]); the
    row dequantises to code * 2^exp. Returns (codes, exps). Codes allocated here are
    stored head-major (each head's rows side by side, returned as the [T, Hkv, D] view),
    the layout tree attention streams fastest; a caller's codes buffer may be token- or
    head-major."""
    _need_cuda("x", x, torch.bfloat16)
    if x.dim() != 3 or (x.numel() and x.stride(2) != 1):
        raise ValueError("x must be [T, Hkv, D] with a contiguous last dim")
    T, H, D = x.shape
    if codes is None:
        codes = torch.empty((H, T, D), dtype=torch.uint8, device=x.device).permute(1, 0, 2)
    if exps is None:
        exps = torch.empty((T, H), dtype=torch.int32, device=x.device)
    _need_cuda("codes", codes, torch.uint8)
    _need_cuda("exps", exps, torch.int32)
    if codes.shape != x.shape or tuple(exps.shape) != (T, H) or not exps.is_contiguous():
        raise ValueError("codes must be [T, Hkv, D] (contiguous last dim), exps a contiguous [T, Hkv]")
    if T == 0:
        return codes, exps
    if codes.stride(2) != 1:
        raise ValueError("codes must have a contiguous last dim")
    _check(lib().tv_kv_quantize_fp8(_ptr(x), x.stride(0), x.stride(1), T, H, D, _ptr(codes), codes.stride(0),
                                    codes.stride(1), _ptr(exps), _stream(stream)), "tv_kv_quantize_fp8")
    return codes, exps


def kv_quantize_mx4(x, codes=None, exps=None, stream=None):
    """Quantise a bf16 cache x [T, Hkv, D] (last dim contiguous) to 4-bit E2M1 codes, two
    per byte (uint8 [T, Hkv, D / 2]; value 2j in the low nibble of byte j), and one
    power-of-two exponent per 32-value block (int8 [T, Hkv, D / 32], contiguous); a block
    dequantises to code * 2^exp. Returns (codes, exps). Codes allocated here are stored
    head-major (each head's 64-byte rows side by side, so tree attention reads whole
    cache lines; returned as the [T, Hkv, D / 2] view); a caller's codes buffer may be
    token- or head-major."""
    _need_cuda("x", x, torch.bfloat16)
    if x.dim() != 3 or (x.numel() and x.stride(2) != 1):
        raise ValueError("x must be [T, Hkv, D] with a contiguous last dim")
    T, H, D = x.shape
    if D % 32:
        raise ValueError("D must be a multiple of 32")
    if codes is None:
        codes = torch.empty((H, T, D // 2), dtype=torch.uint8, device=x.device).permute(1, 0, 2)
    if exps is None:
        exps = torch.empty((T, H, D // 32), dtype=torch.int8, device=x.device)
    _need_cuda("codes", codes, torch.uint8)
    _need_cuda("exps", exps, torch.int8)
    if tuple(codes.shape) != (T, H, D // 2) or tuple(exps.shape) != (T, H, D // 32) or not exps.is_contiguous():
        raise ValueError("codes must be [T, Hkv, D / 2] (contiguous last dim), exps a contiguous [T, Hkv, D / 32]")
    for t in (codes, exps):
        if t.device != x.device:
            raise ValueError("x, codes and exps must be on one device")
    if T == 0:
        return codes, exps
    if codes.stride(2) != 1:
        raise ValueError("codes must have a contiguous last dim")
    _check(lib().tv_kv_quantize_mx4(_ptr(x), x.stride(0), x.stride(1), T, H, D, _ptr(codes), codes.stride(0),
                                    codes.stride(1), _ptr(exps), _stream(stream)), "tv_kv_quantize_mx4")
    return codes, exps


def verify(q, k, v, parent, logits, draft, L=None, scale=None, num_splits=0, attn_workspace=None,
           argmax_ws=None, stream=None):
    """One verify step: tree attention, row argmax and acceptance, all enqueued on one stream."""
    out = tree_attn(q, k, v, parent, L=L, scale=scale, num_splits=num_splits, workspace=attn_workspace,
                    stream=stream)
    tok = argmax(logits, workspace=argmax_ws, stream=stream)
    return out, tok, accept(parent, draft, tok, stream=stream)
