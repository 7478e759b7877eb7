"""Host-side checks of libtv that need no GPU: exports, versions, argument validation.

Every call here is rejected (or answered) by host code before any kernel is enqueued,
so the tests run on machines without a GPU. They need the built library.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import draft_tree_verification_tv_amd as tv
from draft_tree_verification_tv_amd.build import LIB_PATH

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="libtv.so not built")

FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(tv_\w+)\s*\(", src, re.M)))


def test_header_declares_the_documented_calls():
    names = declared_functions()
    for n in ("tv_tree_attn", "tv_argmax", "tv_accept", "tv_argmax_accept", "tv_sample_accept", "tv_kv_commit",
              "tv_kv_quantize_fp8", "tv_tree_attn_fp8", "tv_kv_quantize_mx4", "tv_tree_attn_mx4", "tv_tree_prep",
              "tv_abi_version", "tv_validate_tree_host"):
        assert n in names
    assert set(names) == set(tv.EXPORTS)


def test_every_declared_symbol_is_exported():
    raw = ctypes.CDLL(LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_version_and_strings():
    assert tv.abi_version() == 1
    for s in range(6):
        assert tv.status_string(s)
    assert tv.status_string(99) == "unknown status"


def test_validate_tree_host():
    assert tv.validate_tree_host([-1, 0, 1]) == 0
    assert tv.validate_tree_host([-1, -1, 0, 2]) == 0
    assert tv.validate_tree_host([0]) == 2
    assert tv.validate_tree_host([-1, 1]) == 2
    assert tv.validate_tree_host([-1, -2]) == 2
    assert tv.validate_tree_host(np.full(257, -1)) == 1
    L = tv.lib()
    assert L.tv_validate_tree_host(None, 3) == 1


def attn_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, st=1024, sh=128, parent=FAKE, N=4, L=100, Hq=8, Hkv=2, D=128,
             scale=0.088, splits=0, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 40, err=None, stream=None)
    a.update(kw)
    return tv.lib().tv_tree_attn(a["q"], a["k"], a["v"], a["st"], a["sh"], a["parent"], a["N"], a["L"],
                                 a["Hq"], a["Hkv"], a["D"], a["scale"], a["splits"], a["out"], a["lse"],
                                 a["ws"], a["ws_bytes"], a["err"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(parent=None), 1), (dict(out=None), 1),
    (dict(N=0), 1), (dict(N=257), 1), (dict(L=-1), 1), (dict(Hq=6, Hkv=4), 1), (dict(Hkv=0), 1),
    (dict(D=64), 3), (dict(D=256), 3), (dict(scale=0.0), 1), (dict(scale=-1.0), 1),
    (dict(scale=float("inf")), 1), (dict(st=1001), 1), (dict(sh=-8), 1),
    (dict(q=ctypes.c_void_p(0x10002)), 1), (dict(splits=-1), 1), (dict(splits=5000), 1),
    (dict(ws=None), 4), (dict(ws_bytes=16), 4), (dict(ws=ctypes.c_void_p(0x10008)), 4),
    (dict(st=1 << 20, L=1 << 12), 3),                          # one head's rows past 32-bit offsets
    (dict(st=1 << 62), 1), (dict(sh=1 << 60), 1),              # spans no allocation can have
])
def test_tree_attn_rejects(kw, status):
    assert attn_call(**kw) == status


def attn_fp8_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ek=FAKE, ev=FAKE, st=256, sh=128, parent=FAKE, N=4, L=100, Hq=8, Hkv=2,
             D=128, scale=0.088, splits=0, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 40, err=None, stream=None)
    a.update(kw)
    return tv.lib().tv_tree_attn_fp8(a["q"], a["k"], a["v"], a["ek"], a["ev"], a["st"], a["sh"], a["parent"],
                                     a["N"], a["L"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["splits"], a["out"],
                                     a["lse"], a["ws"], a["ws_bytes"], a["err"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(ek=None), 1), (dict(ev=None), 1),
    (dict(parent=None), 1), (dict(out=None), 1), (dict(N=0), 1), (dict(N=257), 1), (dict(L=-1), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(D=64), 3), (dict(scale=0.0), 1), (dict(st=200), 1), (dict(sh=8), 1),
    (dict(k=ctypes.c_void_p(0x10008)), 1), (dict(ek=ctypes.c_void_p(0x10002)), 1),
    (dict(ev=ctypes.c_void_p(0x10001)), 1), (dict(lse=ctypes.c_void_p(0x10002)), 1),
    (dict(st=1 << 20, L=1 << 12), 3), (dict(Hkv=1 << 20, Hq=1 << 20, L=1 << 12), 3), (dict(st=1 << 62), 1),
    (dict(sh=1 << 60), 1), (dict(ws=None), 4), (dict(ws_bytes=16), 4),
])
def test_tree_attn_fp8_rejects(kw, status):
    assert attn_fp8_call(**kw) == status


def attn_mx4_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ek=FAKE, ev=FAKE, st=128, sh=64, parent=FAKE, N=4, L=100, Hq=8, Hkv=2,
             D=128, scale=0.088, splits=0, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 40, err=None, stream=None)
    a.update(kw)
    return tv.lib().tv_tree_attn_mx4(a["q"], a["k"], a["v"], a["ek"], a["ev"], a["st"], a["sh"], a["parent"],
                                     a["N"], a["L"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["splits"], a["out"],
                                     a["lse"], a["ws"], a["ws_bytes"], a["err"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(ek=None), 1), (dict(ev=None), 1),
    (dict(parent=None), 1), (dict(out=None), 1), (dict(N=0), 1), (dict(N=257), 1), (dict(L=-1), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(D=64), 3), (dict(scale=0.0), 1), (dict(st=120), 1), (dict(sh=8), 1),
    (dict(k=ctypes.c_void_p(0x10008)), 1), (dict(v=ctypes.c_void_p(0x10004)), 1),
    (dict(ek=ctypes.c_void_p(0x10002)), 1), (dict(ev=ctypes.c_void_p(0x10001)), 1),
    (dict(lse=ctypes.c_void_p(0x10002)), 1),
    (dict(st=1 << 20, L=1 << 12), 3), (dict(Hkv=1 << 20, Hq=1 << 20, L=1 << 12), 3), (dict(st=1 << 62), 1),
    (dict(sh=1 << 60), 1), (dict(ws=None), 4), (dict(ws_bytes=16), 4),
])
def test_tree_attn_mx4_rejects(kw, status):
    assert attn_mx4_call(**kw) == status


def test_workspace_sizes():
    s = tv.tree_attn_workspace_size(64, 131072, 32, 8)
    assert s > 0 and s % 256 == 0
    assert tv.tree_attn_workspace_size(64, 131072, 32, 8, D=64) == 0
    assert tv.tree_attn_workspace_size(0, 10, 32, 8) == 0
    # a forced split count is honoured in the size (more splits, more partials)
    assert tv.tree_attn_workspace_size(64, 8192, 32, 8, num_splits=32) > \
        tv.tree_attn_workspace_size(64, 8192, 32, 8, num_splits=2)
    a = tv.argmax_workspace_size(64, 152064)
    assert a > 0 and a % 256 == 0
    assert tv.argmax_workspace_size(0, 10) == 0


@pytest.mark.parametrize("args,status", [
    ((None, 0, 4, 100, 100, FAKE, FAKE, 1 << 30), 1),
    ((FAKE, 0, 4, 100, 100, None, FAKE, 1 << 30), 1),
    ((FAKE, 2, 4, 100, 100, FAKE, FAKE, 1 << 30), 1),
    ((FAKE, 0, 0, 100, 100, FAKE, FAKE, 1 << 30), 1),
    ((FAKE, 0, 4, 0, 100, FAKE, FAKE, 1 << 30), 1),
    ((FAKE, 0, 4, 100, 99, FAKE, FAKE, 1 << 30), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, None, 1 << 30), 4),
    ((FAKE, 0, 4, 100, 100, FAKE, FAKE, 8), 4),
    ((FAKE, 0, 4, 100, 1 << 60, FAKE, FAKE, 1 << 30), 1),     # rows no allocation can hold
])
def test_argmax_rejects(args, status):
    assert tv.lib().tv_argmax(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE, 4, FAKE, FAKE, FAKE), 1),
    ((FAKE, None, FAKE, 4, FAKE, FAKE, FAKE), 1),
    ((FAKE, FAKE, None, 4, FAKE, FAKE, FAKE), 1),
    ((FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE), 1),
    ((FAKE, FAKE, FAKE, 257, FAKE, FAKE, FAKE), 1),
    ((FAKE, FAKE, FAKE, 4, None, FAKE, FAKE), 1),
    ((FAKE, FAKE, FAKE, 4, FAKE, None, FAKE), 1),
    ((FAKE, FAKE, FAKE, 4, FAKE, FAKE, None), 1),
])
def test_accept_rejects(args, status):
    assert tv.lib().tv_accept(*args, None, None, None) == status


# tv_argmax_accept(logits, dtype, N, V, row_stride, parent, draft, tok, len, nodes, tokens,
#                  bonus, workspace, workspace_bytes, dev_error, stream)
@pytest.mark.parametrize("args,status", [
    ((None, 0, 4, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, None, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, FAKE, None, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, FAKE, FAKE, None, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, FAKE, FAKE, FAKE, None, FAKE), 1),
    ((FAKE, 0, 4, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, None), 1),
    ((FAKE, 0, 257, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 0, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 3, 4, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
    ((FAKE, 0, 4, 100, 99, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1),
])
def test_argmax_accept_rejects(args, status):
    assert tv.lib().tv_argmax_accept(*args, None, FAKE, 1 << 30, None, None) == status


def test_argmax_accept_workspace_checks():
    L = tv.lib()
    args = (FAKE, 0, 4, 100, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert L.tv_argmax_accept(*args, None, 1 << 30, None, None) == 4
    assert L.tv_argmax_accept(*args, FAKE, 8, None, None) == 4
    assert L.tv_argmax_accept(*args, ctypes.c_void_p(0x10008), 1 << 30, None, None) == 4


# tv_kv_commit(k, v, stride_t, stride_h, Hkv, D, L, N, accept_len, accept_nodes, new_len, dev_error, stream)
@pytest.mark.parametrize("args,status", [
    ((None, FAKE, 1024, 128, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, None, 1024, 128, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 8, 128, 100, 16, None, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 8, 128, 100, 16, FAKE, None), 1),
    ((FAKE, FAKE, 1024, 128, 8, 128, 100, 0, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 8, 128, 100, 257, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 8, 128, -1, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 0, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 128, 8, 12, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1020, 128, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 124, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((ctypes.c_void_p(0x10008), FAKE, 1024, 128, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1024, 256, 8, 128, 100, 16, FAKE, FAKE), 1),    # heads 4-7 overlap the next token
    ((FAKE, FAKE, 128, 14000, 8, 128, 100, 16, FAKE, FAKE), 1),   # head-major, heads overlap
    ((FAKE, FAKE, -1024, 128, 8, 128, 100, 16, FAKE, FAKE), 1),
    ((FAKE, FAKE, 1 << 62, 1 << 61, 8, 128, 100, 16, FAKE, FAKE), 1),  # (Hkv - 1) * stride_h past 2^63
])
def test_kv_commit_rejects(args, status):
    assert tv.lib().tv_kv_commit(*args, None, None, None) == status


# 3.5e-39: 1/T fits in float32 but log2(e)/T, the factor the kernel applies, does not.
@pytest.mark.parametrize("temp", [0.0, -1.0, float("inf"), float("nan"), 1e-45, 3.5e-39])
def test_sample_accept_rejects_bad_temperature(temp):
    L = tv.lib()
    assert L.tv_sample_accept(FAKE, 0, 4, 100, 100, temp, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                              1 << 30, None, None) == 1


def test_sample_accept_rejects_args():
    L = tv.lib()
    ok = [FAKE, 0, 4, 100, 100, 1.0, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None, None]
    for i in (0, 8, 9, 10, 11, 12, 13):
        bad = list(ok)
        bad[i] = None
        assert L.tv_sample_accept(*bad) == 1, i
    bad = list(ok)
    bad[2] = 257
    assert L.tv_sample_accept(*bad) == 1
    bad = list(ok)
    bad[16] = 8
    assert L.tv_sample_accept(*bad) == 4


def test_tree_prep_rejects():
    L = tv.lib()
    assert L.tv_tree_prep(None, 4, FAKE, FAKE, None, None) == 1
    assert L.tv_tree_prep(FAKE, 0, FAKE, FAKE, None, None) == 1
    assert L.tv_tree_prep(FAKE, 300, FAKE, FAKE, None, None) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        tv.argmax(torch.zeros(2, 8))


# tv_kv_quantize_fp8(src, sst, ssh, T, Hkv, D, codes, cst, csh, exps, stream)
@pytest.mark.parametrize("args,status", [
    ((None, 1024, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, None, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1024, 128, None), 1),
    ((FAKE, 1024, 128, -1, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 0, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 64, FAKE, 1024, 128, FAKE), 3),
    ((FAKE, 1022, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 126, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1024, 127, FAKE), 1),
    ((FAKE, 1028, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1024, 132, FAKE), 1),
    ((ctypes.c_void_p(0x10008), 1024, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, ctypes.c_void_p(0x10004), 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1023, 128, FAKE), 1),
    ((ctypes.c_void_p(0x10002), 1024, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, ctypes.c_void_p(0x10001), 1024, 128, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1024, 128, ctypes.c_void_p(0x10002)), 1),
    ((FAKE, 1 << 40, 128, 1 << 30, 8, 128, FAKE, 1 << 40, 128, FAKE), 1),
    ((FAKE, 1024, 128, 0, 8, 128, FAKE, 1024, 128, FAKE), 0),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 1024, 256, FAKE), 1),   # code heads overlap the next token
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 128, 1024, FAKE), 1),   # head-major, heads overlap
    ((FAKE, -8, 128, 10, 8, 128, FAKE, 1024, 128, FAKE), 1),
])
def test_kv_quantize_rejects(args, status):
    assert tv.lib().tv_kv_quantize_fp8(*args, None) == status


# tv_kv_quantize_mx4(src, sst, ssh, T, Hkv, D, codes, cst, csh, exps, stream): codes rows
# of D / 2 bytes, strides multiples of 16, 16-byte aligned codes; exps int8 (any alignment)
@pytest.mark.parametrize("args,status", [
    ((None, 1024, 128, 10, 8, 128, FAKE, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, None, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 512, 64, None), 1),
    ((FAKE, 1024, 128, -1, 8, 128, FAKE, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 0, 128, FAKE, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 64, FAKE, 512, 64, FAKE), 3),
    ((FAKE, 1022, 128, 10, 8, 128, FAKE, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 496, 64, FAKE), 1),     # codes row stride below 8 heads
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 512, 48, FAKE), 1),     # head stride below D / 2
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 520, 64, FAKE), 1),     # not a multiple of 16
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 512, 72, FAKE), 1),
    ((ctypes.c_void_p(0x10008), 1024, 128, 10, 8, 128, FAKE, 512, 64, FAKE), 1),
    ((FAKE, 1024, 128, 10, 8, 128, ctypes.c_void_p(0x10008), 512, 64, FAKE), 1),
    ((FAKE, 1 << 40, 128, 1 << 30, 8, 128, FAKE, 1 << 40, 64, FAKE), 1),
    ((FAKE, 1024, 128, 0, 8, 128, FAKE, 512, 64, ctypes.c_void_p(0x10003)), 0),
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 512, 128, FAKE), 1),    # code heads overlap the next token
    ((FAKE, 1024, 128, 10, 8, 128, FAKE, 64, 512, FAKE), 1),     # head-major, heads overlap
])
def test_kv_quantize_mx4_rejects(args, status):
    assert tv.lib().tv_kv_quantize_mx4(*args, None) == status


PROBE_HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tv_probe.h")


def test_probe_library_exports_and_validation():
    """The benchmark's probe library exports what include/tv_probe.h declares and refuses
    invalid arguments on the host (status 1) before any launch."""
    from draft_tree_verification_tv_amd import probe
    from draft_tree_verification_tv_amd.build import PROBE_LIB_PATH

    if not os.path.exists(PROBE_LIB_PATH):
        pytest.skip("libtv_probe.so not built")
    src = open(PROBE_HEADER).read()
    names = sorted(set(re.findall(r"^\s*\w+\s+(tv_probe_\w+)\s*\(", src, re.M)))
    assert set(names) == set(probe.EXPORTS)
    raw = ctypes.CDLL(PROBE_LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    L = probe.lib()
    sink = FAKE
    assert L.tv_probe_stream_read(None, 16, 256, 2048, 8, 4, sink, None) == 1          # null buffer
    assert L.tv_probe_stream_read(FAKE, 16, 384, 4096, 8, 4, sink, None) == 1          # not a power of two
    assert L.tv_probe_stream_read(FAKE, 16, 256, 1024, 8, 4, sink, None) == 1          # stride below 8 columns
    assert L.tv_probe_stream_read(ctypes.c_void_p(0x10008), 16, 256, 2048, 8, 4, sink, None) == 1  # misaligned
    assert L.tv_probe_stream_read(FAKE, 0, 256, 2048, 8, 4, sink, None) == 1           # no rows
    assert L.tv_probe_clock(None, 100, None) == 1
    assert L.tv_probe_clock(FAKE, 0, None) == 1
    assert L.tv_probe_coissue(0, 64, 10, None, FAKE, FAKE, None) == 1    # null input
    assert L.tv_probe_coissue(0, 100, 10, FAKE, FAKE, FAKE, None) == 1   # not 64, 256 or 512 threads
    assert L.tv_probe_coissue(0, 64, 0, FAKE, FAKE, FAKE, None) == 1     # no iterations
    assert L.tv_probe_coissue(6, 64, 10, FAKE, FAKE, FAKE, None) == 1    # no such mode
    assert L.tv_probe_mix(0, 0, 512, 256, 10, None, FAKE, FAKE, None) == 1   # null input
    assert L.tv_probe_mix(8, 0, 512, 256, 10, FAKE, FAKE, FAKE, None) == 1   # no such LDS step
    assert L.tv_probe_mix(-1, 0, 512, 256, 10, FAKE, FAKE, FAKE, None) == 1  # no such LDS step
    assert L.tv_probe_mix(0, 2, 512, 256, 10, FAKE, FAKE, FAKE, None) == 1   # valu not 0 or 1
    assert L.tv_probe_mix(0, 0, 64, 256, 10, FAKE, FAKE, FAKE, None) == 1    # not 256 or 512 threads
    assert L.tv_probe_mix(0, 0, 512, 0, 10, FAKE, FAKE, FAKE, None) == 1     # no workgroups
    assert L.tv_probe_mix(0, 0, 512, 256, 0, FAKE, FAKE, FAKE, None) == 1    # no iterations


def noalloc_call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, st=1024, sh=128, parent=FAKE, N=4, L=100, Hq=8, Hkv=2, D=128,
             scale=0.088, splits=0, out=FAKE, lse=None, err=None, stream=None)
    a.update(kw)
    return tv.lib().tv_tree_attn_noalloc(a["q"], a["k"], a["v"], a["st"], a["sh"], a["parent"], a["N"], a["L"],
                                         a["Hq"], a["Hkv"], a["D"], a["scale"], a["splits"], a["out"], a["lse"],
                                         a["err"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(N=0), 1), (dict(D=64), 3), (dict(scale=0.0), 1),
    (dict(st=1001), 1), (dict(q=ctypes.c_void_p(0x10002)), 1),
    # partials beyond the static buffer (8 KV heads x 1024 splits at 128K keys): refused
    (dict(L=131072, st=1024, Hq=32, Hkv=8, splits=1024), 4),
])
def test_tree_attn_noalloc_rejects(kw, status):
    assert noalloc_call(**kw) == status
