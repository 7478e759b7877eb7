"""GPU parity of the 4-bit (MX-style E2M1) key/value cache path against the CPU oracle.

The quantiser is integer work on exactly known numbers, so codes and block exponents must
match the oracle bit for bit.
"""

import numpy as np
import pytest
import torch

import draft_tree_verification_tv_amd as tv
import oracle
from tests.gpu_util import dev_bf16, note
from workloads import bf16_bits_from_f32, make

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def _quantize_dev(bits, src_pad_heads=0, codes_pad=0):
    """Run tv_kv_quantize_mx4 on bits [T, H, D] (optionally through strided views)."""
    T, H, D = bits.shape
    if src_pad_heads:
        big = np.zeros((T, H + src_pad_heads, D), np.uint16)
        big[:, :H] = bits
        x = dev_bf16(big)[:, :H]
    else:
        x = dev_bf16(bits)
    codes = None
    if codes_pad:
        codes = torch.full((T, H, D // 2 + codes_pad), 0xAB, dtype=torch.uint8, device="cuda")[:, :, :D // 2]
    c, e = tv.kv_quantize_mx4(x, codes=codes)
    torch.cuda.synchronize()
    return c.cpu().numpy(), e.cpu().numpy()


def _assert_quant_equal(bits, label, **kw):
    note(f"mx4 quantise {label}: shape {bits.shape}")
    c, e = _quantize_dev(bits, **kw)
    rc, re_ = oracle.quantize_kv_mx4(bits)
    assert np.array_equal(e, re_), f"{label}: exponents differ"
    bad = np.argwhere(c != rc)
    assert bad.size == 0, f"{label}: {len(bad)} code bytes differ, first {bad[0]} gpu {c[tuple(bad[0])]:#x} " \
                          f"oracle {rc[tuple(bad[0])]:#x}"


def _bits(x):
    """float64 values that are exact in bf16 -> bf16 bits (checked)."""
    b = bf16_bits_from_f32(np.asarray(x, np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(b), np.asarray(x, np.float64))
    return b


def _edge_rows():
    """Rows aimed at the rounding and scaling corners: every E2M1 midpoint and its
    neighbours (ties to even), the top of the range, signed zeros, values that round to
    zero, blocks whose maximum sits either side of 6 * 2^e, at many block scales."""
    D = 128
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    block = [6.0] + mids + [-m for m in mids] + [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.0, -0.0, 0.125,
                                                 -0.125, 0.2421875, 0.2578125, 5.03125, 4.96875, 3.0, 0.375]
    assert len(block) == 32
    block = np.array(block)
    rows = []
    for k in range(-60, 61, 5):
        r = np.concatenate([np.ldexp(block, k), np.ldexp(block[::-1], k + 1), np.ldexp(-block, k - 2),
                            np.ldexp(np.roll(block, 7), k)])
        rows.append(r)
    rows.append(np.zeros(D))                           # all-zero blocks: exponent 0, codes 0
    r = np.zeros(D)
    r[5] = -0.0
    r[40] = 6.25                                       # just above 6: exponent 1
    r[70] = 3.0                                        # exactly 6 / 2: exponent -1
    r[100] = 2.0 ** -130                               # bf16 subnormal block maximum: clamped e
    rows.append(r)
    r = np.zeros(D)
    r[0] = 2.0 ** 127 * 1.5                            # above 6 * 2^125: clamped e, saturation
    r[1] = -(2.0 ** 126)
    r[33] = 2.0 ** -126
    rows.append(r)
    return np.stack(rows)


def test_quantize_edge_rows():
    rows = _edge_rows()
    R = len(rows)
    bits = _bits(rows).reshape(R, 1, 128)
    _assert_quant_equal(bits, "edge rows H=1")
    bits2 = np.concatenate([bits, bits[::-1]], axis=1)   # [R, 2, 128]
    _assert_quant_equal(bits2, "edge rows H=2")


def test_quantize_random_rows_many_scales():
    rng = np.random.default_rng(2025)
    for T, H in ((1, 1), (3, 8), (257, 8), (1000, 2), (33, 5)):
        x = rng.standard_normal((T, H, 128)).astype(np.float32)
        x *= np.exp2(rng.integers(-40, 41, size=(T, H, 1))).astype(np.float32)
        x[rng.random((T, H, 128)) < 0.05] = 0
        _assert_quant_equal(bf16_bits_from_f32(x), f"random T={T} H={H}")


def test_quantize_every_bf16_value_once():
    """All finite bf16 values (both signs) in consecutive blocks: every rounding boundary
    of every block exponent."""
    mags = np.arange(0, 0x7F80, dtype=np.uint16)               # +0 .. largest finite
    allbits = np.concatenate([mags, mags | 0x8000])
    pad = (-len(allbits)) % 128
    allbits = np.concatenate([allbits, np.zeros(pad, np.uint16)])
    _assert_quant_equal(allbits.reshape(-1, 1, 128), "all bf16 values")


def test_quantize_strided_views_and_empty():
    rng = np.random.default_rng(5)
    x = bf16_bits_from_f32(rng.standard_normal((40, 3, 128)).astype(np.float32) * 3)
    _assert_quant_equal(x, "strided src", src_pad_heads=2)
    _assert_quant_equal(x, "strided codes", codes_pad=32)
    c, e = tv.kv_quantize_mx4(dev_bf16(np.zeros((0, 4, 128), np.uint16)))
    torch.cuda.synchronize()
    assert c.shape == (0, 4, 64) and e.shape == (0, 4, 4)


def test_quantize_full_size_cache_sampled_rows():
    """long_128k keys and values (131136 tokens x 8 heads): every block exponent, and the
    codes of 2048 sampled rows and the last rows, against the oracle."""
    w = make("long_128k", 0, parts=("qkv",))
    rng = np.random.default_rng(12)
    for name, arr in (("k", w.k), ("v", w.v)):
        note(f"mx4 quantise long_128k {name}")
        c, e = _quantize_dev(arr)
        ts = rng.integers(0, arr.shape[0], 2048)
        rc, re_ = oracle.quantize_kv_mx4(arr[ts])
        assert np.array_equal(c[ts], rc) and np.array_equal(e[ts], re_)
        rc, re_ = oracle.quantize_kv_mx4(arr[-3:])
        assert np.array_equal(c[-3:], rc) and np.array_equal(e[-3:], re_)
        # every exponent: block maxima of the whole cache, by the oracle's scalar rule
        amax = np.abs(oracle.bf16_bits_to_f64(arr).reshape(arr.shape[0], arr.shape[1], 4, 32)).max(axis=3)
        ref_e = np.vectorize(oracle.mx4_block_exponent, otypes=[np.int64])(amax)
        assert np.array_equal(e.astype(np.int64), ref_e)
