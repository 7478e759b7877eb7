"""Pins of the oracle's FP8 (E4M3) key/value quantisation.

Checked against the format's definition, not the oracle's own formulas: every one of the
256 codes decoded from sign/exponent/mantissa fields by hand; encode(decode(c)) == c for
every finite code; nearest-value rounding with ties to even checked by brute force on
midpoints and random values; the per-row power-of-two scale is the smallest that fits;
dequantised values are exactly representable in bfloat16.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32


def _hand_decode(c):
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9               # subnormal: m/8 * 2^(1-7)
    return s * (8 + m) * 2.0 ** (e - 10)       # (1 + m/8) * 2^(e-7)


def test_decode_every_code():
    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        want = _hand_decode(c)
        assert (np.isnan(got[c]) and np.isnan(want)) or got[c] == want, c
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0


def test_encode_decode_identity_on_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals)
    # +0 and -0 both encode to 0x00 (the sign of zero is not kept)
    keep = codes != 0x80
    assert np.array_equal(back[keep], codes[keep])
    assert back[~keep].tolist() == [0]


def test_rounding_nearest_ties_to_even_by_brute_force():
    finite = np.array([c for c in range(0x7F)], dtype=np.uint8)
    vals = oracle.e4m3_decode(finite)
    # midpoints go to the code with an even mantissa (lowest bit 0)
    mids = (vals[:-1] + vals[1:]) / 2
    enc = oracle.e4m3_encode(mids)
    for i, c in enumerate(enc):
        assert c in (finite[i], finite[i + 1])
        assert c % 2 == 0, (mids[i], c)
    rng = np.random.default_rng(0)
    x = rng.uniform(-448, 448, 20000) * 2.0 ** rng.integers(-12, 1, 20000)
    x = np.clip(x, -448, 448)
    enc = oracle.e4m3_encode(x)
    dec = oracle.e4m3_decode(enc)
    allv = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    allv = allv[np.isfinite(allv)]
    best = np.abs(x[:, None] - allv[None, :]).min(axis=1)
    assert np.array_equal(np.abs(x - dec), best)           # always a nearest value
    normal = np.abs(x) >= 2.0 ** -6
    assert (np.abs(dec - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4).all()


def test_scale_is_smallest_power_of_two_that_fits():
    rng = np.random.default_rng(1)
    for a in np.concatenate([[448.0, 448.0 + 1e-9, 1.0, 3.5, 2.0 ** -30, 1e30],
                             rng.uniform(0, 1000, 200) * 2.0 ** rng.integers(-20, 20, 200)]):
        e = oracle.row_scale_exponent(float(a))
        assert a <= 448.0 * 2.0 ** e
        assert a > 448.0 * 2.0 ** (e - 1)
    assert oracle.row_scale_exponent(0.0) == 0


def test_quantize_rows_and_bf16_exact_dequant():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 3, 128)).astype(np.float32)
    x[7, 1] = 0.0
    x[9, 2] *= 1e4
    x[11, 0] *= 1e-6
    bits = bf16_bits_from_f32(x)
    codes, exps = oracle.quantize_kv(bits)
    deq = oracle.dequantize_kv(codes, exps)
    xf = oracle.bf16_bits_to_f64(bits)
    assert exps[7, 1] == 0 and (codes[7, 1] == 0).all()
    amax = np.abs(xf).max(axis=2)
    assert (np.abs(xf) <= 448.0 * 2.0 ** exps[..., None]).all()
    assert (amax[amax > 0] > 448.0 * 2.0 ** (exps[amax > 0] - 1)).all()
    # error per element: half a code step at that element's magnitude (relative 2^-4 for
    # normal codes, absolute 2^-10 * 2^e below the normal range)
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** (exps[..., None] - 10))
    assert (err <= bound).all()
    # exactly representable in bf16: a round trip through torch's bfloat16 is the identity
    t = torch.from_numpy(deq).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(t, deq)


def test_mutant_round_half_up_is_caught():
    finite = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2

    def half_up(v):
        return np.searchsorted(finite, v, side="right").astype(np.uint8)   # always the upper code
    assert not np.array_equal(half_up(mids), oracle.e4m3_encode(mids))


def test_row_exponents_vectorised_equal_scalar_and_chunking_is_invisible():
    rng = np.random.default_rng(4)
    a = np.concatenate([[0.0, 448.0, 449.0, 224.0, 2.0 ** -130, 3e38],
                        rng.uniform(0, 1000, 500) * 2.0 ** rng.integers(-60, 60, 500)])
    vec = oracle.kvquant.row_scale_exponents(a)
    assert vec.tolist() == [oracle.row_scale_exponent(float(x)) for x in a]
    x = rng.standard_normal((37, 2, 128)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (37, 2, 1)))
    bits = bf16_bits_from_f32(x.astype(np.float32))
    c1, e1 = oracle.quantize_kv(bits)
    c2, e2 = oracle.quantize_kv(bits, chunk_rows=5)
    assert np.array_equal(c1, c2) and np.array_equal(e1, e2)
    # a row at a time through the scalar definitions
    xf = oracle.bf16_bits_to_f64(bits)
    for t in (0, 17, 36):
        for h in range(2):
            e = oracle.row_scale_exponent(float(np.abs(xf[t, h]).max()))
            assert e1[t, h] == e
            assert np.array_equal(c1[t, h], oracle.e4m3_encode(np.ldexp(xf[t, h], -e)))
