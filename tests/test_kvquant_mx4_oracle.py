"""Pins of the oracle's 4-bit (MX-style E2M1) key/value quantisation.

Checked against the format's definition, not the oracle's own formulas: the 16 E2M1 code
values as the OCP Microscaling specification tabulates them; encode(decode(c)) == c;
nearest-value rounding with ties to even at every midpoint and by brute force on random
values; saturation; the per-block power-of-two scale is the smallest that fits (and its
clamp); the packing order; dequantised values exact in bfloat16; the whole quantiser equal
to a per-element scalar statement of the same definition.
"""

import math

import numpy as np
import torch

import oracle
from workloads import bf16_bits_from_f32

# OCP Microscaling Formats v1.0, FP4 (E2M1) element values for codes 0b0000 .. 0b0111; the
# sign bit 0b1000 negates them.
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_decode_every_code_matches_the_spec_table():
    got = oracle.e2m1_decode(np.arange(16))
    for c in range(16):
        want = E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0)
        assert got[c] == want, c
    assert got.max() == 6.0 and got.min() == -6.0


def test_encode_decode_identity():
    codes = np.array([c for c in range(16) if c != 8], dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_encode(oracle.e2m1_decode(codes)), codes)
    assert oracle.e2m1_encode(np.array([-0.0]))[0] == 0      # the sign of zero is not kept


def _midpoints_ok(encode):
    """True when encode sends every E2M1 midpoint (and its negative) to the neighbour whose
    mantissa bit is 0."""
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for y, c in cases:
        if encode(np.array([y]))[0] != c or encode(np.array([-y]))[0] != (c | 8 if c else 0):
            return False
    return True


def test_midpoints_round_to_the_even_code():
    assert _midpoints_ok(oracle.e2m1_encode)
    for y in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        lo, hi = np.nextafter(y, 0.0), np.nextafter(y, 10.0)
        v_lo = oracle.e2m1_decode(oracle.e2m1_encode(np.array([lo])))[0]
        v_hi = oracle.e2m1_decode(oracle.e2m1_encode(np.array([hi])))[0]
        assert v_lo < y < v_hi, y                               # off the tie: the nearer side


def test_nearest_value_by_brute_force_and_saturation():
    rng = np.random.default_rng(3)
    y = rng.uniform(-7.5, 7.5, 20000)
    got = oracle.e2m1_decode(oracle.e2m1_encode(y))
    grid = np.array(sorted(set(E2M1_SPEC + [-v for v in E2M1_SPEC])))
    clipped = np.clip(y, -6.0, 6.0)
    best = np.abs(grid[None, :] - clipped[:, None]).min(axis=1)
    assert np.array_equal(np.abs(got - clipped), best)
    assert np.all(got[y > 6] == 6.0) and np.all(got[y < -6] == -6.0)


def test_block_exponent_is_the_smallest_that_fits_and_clamps():
    rng = np.random.default_rng(4)
    amax = np.exp2(rng.uniform(-120, 120, 5000)) * rng.uniform(0.5, 1.0, 5000)
    amax = np.concatenate([amax, [6.0, 3.0, 12.0, 6.0000001, 2.0 ** -200, 2.0 ** 127 * 1.9]])
    for a in amax:
        e = oracle.mx4_block_exponent(float(a))
        if -125 < e < 125:
            assert a <= 6.0 * 2.0 ** e and a > 6.0 * 2.0 ** (e - 1), a
    assert oracle.mx4_block_exponent(0.0) == 0
    assert oracle.mx4_block_exponent(6.0) == 0 and oracle.mx4_block_exponent(3.0) == -1
    assert oracle.mx4_block_exponent(2.0 ** -200) == -125
    assert oracle.mx4_block_exponent(2.0 ** 127 * 1.9) == 125


def _bits(x):
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def test_packing_order_and_block_scales():
    x = np.zeros((1, 1, 128), dtype=np.float32)
    x[0, 0, 0], x[0, 0, 1] = 1.0, -6.0           # block 0: amax 6 -> e = 0
    x[0, 0, 32:64] = 0.5                         # block 1: amax 0.5 -> e = -3 (6/8 fits, 6/16 not)
    x[0, 0, 100] = 96.0                          # block 3: amax 96 -> e = 4
    codes, exps = oracle.quantize_kv_mx4(_bits(x))
    assert codes.shape == (1, 1, 64) and exps.shape == (1, 1, 4)
    assert exps[0, 0].tolist() == [0, -3, 0, 4]
    assert codes[0, 0, 0] == (0x2 | (0xF << 4))  # element 0 (1.0) low nibble, element 1 (-6) high
    assert codes[0, 0, 16] == (0x6 | (0x6 << 4))  # 0.5 / 2^-3 = 4: code 6 in both nibbles
    assert oracle.dequantize_kv_mx4(codes, exps)[0, 0, 100] == 96.0


def test_quantise_rows_exact_in_bf16_and_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 3, 128)) * np.exp2(rng.integers(-30, 30, (40, 3, 1)))).astype(np.float32)
    x[5, 1, :32] = 0.0                           # an all-zero block
    bits = _bits(x)
    codes, exps = oracle.quantize_kv_mx4(bits)
    deq = oracle.dequantize_kv_mx4(codes, exps)
    # exact in bf16: widening to float32 and rounding to bf16 gives the same value back
    t = torch.from_numpy(deq.astype(np.float32))
    assert np.array_equal(t.to(torch.bfloat16).float().numpy().astype(np.float64), deq)
    xe = oracle.bf16_bits_to_f64(bits).reshape(40, 3, 4, 32)
    e = exps.astype(np.int64)[..., None]
    err = np.abs(xe - deq.reshape(40, 3, 4, 32))
    assert np.all(err <= np.ldexp(1.0, e))      # at most half the widest step (4 -> 6)
    assert np.all(np.abs(deq).reshape(40, 3, 4, 32) <= np.ldexp(6.0, e))
    assert exps[5, 1, 0] == 0 and np.all(deq[5, 1, :32] == 0.0)


def test_quantiser_equals_a_scalar_statement():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((3, 2, 128)) * 3).astype(np.float32)
    bits = _bits(x)
    codes, exps = oracle.quantize_kv_mx4(bits)
    xs = oracle.bf16_bits_to_f64(bits)
    for t in range(3):
        for h in range(2):
            for b in range(4):
                blk = xs[t, h, 32 * b:32 * b + 32]
                amax = max(abs(float(v)) for v in blk)
                e = oracle.mx4_block_exponent(amax)
                assert exps[t, h, b] == e
                for i in range(32):
                    y = math.ldexp(float(blk[i]), -e)
                    # nearest spec value, ties to the even code, by a plain scan
                    best, code = None, 0
                    for c in range(8):
                        d = abs(abs(y) - E2M1_SPEC[c])
                        if best is None or d < best or (d == best and c % 2 == 0):
                            best, code = d, c
                    if y < 0 and code:
                        code |= 8
                    d = 32 * b + i
                    got = (codes[t, h, d // 2] >> (4 * (d % 2))) & 0xF
                    assert got == code, (t, h, d)


def test_mutant_round_half_away_is_caught():
    """An encoder that rounds ties away from zero (a plausible slip) fails the midpoint pin."""
    def encode_half_away(y):
        y = np.asarray(y, dtype=np.float64)
        a = np.minimum(np.abs(y), 6.0)
        vals = np.array(E2M1_SPEC)
        d = np.abs(vals[None, :] - a[:, None])
        idx = np.where(np.isclose(d, d.min(axis=1, keepdims=True)), np.arange(8)[None, :], -1).max(axis=1)
        sign = (y < 0) & (idx != 0)
        return (idx | np.where(sign, 8, 0)).astype(np.uint8)
    assert not _midpoints_ok(encode_half_away)
    assert _midpoints_ok(oracle.e2m1_encode)


def test_block_exponents_vectorised_equal_scalar():
    rng = np.random.default_rng(7)
    amax = np.exp2(rng.uniform(-140, 130, 20000)) * rng.uniform(0.5, 1.0, 20000)
    amax = np.concatenate([amax, [0.0, 6.0, 3.0, 0.75, 0.7500001, 2.0 ** -140, 2.0 ** 127 * 1.99]])
    want = np.array([oracle.mx4_block_exponent(float(a)) for a in amax])
    assert np.array_equal(oracle.mx4_block_exponents(amax), want)
