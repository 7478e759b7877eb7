"""GPU parity of the 4-bit (MX-style E2M1) key/value cache path against the CPU oracle.

The quantiser is integer work on exactly known numbers, so codes and block exponents must
match the oracle bit for bit.
"""

import numpy as np
import pytest
import torch

import draft_tree_verification_tv_amd as tv
import oracle
from tests.gpu_util import check_attention, dev_bf16, note
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
        ref_e = oracle.mx4_block_exponents(amax)
        assert np.array_equal(e.astype(np.int64), ref_e)


# ------------------------------------------------------------ 4-bit tree attention


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _dev_i8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).cuda()


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _mx4_attn_gpu(q_bits, kc, ke, vc, ve, parent, L, scale, num_splits=0, dev_error=None):
    N, Hq, _ = q_bits.shape
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_mx4(dev_bf16(q_bits), _dev_u8(kc), _dev_u8(vc), _dev_i8(ke), _dev_i8(ve),
                           _dev_i32(parent), L=L, scale=scale, num_splits=num_splits, lse=lse, dev_error=dev_error)
    torch.cuda.synchronize()
    return out, lse


def _mx4_ref(q_bits, kc, ke, vc, ve, parent, scale):
    return oracle.tree_attention(oracle.bf16_bits_to_f64(q_bits), oracle.dequantize_kv_mx4(kc, ke),
                                 oracle.dequantize_kv_mx4(vc, ve), parent, scale)


def _check_mx4_workload(w, label, num_splits=0):
    kc, ke = oracle.quantize_kv_mx4(w.k)
    vc, ve = oracle.quantize_kv_mx4(w.v)
    note(f"mx4 attention {label}: L={w.L} N={w.N} Hq={w.Hq} Hkv={w.Hkv} splits={num_splits}")
    out, lse = _mx4_attn_gpu(w.q, kc, ke, vc, ve, w.parent, w.L, w.scale, num_splits)
    ref, lref = _mx4_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    return check_attention(out, ref, lse, lref, label)


@pytest.mark.parametrize("name,trials", [("tiny_chain", 3), ("budget22", 3), ("branch_8k", 2)])
def test_mx4_attention_small_workloads(name, trials):
    for trial in range(trials):
        _check_mx4_workload(make(name, trial), f"{name}/{trial}")


MX4_EDGE = [
    ("L0_N1", dict(L=0, N=1, tree="chain", Hq=8, Hkv=2)),
    ("L1_N5", dict(L=1, N=5, tree="random16", Hq=4, Hkv=1)),
    ("L63_N1", dict(L=63, N=1, tree="chain", Hq=2, Hkv=2)),
    ("L65_N3_mha", dict(L=65, N=3, tree="random16", Hq=1, Hkv=1)),
    ("L130_N2", dict(L=130, N=2, tree="chain", Hq=8, Hkv=8)),
    ("L200_N60", dict(L=200, N=60, tree="random16", Hq=8, Hkv=2)),
    ("L1000_kary256_G1", dict(L=1000, N=256, tree="kary4", Hq=8, Hkv=8)),
    ("L300_kary256_G8", dict(L=300, N=256, tree="kary4", Hq=16, Hkv=2)),
    ("L777_G6_chain16", dict(L=777, N=16, tree="chain", Hq=24, Hkv=4)),
    ("L4097_N64", dict(L=4097, N=64, tree="random16", Hq=32, Hkv=8)),
    ("N3_G8_24rows", dict(L=500, N=3, tree="random16", Hq=8, Hkv=1)),
    ("N17_G1_17rows", dict(L=3000, N=17, tree="random16", Hq=4, Hkv=4)),
]


@pytest.mark.parametrize("label,ov", MX4_EDGE, ids=[e[0] for e in MX4_EDGE])
def test_mx4_attention_edge_shapes(label, ov):
    _check_mx4_workload(make("budget22", 7, **ov), label)


MX4_ROWS16 = [
    ("chain16_G1", dict(L=1000, N=16, tree="chain", Hq=8, Hkv=8)),
    ("N4_G4", dict(L=2500, N=4, tree="random16", Hq=16, Hkv=4)),
    ("N2_G8_L0", dict(L=0, N=2, tree="chain", Hq=8, Hkv=1)),
    ("N11_G1_L31", dict(L=31, N=11, tree="random16", Hq=3, Hkv=3)),
    ("N3_G5_L96", dict(L=96, N=3, tree="random16", Hq=10, Hkv=2)),
    ("N1_G8_peaky", dict(L=20000, N=1, tree="chain", Hq=8, Hkv=1, peaky=True)),
]


@pytest.mark.parametrize("label,ov", MX4_ROWS16, ids=[e[0] for e in MX4_ROWS16])
def test_mx4_attention_rows16(label, ov):
    w = make("budget22", 13, **ov)
    assert w.N * w.Hq // w.Hkv <= 16
    _check_mx4_workload(w, f"16-row {label}")


# T = 7022 keys, 110 tiles: 1, 2, 3, 7, 19, 37, 55 and 110 splits (both merge kernels),
# 88 rows through the 256-row kernel.
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 20, 40, 55, 1024])
def test_mx4_attention_forced_splits(splits):
    _check_mx4_workload(make("budget22", 11, L=7000, N=22), f"splits={splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [1, 4, 40, 1024])
def test_mx4_attention_decode_splits(splits):
    _check_mx4_workload(make("decode_1node", 3, L=5000), f"decode splits={splits}", num_splits=splits)


@pytest.mark.parametrize("L,splits", [(700, 12), (700, 6), (700, 4), (700, 3), (700, 2), (700, 1), (1200, 4)])
def test_mx4_attention_dense_short_splits(L, splits):
    _check_mx4_workload(make("branch_8k", 4, L=L), f"8x1 L={L} splits={splits}", num_splits=splits)


def test_mx4_attention_peaky_keys():
    _check_mx4_workload(make("max_256k", 1, L=20000), "peaky 20k")


def test_mx4_attention_own_key_only_is_exact():
    """Every node a root with L = 0: node i sees only its own key, so its output is its
    dequantised V row exactly (p = 1); V blocks span exponents from -125 to 125."""
    rng = np.random.default_rng(9)
    N, Hq, Hkv = 256, 8, 4
    parent = np.full(N, -1, np.int32)
    q = bf16_bits_from_f32(rng.standard_normal((N, Hq, 128)).astype(np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((N, Hkv, 128)).astype(np.float32))
    v32 = rng.standard_normal((N, Hkv, 4, 32)).astype(np.float32)
    shifts = rng.integers(-110, 110, size=(N, Hkv, 4, 1))
    shifts[0, 0, 0] = -122                    # block exponent at the low end
    shifts[1, 0, 3] = 124                     # and at the high end
    v64 = v32.astype(np.float64) / np.abs(v32).max(axis=3, keepdims=True) * np.exp2(shifts.astype(np.float64))
    v = bf16_bits_from_f32(v64.reshape(N, Hkv, 128).astype(np.float32))
    kc, ke = oracle.quantize_kv_mx4(k)
    vc, ve = oracle.quantize_kv_mx4(v)
    assert ve.min() <= -120 and ve.max() >= 120 and ve.min() >= -125 and ve.max() <= 125
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = _mx4_attn_gpu(q, kc, ke, vc, ve, parent, 0, 1 / np.sqrt(128), dev_error=err)
    assert err.item() == 0
    deq = oracle.dequantize_kv_mx4(vc, ve)
    expect = np.repeat(deq, Hq // Hkv, axis=1)
    got = out.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[0]}"
    _, lref = _mx4_ref(q, kc, ke, vc, ve, parent, 1 / np.sqrt(128))
    assert np.abs(lse.cpu().numpy() - lref).max() < 1e-3


def test_mx4_attention_strided_cache():
    """Codes as views into a larger cache (every other head of [T, 2*Hkv, D/2]) and
    exponents sized for a longer cache than L + N."""
    w = make("budget22", 3, L=1500)
    kc, ke = oracle.quantize_kv_mx4(w.k)
    vc, ve = oracle.quantize_kv_mx4(w.v)
    T = w.L + w.N
    big_k = np.zeros((T + 5, 2 * w.Hkv, 64), np.uint8)
    big_v = np.zeros_like(big_k)
    big_k[:T, ::2] = kc
    big_v[:T, ::2] = vc
    ke_big = np.zeros((T + 9, w.Hkv, 4), np.int8)
    ve_big = np.zeros_like(ke_big)
    ke_big[:T], ve_big[:T] = ke, ve
    out = tv.tree_attn_mx4(dev_bf16(w.q), _dev_u8(big_k)[:, ::2], _dev_u8(big_v)[:, ::2], _dev_i8(ke_big),
                           _dev_i8(ve_big), _dev_i32(w.parent), L=w.L, scale=w.scale)
    ref, _ = _mx4_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    check_attention(out, ref, label="mx4 strided")


@pytest.mark.parametrize("name", ["budget22", "decode_1node"])
def test_mx4_head_major_cache(name):
    """A head-major bf16 cache quantised on the GPU into head-major codes ([Hkv, T, D/2]
    viewed as [T, Hkv, D/2]); the exponents stay [T, Hkv, D/32]. Codes and exponents equal
    the oracle's, and attention over them matches the oracle on the dequantised cache."""
    w = make(name, 1)
    T = w.L + w.N
    note(f"mx4 head-major {name}")
    kc, ke = oracle.quantize_kv_mx4(w.k)
    vc, ve = oracle.quantize_kv_mx4(w.v)
    dev = []
    for bits in (w.k, w.v):
        x = dev_bf16(np.ascontiguousarray(bits.transpose(1, 0, 2))).permute(1, 0, 2)
        codes = torch.empty((w.Hkv, T, 64), dtype=torch.uint8, device="cuda").permute(1, 0, 2)
        dev.append(tv.kv_quantize_mx4(x, codes=codes))
    (kcd, ked), (vcd, ved) = dev
    torch.cuda.synchronize()
    assert kcd.stride() == (64, T * 64, 1)
    for got, want in ((kcd, kc), (vcd, vc)):
        assert np.array_equal(got.cpu().numpy(), want)
    for got, want in ((ked, ke), (ved, ve)):
        assert np.array_equal(got.cpu().numpy(), want)
    out = tv.tree_attn_mx4(dev_bf16(w.q), kcd, vcd, ked, ved, _dev_i32(w.parent), L=w.L, scale=w.scale)
    ref, _ = _mx4_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    check_attention(out, ref, label=f"mx4 head-major {name}")


# budget22 (88 rows) widens shared tiles; decode (8 rows) widens each wave's own blocks.
@pytest.mark.parametrize("name", ["budget22", "decode_1node"])
def test_mx4_attention_out_of_range_exponent_is_reported(name):
    w = make(name, 2, L=200)
    kc, ke = oracle.quantize_kv_mx4(w.k)
    vc, ve = oracle.quantize_kv_mx4(w.v)
    for bad_e in (126, -126, -128):
        ve2 = ve.copy()
        ve2[17, 0, 2] = bad_e
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        _mx4_attn_gpu(w.q, kc, ke, vc, ve2, w.parent, w.L, w.scale, dev_error=err)
        assert err.item() == 1, bad_e
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _mx4_attn_gpu(w.q, kc, ke, vc, ve, w.parent, w.L, w.scale, dev_error=err)
    assert err.item() == 0


def test_mx4_gpu_quantise_then_attend_full_size():
    """long_128k: the cache quantised on the GPU (checked code for code against the
    oracle's) feeds the 4-bit attention; reference: the oracle on the oracle's dequantised
    cache."""
    w = make("long_128k", 0, parts=("tree", "qkv"))
    note("mx4 full size: gpu quantise")
    kc_d, ke_d = tv.kv_quantize_mx4(dev_bf16(w.k))
    vc_d, ve_d = tv.kv_quantize_mx4(dev_bf16(w.v))
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_mx4(dev_bf16(w.q), kc_d, vc_d, ke_d, ve_d, _dev_i32(w.parent), L=w.L, scale=w.scale,
                           lse=lse)
    torch.cuda.synchronize()
    note("mx4 full size: oracle quantise")
    kc, ke = oracle.quantize_kv_mx4(w.k)
    vc, ve = oracle.quantize_kv_mx4(w.v)
    assert np.array_equal(kc_d.cpu().numpy(), kc) and np.array_equal(ke_d.cpu().numpy(), ke)
    assert np.array_equal(vc_d.cpu().numpy(), vc) and np.array_equal(ve_d.cpu().numpy(), ve)
    note("mx4 full size: oracle attention")
    ref, lref = _mx4_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    e, r = check_attention(out, ref, lse, lref, "mx4 long_128k")
    note(f"mx4 long_128k: max abs {e:.2e} row rel {r:.2e}")


@pytest.mark.parametrize("name", ["max_256k", "wide_tree", "decode_1node"])
def test_mx4_full_size_sampled_heads(name):
    """The other full-size workloads (the 4x2 kernel over 262160 keys, 2048 stacked rows in
    eight row tiles, the 16-row kernel over 32769 keys): the whole cache quantised and
    attended on the GPU; for the first and the last KV head the GPU's codes are checked
    against the oracle's quantisation of that head, and the attention of that head's query
    group against the oracle on the oracle's dequantised head."""
    w = make(name, 0, parts=("tree", "qkv"))
    G = w.Hq // w.Hkv
    note(f"mx4 {name} full size: gpu quantise and attend")
    kc_d, ke_d = tv.kv_quantize_mx4(dev_bf16(w.k))
    vc_d, ve_d = tv.kv_quantize_mx4(dev_bf16(w.v))
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_mx4(dev_bf16(w.q), kc_d, vc_d, ke_d, ve_d, _dev_i32(w.parent), L=w.L, scale=w.scale,
                           lse=lse)
    torch.cuda.synchronize()
    for h in (0, w.Hkv - 1):
        note(f"mx4 {name}: oracle, KV head {h}")
        kc, ke = oracle.quantize_kv_mx4(w.k[:, h:h + 1])
        vc, ve = oracle.quantize_kv_mx4(w.v[:, h:h + 1])
        assert np.array_equal(kc_d[:, h:h + 1].cpu().numpy(), kc) and np.array_equal(ke_d[:, h:h + 1].cpu().numpy(), ke)
        assert np.array_equal(vc_d[:, h:h + 1].cpu().numpy(), vc) and np.array_equal(ve_d[:, h:h + 1].cpu().numpy(), ve)
        ref, lref = _mx4_ref(w.q[:, h * G:(h + 1) * G], kc, ke, vc, ve, w.parent, w.scale)
        e, r = check_attention(out[:, h * G:(h + 1) * G], ref, lse[:, h * G:(h + 1) * G], lref,
                               f"mx4 {name} head {h}")
        note(f"mx4 {name} head {h}: max abs {e:.2e} row rel {r:.2e}")
