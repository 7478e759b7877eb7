"""GPU parity of the FP8 (E4M3) key/value cache path against the CPU oracle.

The quantiser is integer work on exactly known numbers, so codes and exponents must match
the oracle bit for bit; the FP8 attention must match the oracle's attention over the
dequantised cache (which is exact in bf16) to the same tolerance as the bf16 path.
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
    """Run tv_kv_quantize_fp8 on bits [T, H, D] (optionally through strided views)."""
    T, H, D = bits.shape
    if src_pad_heads:
        big = np.zeros((T, H + src_pad_heads, D), np.uint16)
        big[:, :H] = bits
        x = dev_bf16(big)[:, :H]
    else:
        x = dev_bf16(bits)
    codes = None
    if codes_pad:
        codes = torch.full((T, H, D + codes_pad), 0xAB, dtype=torch.uint8, device="cuda")[:, :, :D]
    c, e = tv.kv_quantize_fp8(x, codes=codes)
    torch.cuda.synchronize()
    return c.cpu().numpy(), e.cpu().numpy()


def _assert_quant_equal(bits, label, **kw):
    note(f"fp8 quantise {label}: shape {bits.shape}")
    c, e = _quantize_dev(bits, **kw)
    rc, re_ = oracle.quantize_kv(bits)
    assert np.array_equal(e, re_), f"{label}: exponents differ"
    bad = np.argwhere(c != rc)
    assert bad.size == 0, f"{label}: {len(bad)} codes differ, first {bad[0]} gpu {c[tuple(bad[0])]:#x} " \
                          f"oracle {rc[tuple(bad[0])]:#x}"


def _bits(x):
    """float64 values that are exact in bf16 -> bf16 bits (checked)."""
    b = bf16_bits_from_f32(np.asarray(x, np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(b), np.asarray(x, np.float64))
    return b


def _edge_rows():
    """Rows aimed at the rounding and scaling corners: code midpoints (ties to even),
    the subnormal grid, the top of the range, signed zeros, the carry into the next
    binade, each at many power-of-two row scales."""
    D = 128
    base = np.zeros(D)
    vals = [448.0, 1.0625, 1.1875, -1.0625, -1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10, 248.0, -248.0,
            2.0 ** -9, 2.0 ** -6, 15 * 2.0 ** -10, 0.9375 * 2.0 ** -6 + 2.0 ** -11, 1.9375, 3.875, 30.0, 464.0 / 2,
            0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -12, 7 * 2.0 ** -11]
    base[:len(vals)] = vals
    base[len(vals):] = np.round(np.linspace(-440, 440, D - len(vals)) / 4) * 4
    rows = []
    for k in range(-30, 31, 3):
        rows.append(np.ldexp(base, k))
    rows.append(np.zeros(D))                          # all-zero row: exponent 0, codes 0
    r = np.zeros(D)
    r[5] = -0.0
    rows.append(r)
    r = base.copy()
    r[0] = 450.0                                       # just above 448: exponent 1
    rows.append(r)
    r = base.copy() / 448 * 224                        # amax 224: exponent -1 (224 = 448 / 2)
    rows.append(np.round(r))
    for m in (0.5, 0.75, 0.875, 0.90625, 0.99609375):  # mantissa either side of 448 = 0.875 * 2^9
        r = np.zeros(D)
        r[3] = m * 2.0 ** 12
        r[7] = -m * 2.0 ** 5
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
    rng = np.random.default_rng(2024)
    for T, H in ((1, 1), (3, 8), (257, 8), (1000, 2), (33, 5)):
        x = rng.standard_normal((T, H, 128)).astype(np.float32)
        x *= np.exp2(rng.integers(-40, 41, size=(T, H, 1))).astype(np.float32)
        x[rng.random((T, H, 128)) < 0.05] = 0
        _assert_quant_equal(bf16_bits_from_f32(x), f"random T={T} H={H}")


def test_quantize_every_bf16_value_once():
    """All finite bf16 magnitudes (both signs) in rows that share a top value: every code
    boundary the rounding meets for each row exponent."""
    mags = np.arange(0, 0x7F80, dtype=np.uint16)               # +0 .. largest finite
    allbits = np.concatenate([mags, mags | 0x8000])
    pad = (-len(allbits)) % 128
    allbits = np.concatenate([allbits, np.zeros(pad, np.uint16)])
    bits = allbits.reshape(-1, 1, 128)
    _assert_quant_equal(bits, "all bf16 values")


def test_quantize_strided_views_and_empty():
    rng = np.random.default_rng(5)
    x = bf16_bits_from_f32(rng.standard_normal((40, 3, 128)).astype(np.float32) * 3)
    _assert_quant_equal(x, "strided src", src_pad_heads=2)
    _assert_quant_equal(x, "strided codes", codes_pad=64)
    c, e = tv.kv_quantize_fp8(dev_bf16(np.zeros((0, 4, 128), np.uint16)))
    torch.cuda.synchronize()
    assert c.shape == (0, 4, 128) and e.shape == (0, 4)


def test_quantize_full_size_cache_sampled_rows():
    """long_128k keys and values (131136 tokens x 8 heads): every exponent, and the codes of
    2048 sampled rows, against the oracle row by row."""
    w = make("long_128k", 0, parts=("qkv",))
    rng = np.random.default_rng(11)
    for name, arr in (("k", w.k), ("v", w.v)):
        note(f"fp8 quantise long_128k {name}")
        c, e = _quantize_dev(arr)
        amax = np.abs(oracle.bf16_bits_to_f64(arr)).max(axis=2)
        ref_e = np.vectorize(oracle.row_scale_exponent, otypes=[np.int32])(amax)
        assert np.array_equal(e, ref_e)
        ts = rng.integers(0, arr.shape[0], 256)
        rc, re_ = oracle.quantize_kv(arr[ts])
        assert np.array_equal(c[ts], rc) and np.array_equal(e[ts], re_)
        assert np.array_equal(c[-3:], oracle.quantize_kv(arr[-3:])[0])


# ------------------------------------------------------------ FP8 tree attention


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _fp8_attn_gpu(q_bits, kc, ke, vc, ve, parent, L, scale, num_splits=0, dev_error=None):
    N, Hq, _ = q_bits.shape
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_fp8(dev_bf16(q_bits), _dev_u8(kc), _dev_u8(vc), _dev_i32(ke), _dev_i32(ve),
                           _dev_i32(parent), L=L, scale=scale, num_splits=num_splits, lse=lse, dev_error=dev_error)
    torch.cuda.synchronize()
    return out, lse


def _fp8_ref(q_bits, kc, ke, vc, ve, parent, scale):
    return oracle.tree_attention(oracle.bf16_bits_to_f64(q_bits), oracle.dequantize_kv(kc, ke),
                                 oracle.dequantize_kv(vc, ve), parent, scale)


def _check_fp8_workload(w, label, num_splits=0):
    kc, ke = oracle.quantize_kv(w.k)
    vc, ve = oracle.quantize_kv(w.v)
    note(f"fp8 attention {label}: L={w.L} N={w.N} Hq={w.Hq} Hkv={w.Hkv} splits={num_splits}")
    out, lse = _fp8_attn_gpu(w.q, kc, ke, vc, ve, w.parent, w.L, w.scale, num_splits)
    ref, lref = _fp8_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    return check_attention(out, ref, lse, lref, label)


@pytest.mark.parametrize("name,trials", [("tiny_chain", 3), ("budget22", 3)])
def test_fp8_attention_small_workloads(name, trials):
    for trial in range(trials):
        _check_fp8_workload(make(name, trial), f"{name}/{trial}")


FP8_EDGE = [
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
]


@pytest.mark.parametrize("label,ov", FP8_EDGE, ids=[e[0] for e in FP8_EDGE])
def test_fp8_attention_edge_shapes(label, ov):
    _check_fp8_workload(make("budget22", 7, **ov), label)


# T = 7022 keys, 110 tiles: the requests below give 1, 2, 3, 7, 19, 37, 55 and 110 splits,
# i.e. every 16-split batch count of the single-round-trip merge (up to 64 splits) and the
# chunked merge beyond.
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 20, 40, 55, 1024])
def test_fp8_attention_forced_splits(splits):
    _check_fp8_workload(make("budget22", 11, L=7000, N=22), f"splits={splits}", num_splits=splits)


# Eight stacked rows (the 16-row kernel): each wave streams and widens its own blocks.
# T = 5001 keys: the requests give 1, 4, 40 and 157 splits of 157, 40, 4 and 1 blocks, so
# with few blocks most waves have none, and the last block is cut by the end of the keys.
@pytest.mark.parametrize("splits", [1, 4, 40, 1024])
def test_fp8_attention_single_row_wave_splits(splits):
    _check_fp8_workload(make("decode_1node", 3, L=5000), f"decode splits={splits}", num_splits=splits)


# The 256-row kernel with every short split length (tiles per split 1, 2, 3, 4, 5, 6 and
# 12): the early start of its prologue widens tile 0 alone, then tile 1 midway through
# step 0; the raw-tile ring holds four tiles.
@pytest.mark.parametrize("L,splits", [(700, 12), (700, 6), (700, 4), (700, 3), (700, 2), (700, 1), (1200, 4)])
def test_fp8_attention_dense_short_splits(L, splits):
    _check_fp8_workload(make("branch_8k", 4, L=L), f"8x1 L={L} splits={splits}", num_splits=splits)


# At most 16 stacked rows: the 16-row kernel with K widened in registers and V widened
# into each wave's stage (the same shapes as the bf16 16-row cases); then 17-32 rows, the
# single-row-wave kernel with its own widening.
FP8_ROWS16 = [
    ("chain16_G1", dict(L=1000, N=16, tree="chain", Hq=8, Hkv=8)),
    ("N4_G4", dict(L=2500, N=4, tree="random16", Hq=16, Hkv=4)),
    ("N2_G8_L0", dict(L=0, N=2, tree="chain", Hq=8, Hkv=1)),
    ("N11_G1_L31", dict(L=31, N=11, tree="random16", Hq=3, Hkv=3)),
    ("N3_G5_L96", dict(L=96, N=3, tree="random16", Hq=10, Hkv=2)),
    ("N1_G8_peaky", dict(L=20000, N=1, tree="chain", Hq=8, Hkv=1, peaky=True)),
    ("N2_G6_peaky", dict(L=9000, N=2, tree="chain", Hq=24, Hkv=4, peaky=True)),
]
FP8_ROWS32 = [
    ("N3_G8", dict(L=500, N=3, tree="random16", Hq=8, Hkv=1)),
    ("N17_G1", dict(L=3000, N=17, tree="random16", Hq=4, Hkv=4)),
]


@pytest.mark.parametrize("label,ov", FP8_ROWS16, ids=[e[0] for e in FP8_ROWS16])
def test_fp8_attention_rows16(label, ov):
    w = make("budget22", 13, **ov)
    assert w.N * w.Hq // w.Hkv <= 16
    _check_fp8_workload(w, f"16-row {label}")


@pytest.mark.parametrize("label,ov", FP8_ROWS32, ids=[e[0] for e in FP8_ROWS32])
def test_fp8_attention_rows17_to_32(label, ov):
    w = make("budget22", 14, **ov)
    assert 16 < w.N * w.Hq // w.Hkv <= 32
    _check_fp8_workload(w, f"single-row-wave {label}")


def test_fp8_attention_peaky_keys():
    _check_fp8_workload(make("max_256k", 1, L=20000), "peaky 20k")


def test_fp8_attention_own_key_only_is_exact():
    """Every node a root with L = 0: node i sees only its own key, so its output is its
    dequantised V row exactly (p = 1), whatever the row's scale; the log-sum-exp is the
    scaled score of that key. V rows span exponents from -117 to 119."""
    rng = np.random.default_rng(8)
    N, Hq, Hkv = 256, 8, 4
    parent = np.full(N, -1, np.int32)
    q = bf16_bits_from_f32(rng.standard_normal((N, Hq, 128)).astype(np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((N, Hkv, 128)).astype(np.float32))
    v32 = rng.standard_normal((N, Hkv, 128)).astype(np.float32)
    shifts = rng.integers(-100, 100, size=(N, Hkv, 1))
    shifts[0, 0] = -108                       # amax ~ 2^-106 .. : exponent near the low end
    shifts[1, 0] = 124                        # exponent near the high end
    v64 = v32.astype(np.float64) / np.abs(v32).max(axis=2, keepdims=True) * np.exp2(shifts.astype(np.float64))
    v = bf16_bits_from_f32(v64.astype(np.float32))
    kc, ke = oracle.quantize_kv(k)
    vc, ve = oracle.quantize_kv(v)
    assert ve.min() <= -114 and ve.max() >= 115 and ve.min() >= -117 and ve.max() <= 119
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = _fp8_attn_gpu(q, kc, ke, vc, ve, parent, 0, 1 / np.sqrt(128), dev_error=err)
    assert err.item() == 0
    deq = oracle.dequantize_kv(vc, ve)
    g = Hq // Hkv
    expect = np.repeat(deq, g, axis=1)                          # [N, Hq, D]
    got = out.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[0]}"
    _, lref = _fp8_ref(q, kc, ke, vc, ve, parent, 1 / np.sqrt(128))
    assert np.abs(lse.cpu().numpy() - lref).max() < 1e-3


def test_fp8_attention_strided_cache():
    """Codes as views into a larger cache (every other head of [T, 2*Hkv, D]) and
    exponents sized for a longer cache than L + N."""
    w = make("budget22", 3, L=1500)
    kc, ke = oracle.quantize_kv(w.k)
    vc, ve = oracle.quantize_kv(w.v)
    T = w.L + w.N
    big_k = np.zeros((T + 5, 2 * w.Hkv, 128), np.uint8)
    big_v = np.zeros_like(big_k)
    big_k[:T, ::2] = kc
    big_v[:T, ::2] = vc
    ke_big = np.zeros((T + 9, w.Hkv), np.int32)
    ve_big = np.zeros_like(ke_big)
    ke_big[:T], ve_big[:T] = ke, ve
    out = tv.tree_attn_fp8(dev_bf16(w.q), _dev_u8(big_k)[:, ::2], _dev_u8(big_v)[:, ::2], _dev_i32(ke_big),
                           _dev_i32(ve_big), _dev_i32(w.parent), L=w.L, scale=w.scale)
    ref, _ = _fp8_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    check_attention(out, ref, label="fp8 strided")


@pytest.mark.parametrize("name", ["budget22", "decode_1node"])
def test_fp8_head_major_cache(name):
    """A head-major bf16 cache quantised on the GPU into head-major codes ([Hkv, T, D]
    viewed as [T, Hkv, D]); the exponents stay [T, Hkv]. Codes and exponents equal the
    oracle's, and attention over them matches the oracle on the dequantised cache."""
    w = make(name, 1)
    T = w.L + w.N
    note(f"fp8 head-major {name}")
    kc, ke = oracle.quantize_kv(w.k)
    vc, ve = oracle.quantize_kv(w.v)
    dev = []
    for bits in (w.k, w.v):
        x = dev_bf16(np.ascontiguousarray(bits.transpose(1, 0, 2))).permute(1, 0, 2)
        codes = torch.empty((w.Hkv, T, 128), dtype=torch.uint8, device="cuda").permute(1, 0, 2)
        dev.append(tv.kv_quantize_fp8(x, codes=codes))
    (kcd, ked), (vcd, ved) = dev
    torch.cuda.synchronize()
    assert kcd.stride() == (128, T * 128, 1)
    for got, want in ((kcd, kc), (vcd, vc)):
        assert np.array_equal(got.cpu().numpy(), want)
    for got, want in ((ked, ke), (ved, ve)):
        assert np.array_equal(got.cpu().numpy(), want)
    out = tv.tree_attn_fp8(dev_bf16(w.q), kcd, vcd, ked, ved, _dev_i32(w.parent), L=w.L, scale=w.scale)
    ref, _ = _fp8_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    check_attention(out, ref, label=f"fp8 head-major {name}")


# budget22 (88 rows) widens shared tiles; decode (8 rows) widens each wave's own blocks.
@pytest.mark.parametrize("name", ["budget22", "decode_1node"])
def test_fp8_attention_out_of_range_exponent_is_reported(name):
    w = make(name, 2, L=200)
    kc, ke = oracle.quantize_kv(w.k)
    vc, ve = oracle.quantize_kv(w.v)
    for bad_e in (200, -300):
        ve2 = ve.copy()
        ve2[17, 0] = bad_e
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        _fp8_attn_gpu(w.q, kc, ke, vc, ve2, w.parent, w.L, w.scale, dev_error=err)
        assert err.item() == 1, bad_e
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _fp8_attn_gpu(w.q, kc, ke, vc, ve, w.parent, w.L, w.scale, dev_error=err)
    assert err.item() == 0


def test_fp8_gpu_quantise_then_attend_full_size():
    """long_128k: the cache quantised on the GPU (checked code for code against the
    oracle's) feeds the FP8 attention; reference: the oracle on the oracle's dequantised
    cache."""
    w = make("long_128k", 0, parts=("tree", "qkv"))
    note("fp8 full size: gpu quantise")
    kc_d, ke_d = tv.kv_quantize_fp8(dev_bf16(w.k))
    vc_d, ve_d = tv.kv_quantize_fp8(dev_bf16(w.v))
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_fp8(dev_bf16(w.q), kc_d, vc_d, ke_d, ve_d, _dev_i32(w.parent), L=w.L, scale=w.scale,
                           lse=lse)
    torch.cuda.synchronize()
    note("fp8 full size: oracle quantise")
    kc, ke = oracle.quantize_kv(w.k)
    vc, ve = oracle.quantize_kv(w.v)
    assert np.array_equal(kc_d.cpu().numpy(), kc) and np.array_equal(ke_d.cpu().numpy(), ke)
    assert np.array_equal(vc_d.cpu().numpy(), vc) and np.array_equal(ve_d.cpu().numpy(), ve)
    note("fp8 full size: oracle attention")
    ref, lref = _fp8_ref(w.q, kc, ke, vc, ve, w.parent, w.scale)
    e, r = check_attention(out, ref, lse, lref, "fp8 long_128k")
    note(f"fp8 long_128k: max abs {e:.2e} row rel {r:.2e}")


@pytest.mark.parametrize("name", ["max_256k", "wide_tree", "decode_1node"])
def test_fp8_full_size_sampled_heads(name):
    """The other full-size workloads, as for the 4-bit cache: the whole cache quantised and
    attended on the GPU; for the first and the last KV head the GPU's codes are checked
    against the oracle's quantisation of that head, and that head's query group against the
    oracle on the oracle's dequantised head."""
    w = make(name, 0, parts=("tree", "qkv"))
    G = w.Hq // w.Hkv
    note(f"fp8 {name} full size: gpu quantise and attend")
    kc_d, ke_d = tv.kv_quantize_fp8(dev_bf16(w.k))
    vc_d, ve_d = tv.kv_quantize_fp8(dev_bf16(w.v))
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn_fp8(dev_bf16(w.q), kc_d, vc_d, ke_d, ve_d, _dev_i32(w.parent), L=w.L, scale=w.scale,
                           lse=lse)
    torch.cuda.synchronize()
    for h in (0, w.Hkv - 1):
        note(f"fp8 {name}: oracle, KV head {h}")
        kc, ke = oracle.quantize_kv(w.k[:, h:h + 1])
        vc, ve = oracle.quantize_kv(w.v[:, h:h + 1])
        assert np.array_equal(kc_d[:, h:h + 1].cpu().numpy(), kc) and np.array_equal(ke_d[:, h:h + 1].cpu().numpy(), ke)
        assert np.array_equal(vc_d[:, h:h + 1].cpu().numpy(), vc) and np.array_equal(ve_d[:, h:h + 1].cpu().numpy(), ve)
        ref, lref = _fp8_ref(w.q[:, h * G:(h + 1) * G], kc, ke, vc, ve, w.parent, w.scale)
        e, r = check_attention(out[:, h * G:(h + 1) * G], ref, lse[:, h * G:(h + 1) * G], lref,
                               f"fp8 {name} head {h}")
        note(f"fp8 {name} head {h}: max abs {e:.2e} row rel {r:.2e}")
