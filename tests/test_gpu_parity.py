"""GPU parity: every libtv entry point against the CPU oracle on the same seeded inputs.

Integer results (ancestor masks, depths, argmax, acceptance) must be bit exact. Attention
must satisfy max-abs error <= 1e-2 and per-row relative L2 error <= 2e-2 (bf16 output,
fp32 accumulation), and |lse error| <= 1e-3.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import check_attention, dev_bf16, dev_i32, note
from workloads import (accept_trial, bf16_bits_from_f32, chain_parent, kary_bfs_parent, make, random_tree_parent,
                       rng_for, tie_rows)

pytestmark = pytest.mark.gpu

tv = pytest.importorskip("draft_tree_verification_tv_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


# ------------------------------------------------------------------ a1 tree prep


def tree_cases():
    cases = [("chain1", chain_parent(1)), ("chain16", chain_parent(16)), ("chain256", chain_parent(256)),
             ("kary256", kary_bfs_parent(256, 4)), ("kary85_3", kary_bfs_parent(85, 3))]
    for n in (2, 5, 22, 63, 64, 65, 130, 256):
        for seed in range(3):
            cases.append((f"rand{n}_{seed}", random_tree_parent(rng_for(90, seed * 1000 + n), n, 16, 4)))
    cases.append(("flat256", np.full(256, -1, dtype=np.int32)))
    return cases


def test_tree_prep_matches_oracle():
    for name, parent in tree_cases():
        anc, depth = tv.tree_prep(dev_i32(parent))
        torch.cuda.synchronize()
        exp_anc = oracle.anc_bitmask_words(parent)
        exp_depth, _ = oracle.tree_structure(parent)
        got = anc.cpu().numpy().view(np.uint64)
        assert np.array_equal(got, exp_anc), name
        assert np.array_equal(depth.cpu().numpy(), exp_depth), name


def test_tree_prep_every_small_tree():
    for n in range(1, 6):
        for p in itertools.product(*[range(-1, i) for i in range(n)]):
            parent = np.array(p, dtype=np.int32)
            anc, depth = tv.tree_prep(dev_i32(parent))
            assert np.array_equal(anc.cpu().numpy().view(np.uint64), oracle.anc_bitmask_words(parent))
            assert np.array_equal(depth.cpu().numpy(), oracle.tree_structure(parent)[0])


def test_bad_tree_reported_and_clamped():
    bad = np.array([-1, 0, 5, 1, -7], dtype=np.int32)      # entries 2 and 4 are invalid
    clamped = np.array([-1, 0, -1, 1, -1], dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    anc, depth = tv.tree_prep(dev_i32(bad), dev_error=err)
    assert err.item() == 2
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), oracle.anc_bitmask_words(clamped))
    err.zero_()
    tv.tree_prep(dev_i32(clamped), dev_error=err)
    assert err.item() == 0


# ------------------------------------------------------------------ a6 accept


def run_accept(parent, draft, tok):
    ln, nodes, toks, bonus = tv.accept(dev_i32(parent), dev_i32(draft), dev_i32(tok))
    return ln.item(), nodes.cpu().numpy(), toks.cpu().numpy(), bonus.item()


def assert_accept_equal(parent, draft, tok, label):
    ln, nodes, toks, bonus = run_accept(parent, draft, tok)
    e_ln, e_nodes, e_toks, e_bonus = oracle.accept(parent, draft, tok)
    n = len(parent)
    assert ln == e_ln, label
    assert nodes[:ln].tolist() == e_nodes.tolist(), label
    assert toks[:ln].tolist() == e_toks.tolist(), label
    assert (nodes[ln:] == -1).all() and (toks[ln:] == -1).all(), label
    assert bonus == e_bonus, label
    assert len(nodes) == n


def test_accept_branch_8k_1000_trials():
    for trial in range(1000):
        parent, draft, tok, plen, pend = accept_trial("branch_8k", trial)
        ln, nodes, _, _ = run_accept(parent, draft, tok)
        assert ln == plen, trial
        if plen:
            assert nodes[ln - 1] == pend
        if trial % 50 == 0:
            assert_accept_equal(parent, draft, tok, f"branch_8k/{trial}")


@pytest.mark.parametrize("name,trials", [("tiny_chain", 100), ("wide_tree", 50), ("max_256k", 30),
                                         ("budget22", 100), ("decode_1node", 20)])
def test_accept_planted(name, trials):
    for trial in range(trials):
        parent, draft, tok, _, _ = accept_trial(name, trial)
        assert_accept_equal(parent, draft, tok, f"{name}/{trial}")


def test_accept_random_small_vocab():
    """Tiny vocabularies make many nodes match, so ties between paths are common."""
    rng = np.random.default_rng(123)
    for case in range(400):
        n = int(rng.integers(1, 257)) if case % 4 == 0 else int(rng.integers(1, 20))
        parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
        vocab = int(rng.integers(1, 4))
        draft = rng.integers(0, vocab, n).astype(np.int32)
        tok = rng.integers(0, vocab, n).astype(np.int32)
        assert_accept_equal(parent, draft, tok, f"random/{case}")


def test_accept_all_match_and_none():
    w = make("wide_tree", 0, parts=("tree",), plant="all")
    assert_accept_equal(w.parent, w.draft, w.draft, "wide all")
    ln, nodes, _, _ = run_accept(w.parent, w.draft, w.draft)
    assert ln == 4 and nodes[:4].tolist() == [0, 4, 20, 84]
    assert_accept_equal(w.parent, w.draft, w.draft + 1, "wide none")


# ------------------------------------------------------------------ a5 argmax


def run_argmax(x, dtype, row_stride=None):
    n, v = x.shape
    if row_stride is not None and row_stride != v:
        pad = np.zeros((n, row_stride), dtype=x.dtype)
        pad[:, :v] = x
        x_dev = pad
    else:
        x_dev = x
    t = dev_bf16(x_dev) if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(x_dev)).cuda()
    return tv.argmax(t, V=v).cpu().numpy()


def oracle_rows(x, dtype):
    return oracle.argmax_rows(oracle.bf16_bits_to_f64(x) if dtype == "bf16" else x.astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 8, 9, 100, 4095, 4096, 4097, 65536, 152063, 152064])
def test_argmax_tie_rows(dtype, V):
    rng = np.random.default_rng(V)
    if V < 3:
        x = rng.standard_normal((3, V)).astype(np.float32)
        from workloads import bf16_bits_from_f32
        x = bf16_bits_from_f32(x) if dtype == "bf16" else x
    else:
        x = tie_rows(rng, V, dtype)
    exp = oracle_rows(x, dtype)
    assert np.array_equal(run_argmax(x, dtype), exp)
    assert np.array_equal(run_argmax(x, dtype, row_stride=V + 3), exp)     # unaligned rows


@pytest.mark.parametrize("name,trials", [("tiny_chain", 10), ("branch_8k", 6), ("wide_tree", 2),
                                         ("max_256k", 2), ("decode_1node", 3), ("budget22", 4)])
def test_argmax_workloads(name, trials):
    ties = 0
    for trial in range(trials):
        w = make(name, trial, parts=("tree", "logits"))
        exp = oracle_rows(w.logits, w.logits_dtype)
        got = run_argmax(w.logits, w.logits_dtype)
        assert np.array_equal(got, exp), (name, trial)
        x = oracle.bf16_bits_to_f64(w.logits) if w.logits_dtype == "bf16" else w.logits
        ties += int(((x == x.max(axis=1, keepdims=True)).sum(axis=1) > 1).sum())
    note(f"{name}: {ties} tied rows checked")


def test_argmax_many_rows_reuses_workspace():
    rng = np.random.default_rng(5)
    ws = tv.argmax_workspace(300, 5000, "cuda")
    for rep in range(3):
        x = rng.standard_normal((300, 5000)).astype(np.float32)
        x[:, 17] = x.max(axis=1) if rep == 1 else x[:, 17]
        t = torch.from_numpy(x).cuda()
        got = tv.argmax(t, workspace=ws).cpu().numpy()
        assert np.array_equal(got, oracle.argmax_rows(x.astype(np.float64)))


# ------------------------------------------------------------------ a2-a4 attention


def attn_gpu(w, num_splits=0, with_lse=True):
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda") if with_lse else None
    out = tv.tree_attn(q, k, v, dev_i32(w.parent), L=w.L, scale=w.scale, num_splits=num_splits, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def attn_ref(w):
    return oracle.tree_attention(oracle.bf16_bits_to_f64(w.q), oracle.bf16_bits_to_f64(w.k),
                                 oracle.bf16_bits_to_f64(w.v), w.parent, w.scale)


@pytest.mark.parametrize("name,trials", [("tiny_chain", 4), ("budget22", 3)])
def test_attention_small_workloads(name, trials):
    for trial in range(trials):
        w = make(name, trial)
        note(f"attention {name} trial {trial}")
        out, lse = attn_gpu(w)
        ref, lref = attn_ref(w)
        check_attention(out, ref, lse, lref, f"{name}/{trial}")


EDGE = [
    # (label, overrides)
    ("L0_N1", dict(L=0, N=1, tree="chain", Hq=8, Hkv=2)),
    ("L0_N22", dict(L=0, N=22, tree="random16", Hq=8, Hkv=8)),
    ("L1_N5", dict(L=1, N=5, tree="random16", Hq=4, Hkv=1)),
    ("L63_N1", dict(L=63, N=1, tree="chain", Hq=2, Hkv=2)),
    ("L65_N3_mha", dict(L=65, N=3, tree="random16", Hq=1, Hkv=1)),
    ("L1000_kary256_G1", dict(L=1000, N=256, tree="kary4", Hq=8, Hkv=8)),
    ("L300_kary256_G8", dict(L=300, N=256, tree="kary4", Hq=16, Hkv=2)),
    ("L777_G6_chain16", dict(L=777, N=16, tree="chain", Hq=24, Hkv=4)),
    ("L4097_N64", dict(L=4097, N=64, tree="random16", Hq=32, Hkv=8)),
    ("L2048_N40_G5", dict(L=2048, N=40, tree="random16", Hq=10, Hkv=2)),
]


@pytest.mark.parametrize("label,ov", EDGE, ids=[e[0] for e in EDGE])
def test_attention_edge_shapes(label, ov):
    w = make("budget22", 7, **ov)
    note(f"attention edge {label}")
    out, lse = attn_gpu(w)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, label)


# T = 7022 keys, 110 tiles: the requests below give 1, 2, 3, 7, 19, 37, 55 and 110 splits,
# i.e. every 16-split batch count of the single-round-trip merge (up to 64 splits) and the
# chunked merge beyond.
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 20, 40, 55, 1024])
def test_attention_forced_splits(splits):
    w = make("budget22", 11, L=7000, N=22)
    note(f"attention forced splits {splits}")
    out, lse = attn_gpu(w, num_splits=splits)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, f"splits={splits}")


# At most 16 stacked rows: every wave streams its own 32-key blocks, and splits are whole
# blocks. T = 5001 keys, 157 blocks: the requests give 1, 4, 40 and 157 splits of 157, 40,
# 4 and 1 blocks (the last split's final block is cut by the end of the keys), so with 4
# or 1 blocks most waves have none.
@pytest.mark.parametrize("splits", [1, 4, 40, 1024])
def test_attention_single_row_wave_splits(splits):
    w = make("decode_1node", 3, L=5000)
    note(f"attention decode forced splits {splits}")
    out, lse = attn_gpu(w, num_splits=splits)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, f"decode splits={splits}")


# At most 16 stacked rows (N * G <= 16): the 16x16-tile kernel. The shapes fill the tile
# exactly (16 x 1, 4 x 4, 2 x 8 rows) or partly, put tree keys in the last block (chains,
# random trees, a pure tree with L = 0, ragged lengths) and, with peaky keys, move the
# lazy softmax reference often.
ROWS16 = [
    ("chain16_G1", dict(L=1000, N=16, tree="chain", Hq=8, Hkv=8)),
    ("N4_G4", dict(L=2500, N=4, tree="random16", Hq=16, Hkv=4)),
    ("N2_G8_L0", dict(L=0, N=2, tree="chain", Hq=8, Hkv=1)),
    ("N11_G1_L31", dict(L=31, N=11, tree="random16", Hq=3, Hkv=3)),
    ("N3_G5_L96", dict(L=96, N=3, tree="random16", Hq=10, Hkv=2)),
    ("N1_G8_peaky", dict(L=20000, N=1, tree="chain", Hq=8, Hkv=1, peaky=True)),
    ("N2_G6_peaky", dict(L=9000, N=2, tree="chain", Hq=24, Hkv=4, peaky=True)),
]


@pytest.mark.parametrize("label,ov", ROWS16, ids=[e[0] for e in ROWS16])
def test_attention_rows16(label, ov):
    w = make("budget22", 13, **ov)
    assert w.N * w.Hq // w.Hkv <= 16
    note(f"attention 16-row {label}")
    out, lse = attn_gpu(w)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, label)


# The 256-row kernel (8 row-waves) with every short split length: at L = 700, T = 764
# keys, 12 tiles, and the requests give splits of 1, 2, 3, 4, 6 and 12 tiles; at L = 1200,
# T = 1264 keys, 20 tiles, four splits of 5 tiles (the last one cut short). They exercise
# the prologue's early start (tile 0 only, then tile 1 midway through step 0) and the
# unroll's remainder.
DENSE_SHORT = [(700, 12), (700, 6), (700, 4), (700, 3), (700, 2), (700, 1), (1200, 4)]


@pytest.mark.parametrize("L,splits", DENSE_SHORT)
def test_attention_dense_short_splits(L, splits):
    w = make("branch_8k", 4, L=L)
    note(f"attention 8x1 L={L} forced splits {splits}")
    out, lse = attn_gpu(w, num_splits=splits)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, f"8x1 splits={splits}")


def test_attention_peaky_keys():
    w = make("max_256k", 1, L=20000)
    note("attention peaky 20k")
    out, lse = attn_gpu(w)
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, "peaky")


def test_attention_strided_cache():
    """K/V given as views into a larger cache ([T, 2*Hkv, D], using even heads)."""
    w = make("budget22", 3, L=1500)
    big_k = np.zeros((w.L + w.N + 5, 2 * w.Hkv, 128), dtype=np.uint16)
    big_v = np.zeros_like(big_k)
    big_k[: w.L + w.N, ::2] = w.k
    big_v[: w.L + w.N, ::2] = w.v
    kd, vd = dev_bf16(big_k)[:, ::2], dev_bf16(big_v)[:, ::2]
    out = tv.tree_attn(dev_bf16(w.q), kd, vd, dev_i32(w.parent), L=w.L, scale=w.scale)
    ref, _ = attn_ref(w)
    check_attention(out, ref, label="strided")


# One case per kernel: the 16-row kernel (decode), 2x4 (tiny_chain), 4x2 (budget22), 8x1
# (branch_8k).
@pytest.mark.parametrize("name,trial", [("decode_1node", 0), ("tiny_chain", 1), ("budget22", 3), ("branch_8k", 2)])
def test_attention_head_major_cache(name, trial):
    """K and V stored head-major ([Hkv, T, D]: each head's rows contiguous) and passed as
    [T, Hkv, D] views with strides (D, T*D): the same kernels, through the strides."""
    w = make(name, trial)
    T = w.L + w.N
    note(f"attention head-major {name} trial {trial}")
    kh = dev_bf16(np.ascontiguousarray(w.k.transpose(1, 0, 2)))
    vh = dev_bf16(np.ascontiguousarray(w.v.transpose(1, 0, 2)))
    k, v = kh.permute(1, 0, 2), vh.permute(1, 0, 2)
    assert k.stride() == (128, T * 128, 1)
    lse = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn(dev_bf16(w.q), k, v, dev_i32(w.parent), L=w.L, scale=w.scale, lse=lse)
    torch.cuda.synchronize()
    ref, lref = attn_ref(w)
    check_attention(out, ref, lse, lref, f"{name} head-major")


def test_binding_uses_the_current_stream():
    """A call without an explicit stream runs on torch's current stream. On a side stream
    the query is overwritten behind a spin of several milliseconds, then attention reads
    it: only a launch on that same stream sees the new query."""
    w = make("budget22", 5)
    q_new_bits = np.ascontiguousarray(np.flip(w.q, axis=1))
    k, v, parent = dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.parent)
    q = dev_bf16(w.q)
    q_new = dev_bf16(q_new_bits)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
        q.copy_(q_new)
        out = tv.tree_attn(q, k, v, parent, L=w.L, scale=w.scale)
    side.synchronize()
    ref, _ = oracle.tree_attention(oracle.bf16_bits_to_f64(q_new_bits), oracle.bf16_bits_to_f64(w.k),
                                   oracle.bf16_bits_to_f64(w.v), w.parent, w.scale)
    check_attention(out, ref, None, None, "side stream")


def test_attention_bad_tree_flag():
    w = make("budget22", 2, L=200)
    bad = w.parent.copy()
    bad[5] = 9
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = tv.tree_attn(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_i32(bad), L=w.L, scale=w.scale,
                       dev_error=err)
    torch.cuda.synchronize()
    assert err.item() == 2
    fixed = bad.copy()
    fixed[5] = -1
    ref, _ = oracle.tree_attention(oracle.bf16_bits_to_f64(w.q), oracle.bf16_bits_to_f64(w.k),
                                   oracle.bf16_bits_to_f64(w.v), fixed, w.scale)
    check_attention(out, ref, label="clamped tree")


# ---------------------------------------------------------- full-size workloads


@pytest.mark.parametrize("name,trial", [("branch_8k", 0), ("branch_8k", 1), ("long_128k", 0),
                                        ("max_256k", 0), ("wide_tree", 0), ("decode_1node", 0)])
def test_attention_full_size(name, trial):
    note(f"full-size attention {name} trial {trial}: generating")
    w = make(name, trial, parts=("tree", "qkv"))
    note(f"full-size attention {name}: gpu")
    out, lse = attn_gpu(w)
    note(f"full-size attention {name}: oracle")
    ref, lref = attn_ref(w)
    e, r = check_attention(out, ref, lse, lref, f"{name}/{trial}")
    note(f"{name}: max abs {e:.2e} row rel {r:.2e}")


# ---------------------------------------------------------- whole verify step


@pytest.mark.parametrize("name,trial", [("tiny_chain", 0), ("tiny_chain", 5), ("budget22", 1),
                                        ("branch_8k", 2)])
def test_verify_pipeline(name, trial):
    w = make(name, trial)
    logits = dev_bf16(w.logits) if w.logits_dtype == "bf16" else torch.from_numpy(w.logits).cuda()
    out, tok, (ln, nodes, toks, bonus) = tv.verify(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                                   dev_i32(w.parent), logits, dev_i32(w.draft), L=w.L,
                                                   scale=w.scale)
    ref, _, etok, (eln, enodes, etoks, ebonus) = oracle.verify(
        oracle.bf16_bits_to_f64(w.q), oracle.bf16_bits_to_f64(w.k), oracle.bf16_bits_to_f64(w.v), w.parent,
        w.scale, oracle.bf16_bits_to_f64(w.logits) if w.logits_dtype == "bf16" else w.logits, w.draft)
    check_attention(out, ref, label=name)
    assert np.array_equal(tok.cpu().numpy(), etok)
    assert ln.item() == eln == w.planted_len
    assert nodes.cpu().numpy()[:eln].tolist() == enodes.tolist()
    assert toks.cpu().numpy()[:eln].tolist() == etoks.tolist()
    assert bonus.item() == ebonus


# ------------------------------------------------------ a5 + a6 in one call


def check_argmax_accept(logits_dev, parent, draft, etok, label):
    tok, (ln, nodes, toks, bonus) = tv.argmax_accept(logits_dev, dev_i32(parent), dev_i32(draft))
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), etok), label
    e_ln, e_nodes, e_toks, e_bonus = oracle.accept(parent, draft, etok)
    ln = ln.item()
    nodes, toks = nodes.cpu().numpy(), toks.cpu().numpy()
    assert ln == e_ln, label
    assert nodes[:ln].tolist() == e_nodes.tolist(), label
    assert toks[:ln].tolist() == e_toks.tolist(), label
    assert (nodes[ln:] == -1).all() and (toks[ln:] == -1).all(), label
    assert bonus.item() == e_bonus, label
    return ln


@pytest.mark.parametrize("name,trials", [("tiny_chain", 6), ("branch_8k", 12), ("wide_tree", 3),
                                         ("max_256k", 2), ("budget22", 4), ("decode_1node", 2)])
def test_argmax_accept_workloads(name, trials):
    """Fused argmax + walk equals the oracle's argmax and walk (and the planted length)."""
    for trial in range(trials):
        w = make(name, trial, parts=("tree", "logits"))
        note(f"argmax_accept {name} trial {trial}")
        if w.logits_dtype == "bf16":
            lg, etok = dev_bf16(w.logits), oracle.argmax_rows(oracle.bf16_bits_to_f64(w.logits))
        else:
            lg, etok = torch.from_numpy(w.logits).cuda(), oracle.argmax_rows(w.logits.astype(np.float64))
        ln = check_argmax_accept(lg, w.parent, w.draft, etok, f"{name}/{trial}")
        assert ln == w.planted_len


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,stride", [(1, 1), (4096, 4096), (8192, 8192), (8193, 8200), (152064, 152064),
                                      (152063, 152067)])
def test_argmax_accept_small_vocab_trees(dtype, V, stride):
    """Random trees with draft tokens drawn from the top few logits, so paths and ties vary;
    one and several slices per row, aligned and unaligned rows."""
    rng = np.random.default_rng(V + 7 * stride)
    for case in range(3):
        n = [1, 37, 256][case]
        parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
        x = rng.standard_normal((n, stride)).astype(np.float32)
        x[:, : min(V, 3)] += 5.0                     # a few large candidates per row
        if V >= 3 and case == 1:
            x[::3, 1] = x[::3, 0]                    # exact ties at the maximum
        xv = x if dtype == "f32" else None
        if dtype == "bf16":
            bits = bf16_bits_from_f32(x)
            etok = oracle.argmax_rows(oracle.bf16_bits_to_f64(bits[:, :V]))
            lg = dev_bf16(bits)[:, :V]
        else:
            etok = oracle.argmax_rows(xv[:, :V].astype(np.float64))
            lg = torch.from_numpy(xv).cuda()[:, :V]
        draft = np.where(rng.random(n) < 0.7, etok, rng.integers(0, max(V, 1), n)).astype(np.int32)
        check_argmax_accept(lg, parent, draft, etok, f"{dtype}/V{V}/s{stride}/n{n}")


def test_argmax_accept_random_trees():
    rng = np.random.default_rng(2024)
    for case in range(200):
        n = int(rng.integers(1, 257)) if case % 4 == 0 else int(rng.integers(1, 24))
        parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
        V = int(rng.integers(1, 5)) * 4096 + int(rng.integers(0, 9))
        x = rng.standard_normal((n, V)).astype(np.float32)
        bits = bf16_bits_from_f32(x)
        etok = oracle.argmax_rows(oracle.bf16_bits_to_f64(bits))
        draft = np.where(rng.random(n) < 0.8, etok, (etok + 1) % V).astype(np.int32)
        check_argmax_accept(dev_bf16(bits), parent, draft, etok, f"random/{case}")


# ------------------------------------------------------ NEXT: accepted-path KV commit


def _commit_case(rng, n, L, hkv, d, stride_extra_heads=0, chain=False):
    if chain:   # long accepted paths (several batches of 16 rows)
        parent = np.arange(-1, n - 1, dtype=np.int32)
    else:
        parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
    tok = rng.integers(0, 3, n).astype(np.int32)
    draft = np.where(rng.random(n) < (0.98 if chain else 0.8), tok, (tok + 1) % 3).astype(np.int32)
    hs = hkv + stride_extra_heads
    k = rng.integers(0, 1 << 16, (L + n + 3, hs, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (L + n + 3, hs, d), dtype=np.uint16)
    return parent, draft, tok, k, v


def _run_commit(parent, draft, tok, k, v, L, hkv):
    """GPU accept feeding the GPU commit; compared bit for bit with the oracle."""
    kd = torch.from_numpy(k.view(np.int16)).cuda()
    vd = torch.from_numpy(v.view(np.int16)).cuda()
    kv_k, kv_v = kd[:, :hkv], vd[:, :hkv]
    ln, nodes, _, _ = tv.accept(dev_i32(parent), dev_i32(draft), dev_i32(tok))
    new_len = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tv.kv_commit(kv_k, kv_v, L, ln, nodes, new_len=new_len, dev_error=err)
    torch.cuda.synchronize()
    m, enodes, _, _ = oracle.accept(parent, draft, tok)
    ek, ev = oracle.kv_commit(k[:, :hkv], v[:, :hkv], L, enodes)
    gk = kd.cpu().numpy().view(np.uint16)
    gv = vd.cpu().numpy().view(np.uint16)
    assert err.item() == 0 and new_len.item() == L + m
    assert np.array_equal(gk[:, :hkv], ek) and np.array_equal(gv[:, :hkv], ev)
    assert np.array_equal(gk[:, hkv:], k[:, hkv:]) and np.array_equal(gv[:, hkv:], v[:, hkv:])
    return m


def test_kv_commit_random_trees():
    rng = np.random.default_rng(77)
    lens = []
    for case in range(60):
        n = int(rng.integers(1, 257)) if case % 5 == 0 else int(rng.integers(1, 40))
        L = int(rng.integers(0, 300))
        hkv, d = [(8, 128), (2, 128), (1, 64), (4, 8)][case % 4]
        chain = case % 3 == 1
        parent, draft, tok, k, v = _commit_case(rng, n, L, hkv, d, chain=chain)
        note(f"kv_commit case {case}: n={n} L={L} hkv={hkv} d={d} chain={chain}")
        lens.append(_run_commit(parent, draft, tok, k, v, L, hkv))
    assert max(lens) > 16                           # several batches of 16 rows crossed


def test_kv_commit_strided_view_and_chain():
    rng = np.random.default_rng(3)
    parent, draft, tok, k, v = _commit_case(rng, 40, 100, 4, 128, stride_extra_heads=3)
    _run_commit(parent, draft, tok, k, v, 100, 4)
    n = 20
    parent = np.arange(-1, n - 1, dtype=np.int32)      # a chain fully accepted: identity
    k = rng.integers(0, 1 << 16, (50 + n, 2, 128), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (50 + n, 2, 128), dtype=np.uint16)
    assert _run_commit(parent, np.zeros(n, np.int32), np.zeros(n, np.int32), k, v, 50, 2) == n
    # nothing accepted: the cache must not change
    assert _run_commit(parent, np.zeros(n, np.int32), np.ones(n, np.int32), k, v, 50, 2) == 0


def test_kv_commit_head_major_cache():
    """A head-major cache ([Hkv, T, D] viewed as [T, Hkv, D]): GPU accept feeding the GPU
    commit, bit for bit against the oracle; rows past L + N stay untouched."""
    rng = np.random.default_rng(41)
    for case, (n, L, hkv, d, chain) in enumerate(((40, 100, 4, 128, False), (33, 70, 8, 128, True),
                                                 (200, 5, 2, 64, False))):
        parent, draft, tok, k, v = _commit_case(rng, n, L, hkv, d, chain=chain)
        note(f"kv_commit head-major case {case}: n={n} L={L} hkv={hkv} d={d}")
        kh = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)).view(np.int16)).cuda()
        vh = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)).view(np.int16)).cuda()
        kd, vd = kh.permute(1, 0, 2), vh.permute(1, 0, 2)
        assert kd.stride() == (d, k.shape[0] * d, 1)
        ln, nodes, _, _ = tv.accept(dev_i32(parent), dev_i32(draft), dev_i32(tok))
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        tv.kv_commit(kd, vd, L, ln, nodes, dev_error=err)
        torch.cuda.synchronize()
        m, enodes, _, _ = oracle.accept(parent, draft, tok)
        ek, ev = oracle.kv_commit(k, v, L, enodes)
        assert err.item() == 0 and int(ln.item()) == m
        assert np.array_equal(kh.cpu().numpy().view(np.uint16).transpose(1, 0, 2), ek)
        assert np.array_equal(vh.cpu().numpy().view(np.uint16).transpose(1, 0, 2), ev)


def test_kv_commit_full_size_cache():
    w = make("long_128k", 0, parts=("tree", "qkv"))
    tok = np.where(w.matched, w.draft, (w.draft + 1) % w.V).astype(np.int32)
    note(f"kv_commit long_128k planted length {w.planted_len}")
    m = _run_commit(w.parent, w.draft, tok, w.k, w.v, w.L, w.Hkv)
    assert m == w.planted_len


def test_kv_commit_rejects_bad_paths_on_device():
    rng = np.random.default_rng(9)
    k = rng.integers(0, 1 << 16, (60, 2, 128), dtype=np.uint16)
    kd = torch.from_numpy(k.view(np.int16)).cuda()
    vd = kd.clone()
    for ln, nodes in ((3, [0, 2, 2, 9]), (2, [1, 0, 5, 6]), (5, [0, 1, 2, 3]), (-1, [0, 1, 2, 3]),
                      (2, [0, 4, 0, 0])):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        tv.kv_commit(kd, vd, 50, dev_i32([ln]), dev_i32(nodes), dev_error=err)
        torch.cuda.synchronize()
        assert err.item() == 1, (ln, nodes)
        assert np.array_equal(kd.cpu().numpy().view(np.uint16), k)


# ------------------------------------------------------ NEXT: sampled verification (T > 0)


def _sample_dev(logits_dev, parent, draft, T, seed, offset):
    tok, (ln, nodes, toks, bonus) = tv.sample_accept(logits_dev, dev_i32(parent), dev_i32(draft), T, seed, offset)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), ln.item(), nodes.cpu().numpy(), toks.cpu().numpy(), bonus.item()


def _check_sampled_tokens(x, T, seed, offset, tok):
    """The kernel scores logit / T + Gumbel noise in float32; the oracle in float64. The
    sampled token is unique unless a row's two best scores lie within the float32 error of
    the kernel's score: fma rounding of x / T plus two hardware logarithms, bounded here by
    2^-20 (1 + |x / T| + 17) per score (|G| <= 17 for the 23-bit uniforms). Tokens must
    equal the oracle's, except on such near-tie rows, where the kernel's token must score
    within twice that bound of the row maximum."""
    u = oracle.uniforms(x.shape[0], x.shape[1], seed, offset)
    sc = x / T - np.log(-np.log(u))
    etok = sc.argmax(axis=1)
    diff = np.flatnonzero(tok != etok)
    for i in diff:
        tol = 2 * 2.0 ** -20 * (1 + np.abs(x[i] / T).max() + 17)
        assert sc[i, tok[i]] >= sc[i].max() - tol, (i, tok[i], etok[i])
    assert len(diff) <= max(1, len(tok) // 50), diff
    return etok


@pytest.mark.parametrize("name,T,seed,offset", [("tiny_chain", 1.0, 7, 0), ("tiny_chain", 0.3, 7, 1),
                                                ("budget22", 1.0, 123456789012, 5), ("budget22", 2.5, 3, 1 << 40),
                                                ("decode_1node", 0.8, 42, 9)])
def test_sample_accept_matches_oracle(name, T, seed, offset):
    """Same Philox stream and Gumbel-max rule: the sampled tokens are the oracle's (up to
    float32 near-ties, see _check_sampled_tokens), and the walk on them is bit exact."""
    w = make(name, 0, parts=("tree", "logits"))
    note(f"sample_accept {name} T={T}")
    if w.logits_dtype == "bf16":
        lg, x = dev_bf16(w.logits), oracle.bf16_bits_to_f64(w.logits)
    else:
        lg, x = torch.from_numpy(w.logits).cuda(), w.logits.astype(np.float64)
    tok, ln, nodes, toks, bonus = _sample_dev(lg, w.parent, w.draft, T, seed, offset)
    etok = _check_sampled_tokens(x, T, seed, offset, tok)
    if np.array_equal(tok, etok):
        otok, _ = oracle.sample_accept(w.parent, w.draft, x, T, seed, offset)
        assert np.array_equal(otok, etok)
    eln, enodes, etoks, ebonus = oracle.accept(w.parent, w.draft, tok)
    assert ln == eln and nodes[:ln].tolist() == enodes.tolist() and toks[:ln].tolist() == etoks.tolist()
    assert (nodes[ln:] == -1).all() and bonus == ebonus


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,stride", [(5, 5), (4096, 4096), (8200, 8203), (40000, 40000)])
def test_sample_accept_layouts(dtype, V, stride):
    rng = np.random.default_rng(V + stride)
    n = 19
    parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
    x = (rng.standard_normal((n, stride)) * 2).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(x)
        lg, xv = dev_bf16(bits)[:, :V], oracle.bf16_bits_to_f64(bits[:, :V])
    else:
        lg, xv = torch.from_numpy(x).cuda()[:, :V], x[:, :V].astype(np.float64)
    etok = oracle.sample_rows(xv, 1.3, 77, 3)
    draft = np.where(rng.random(n) < 0.6, etok, (etok + 1) % V).astype(np.int32)
    tok, ln, nodes, _, bonus = _sample_dev(lg, parent, draft, 1.3, 77, 3)
    _check_sampled_tokens(xv, 1.3, 77, 3, tok)
    e_ln, e_nodes, _, e_bonus = oracle.accept(parent, draft, tok)
    assert ln == e_ln and nodes[:ln].tolist() == e_nodes.tolist() and bonus == e_bonus


def test_sample_frequencies_follow_softmax():
    """GPU samples over many offsets: chi-square against softmax(logits / T)."""
    logits = np.array([0.0, 1.0, -0.5, 2.0, 0.3, -2.0, 1.5, 0.0], dtype=np.float32)
    T, n = 0.8, 64
    x = np.tile(logits, (n, 1))
    lg = torch.from_numpy(x).cuda()
    parent = np.arange(-1, n - 1, dtype=np.int32)
    counts = np.zeros(8)
    for off in range(300):
        tok, *_ = _sample_dev(lg, parent, np.zeros(n, np.int32), T, 2024, off)
        counts += np.bincount(tok, minlength=8)
    p = np.exp(logits / T - (logits / T).max())
    p /= p.sum()
    tot = counts.sum()
    chi2 = ((counts - tot * p) ** 2 / (tot * p)).sum()
    assert chi2 < 24, (counts, tot * p)          # 7 dof: p ~ 0.001


def test_sample_low_temperature_is_greedy_and_repeatable():
    w = make("branch_8k", 3, parts=("tree", "logits"))
    lg = dev_bf16(w.logits)
    tok_g, (ln_g, nodes_g, _, _) = tv.argmax_accept(lg, dev_i32(w.parent), dev_i32(w.draft))
    tok_s, ln_s, nodes_s, _, _ = _sample_dev(lg, w.parent, w.draft, 1e-6, 5, 0)
    # At T = 1e-6 one bf16 step of a logit outweighs any Gumbel difference, so the sample is
    # a maximal logit: the argmax where the maximum is unique, one of the tied maxima else.
    x = oracle.bf16_bits_to_f64(w.logits)
    for i in range(w.N):
        top = np.flatnonzero(x[i] == x[i].max())
        assert tok_s[i] in top, i
        if top.size == 1:
            assert tok_s[i] == tok_g[i].item(), i
    assert ln_s == ln_g.item() == w.planted_len      # planted rows have a unique +16 maximum
    a = _sample_dev(lg, w.parent, w.draft, 1.0, 5, 0)[0]
    b = _sample_dev(lg, w.parent, w.draft, 1.0, 5, 0)[0]
    c = _sample_dev(lg, w.parent, w.draft, 1.0, 5, 1)[0]
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_one_workspace_serves_any_sequence_of_calls():
    """One argmax workspace, sized for the largest call, reused by tv_argmax,
    tv_argmax_accept and tv_sample_accept calls of varying shapes: every result still
    matches the oracle (no call depends on what an earlier one left in it)."""
    rng = np.random.default_rng(31)
    Nmax, Vmax = 256, 20000
    ws = tv.argmax_workspace(Nmax, Vmax, "cuda")
    for case in range(24):
        n = int(rng.integers(1, Nmax + 1))
        V = int(rng.integers(1, Vmax + 1))
        parent = random_tree_parent(rng, n, 16, 4) if n > 1 else np.array([-1], np.int32)
        x = rng.standard_normal((n, V)).astype(np.float32)
        etok = oracle.argmax_rows(x.astype(np.float64))
        draft = np.where(rng.random(n) < 0.7, etok, (etok + 1) % V).astype(np.int32)
        lg = torch.from_numpy(x).cuda()
        note(f"workspace reuse case {case}: N={n} V={V}")
        if case % 3 == 2:
            t = tv.argmax(lg, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(t.cpu().numpy(), etok)
        if case % 4 == 3:
            tok, (ln, nodes, _, bonus) = tv.sample_accept(lg, dev_i32(parent), dev_i32(draft), 0.7, 9, case,
                                                          workspace=ws)
        else:
            tok, (ln, nodes, _, bonus) = tv.argmax_accept(lg, dev_i32(parent), dev_i32(draft), workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(tok.cpu().numpy(), etok), case
        torch.cuda.synchronize()
        tk = tok.cpu().numpy()
        eln, enodes, _, ebonus = oracle.accept(parent, draft, tk)
        assert ln.item() == eln and nodes.cpu().numpy()[:eln].tolist() == enodes.tolist() and bonus.item() == ebonus
