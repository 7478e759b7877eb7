"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force: pure-Python loops with math.exp / math.fsum on tiny inputs, every tree
  shape up to four nodes;
* textbook special cases through a library routine: a chain equals causal attention
  (bottom-right aligned) and a single node equals one-token decode, both through
  torch's scaled_dot_product_attention in float64 on the CPU;
* the explicit tree mask through the same library routine, with the mask built here by
  walking parent pointers;
* invariants and closed forms: context permutation, non-ancestor perturbation, constant
  values, zero queries (mean of the visible values, lse = log(count)).
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import chain_parent, kary_bfs_parent, random_tree_parent


def all_trees(n):
    """Every valid parent array with n nodes (parent[i] in [-1, i-1])."""
    return [np.array(p, dtype=np.int32)
            for p in itertools.product(*[range(-1, i) for i in range(n)])]


def brute_attention(q, k, v, parent, scale):
    """Pure-Python masked attention: visibility found by walking parent pointers."""
    n = len(parent)
    t = len(k)
    L = t - n
    hq = len(q[0])
    hkv = len(k[0])
    d = len(q[0][0])
    group = hq // hkv
    out = [[None] * hq for _ in range(n)]
    lse = [[None] * hq for _ in range(n)]
    for i in range(n):
        on_path = set()
        u = i
        while u != -1:
            on_path.add(u)
            u = int(parent[u])
        keys = list(range(L)) + [L + a for a in sorted(on_path)]
        for h in range(hq):
            kh = h // group
            sc = [scale * math.fsum(q[i][h][c] * k[j][kh][c] for c in range(d)) for j in keys]
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            z = math.fsum(w)
            out[i][h] = [math.fsum(w[a] * v[keys[a]][kh][c] for a in range(len(keys))) / z
                         for c in range(d)]
            lse[i][h] = m + math.log(z)
    return np.array(out), np.array(lse)


def rand_qkv(rng, n, L, hq, hkv, d):
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((L + n, hkv, d))
    v = rng.standard_normal((L + n, hkv, d))
    return q, k, v


@pytest.mark.parametrize("L,d,hq,hkv", [(0, 4, 2, 1), (1, 1, 1, 1), (2, 4, 4, 2),
                                        (3, 4, 2, 2), (8, 4, 4, 1)])
def test_bruteforce_all_small_trees(L, d, hq, hkv):
    rng = np.random.default_rng(1000 + L * 10 + d)
    for n in range(1, 5):
        for parent in all_trees(n):
            q, k, v = rand_qkv(rng, n, L, hq, hkv, d)
            scale = 0.7
            o, s = oracle.tree_attention(q, k, v, parent, scale)
            bo, bs = brute_attention(q.tolist(), k.tolist(), v.tolist(), parent, scale)
            np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(s, bs, rtol=0, atol=1e-12)


def test_bruteforce_head_dim_128():
    rng = np.random.default_rng(7)
    for parent in [np.array([-1, 0, 0, 1]), np.array([-1, -1, 1]), np.array([-1])]:
        n = len(parent)
        q, k, v = rand_qkv(rng, n, 5, 4, 2, 128)
        o, s = oracle.tree_attention(q, k, v, parent, 1 / math.sqrt(128))
        bo, bs = brute_attention(q.tolist(), k.tolist(), v.tolist(), parent, 1 / math.sqrt(128))
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(s, bs, rtol=0, atol=1e-12)


def sdpa(q, k, v, mask, scale):
    """torch SDPA in float64 on the CPU; q [N,Hq,D], k/v [T,Hkv,D], mask [N,T] or None."""
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)          # [Hq, N, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("L,n", [(0, 5), (17, 16), (512, 16), (100, 1)])
def test_chain_equals_causal_attention(L, n):
    """A chain of n nodes after L context tokens is causal attention over L+n positions."""
    rng = np.random.default_rng(L + n)
    q, k, v = rand_qkv(rng, n, L, 8, 2, 128)
    scale = 1 / math.sqrt(128)
    pos_q = L + np.arange(n)[:, None]
    pos_k = np.arange(L + n)[None, :]
    causal = pos_k <= pos_q                           # bottom-right aligned
    ref = sdpa(q, k, v, causal, scale)
    o, _ = oracle.tree_attention(q, k, v, chain_parent(n), scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [0, 1, 33, 4096])
def test_single_node_equals_decode(L):
    """One node under the prefix attends to all L+1 keys: plain one-token decode."""
    rng = np.random.default_rng(L)
    q, k, v = rand_qkv(rng, 1, L, 8, 4, 128)
    ref = sdpa(q, k, v, None, 0.125)
    o, _ = oracle.tree_attention(q, k, v, np.array([-1]), 0.125)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def walk_mask(parent, L):
    n = len(parent)
    m = np.zeros((n, L + n), dtype=bool)
    m[:, :L] = True
    for i in range(n):
        u = i
        while u >= 0:
            m[i, L + u] = True
            u = int(parent[u])
    return m


@pytest.mark.parametrize("seed", range(6))
def test_tree_mask_library_crosscheck(seed):
    rng = np.random.default_rng(seed)
    n = [3, 12, 22, 40, 64, 9][seed]
    L = [0, 5, 64, 300, 129, 1][seed]
    parent = random_tree_parent(rng, n, 16, 4)
    q, k, v = rand_qkv(rng, n, L, 8, 2, 128)
    ref = sdpa(q, k, v, walk_mask(parent, L), 0.088)
    o, _ = oracle.tree_attention(q, k, v, parent, 0.088)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_context_permutation_invariance():
    rng = np.random.default_rng(3)
    n, L = 21, 200
    parent = random_tree_parent(rng, n, 16, 4)
    q, k, v = rand_qkv(rng, n, L, 4, 2, 128)
    o, s = oracle.tree_attention(q, k, v, parent, 0.1)
    perm = np.concatenate([rng.permutation(L), L + np.arange(n)])
    o2, s2 = oracle.tree_attention(q, k[perm], v[perm], parent, 0.1)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-12)


def test_non_ancestor_perturbation_invariance():
    rng = np.random.default_rng(4)
    n, L = 30, 50
    parent = random_tree_parent(rng, n, 16, 4)
    depth, anc = oracle.tree_structure(parent)
    q, k, v = rand_qkv(rng, n, L, 4, 1, 128)
    o, _ = oracle.tree_attention(q, k, v, parent, 0.1)
    for i in [0, n // 2, n - 1]:
        k2, v2 = k.copy(), v.copy()
        others = [j for j in range(n) if not anc[i, j]]
        k2[L + np.array(others, dtype=int)] += 5.0
        v2[L + np.array(others, dtype=int)] -= 3.0
        o2, _ = oracle.tree_attention(q, k2, v2, parent, 0.1)
        np.testing.assert_allclose(o2[i], o[i], rtol=0, atol=1e-12)
        # an ancestor's change must show
        k3 = k.copy()
        k3[L + i] += 5.0
        o3, _ = oracle.tree_attention(q, k3, v, parent, 0.1)
        assert np.abs(o3[i] - o[i]).max() > 1e-6


def test_constant_values_give_that_value():
    rng = np.random.default_rng(5)
    n, L = 10, 40
    parent = random_tree_parent(rng, n, 16, 4)
    q, k, _ = rand_qkv(rng, n, L, 4, 2, 128)
    vec = rng.standard_normal(128)
    v = np.broadcast_to(vec, (L + n, 2, 128)).copy()
    o, _ = oracle.tree_attention(q, k, v, parent, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(vec, o.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L", [0, 7, 1000])
def test_zero_query_is_mean_of_visible_values(L):
    """q = 0 gives equal weights: out = mean of visible V rows, lse = log(L + depth)."""
    rng = np.random.default_rng(L)
    parent = kary_bfs_parent(40, 3)
    n = len(parent)
    _, k, v = rand_qkv(rng, n, L, 6, 3, 128)
    q = np.zeros((n, 6, 128))
    o, s = oracle.tree_attention(q, k, v, parent, 0.5)
    vis = walk_mask(parent, L)
    for i in range(n):
        cnt = vis[i].sum()
        for h in range(6):
            np.testing.assert_allclose(o[i, h], v[vis[i], h // 2, :].mean(axis=0), atol=1e-12)
            assert abs(s[i, h] - math.log(cnt)) < 1e-12


def test_two_key_closed_form():
    """One node, one context key: weights are the logistic of the score difference."""
    q = np.zeros((1, 1, 2))
    q[0, 0] = [1.0, 2.0]
    k = np.array([[[3.0, 0.5]], [[-1.0, 1.0]]])   # context key, then the node's own key
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    o, s = oracle.tree_attention(q, k, v, np.array([-1]), 1.0)
    s0, s1 = 4.0, 1.0
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(o[0, 0], [w0, 1 - w0], atol=1e-15)
    assert abs(s[0, 0] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-15


# --------------------------------------------------------------------- structure


def test_structure_chain_and_kary():
    d, anc = oracle.tree_structure(chain_parent(9))
    assert d.tolist() == list(range(1, 10))
    assert (anc == np.tril(np.ones((9, 9), dtype=bool))).all()
    d, anc = oracle.tree_structure(kary_bfs_parent(256, 4))
    assert np.bincount(d).tolist() == [0, 4, 16, 64, 172]
    assert (anc.sum(axis=1) == d).all()


def test_bitmask_words():
    parent = kary_bfs_parent(256, 4)
    w = oracle.anc_bitmask_words(parent)
    # node 255 = 4th level; ancestors 62, 14, 2 and itself
    expect = np.zeros(4, dtype=np.uint64)
    for j in (2, 14, 62, 255):
        expect[j // 64] |= np.uint64(1) << np.uint64(j % 64)
    assert (w[255] == expect).all()
    assert (w[0] == np.array([1, 0, 0, 0], dtype=np.uint64)).all()


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 3], [-2], [-1, -3]])
def test_validate_rejects(bad):
    with pytest.raises(ValueError):
        oracle.validate_parent(bad)


# -------------------------------------------------------------------------- argmax


def brute_argmax(row):
    best, idx = None, -1
    for j, x in enumerate(row):
        if best is None or x > best:
            best, idx = x, j
    return idx


def test_argmax_matches_brute_force_on_tie_rows():
    from workloads import tie_rows
    rng = np.random.default_rng(11)
    for dtype in ("bf16", "f32"):
        rows = tie_rows(rng, 3001, dtype)
        x = oracle.bf16_bits_to_f64(rows) if dtype == "bf16" else rows.astype(np.float64)
        got = oracle.argmax_rows(x)
        for r in range(x.shape[0]):
            assert got[r] == brute_argmax(x[r].tolist()), r
    # the hand-built rows: all-equal -> 0; +0/-0 tie -> the earlier one; both ends -> 0
    x = oracle.bf16_bits_to_f64(tie_rows(np.random.default_rng(0), 999))
    got = oracle.argmax_rows(x)
    assert got[0] == 0 and got[2] == 998 and got[3] == 999 // 3 and got[4] == 997 and got[6] == 0


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(2)
    f = rng.standard_normal(10000).astype(np.float32) * 100
    from workloads import bf16_bits_from_f32
    bits = bf16_bits_from_f32(f)
    ref = torch.from_numpy(f).to(torch.bfloat16)
    assert (ref.view(torch.int16).numpy().view(np.uint16) == bits).all()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), ref.to(torch.float64).numpy())
