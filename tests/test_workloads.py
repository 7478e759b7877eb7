"""Properties of the seeded workload generators (CPU only)."""

import numpy as np
import pytest

import oracle
from workloads import (CONFIGS, bf16_bits_from_f32, chain_parent, kary_bfs_parent, make,
                       random_tree_parent, rng_for)


def children_counts(parent):
    n = len(parent)
    c = np.zeros(n + 1, dtype=int)          # last slot: the implicit root
    for p in parent:
        c[p] += 1
    return c


@pytest.mark.parametrize("n", [1, 2, 16, 22, 64, 256])
def test_random_tree_shape(n):
    for seed in range(60):
        p = random_tree_parent(rng_for(1, seed), n, 16, 4)
        assert len(p) == n and p[0] == -1
        assert (p < np.arange(n)).all() and (p >= -1).all()
        depth, _ = oracle.tree_structure(p)
        assert depth.max() <= 16
        assert children_counts(p).max() <= 4
        # breadth-first numbering: depth never decreases, siblings grouped by parent
        assert (np.diff(depth) >= 0).all()
        for d in range(1, depth.max() + 1):
            lvl = p[depth == d]
            assert (np.diff(lvl) >= 0).all()


def test_random_tree_deterministic_and_varied():
    a = random_tree_parent(rng_for(1, 5), 64)
    b = random_tree_parent(rng_for(1, 5), 64)
    c = random_tree_parent(rng_for(1, 6), 64)
    assert (a == b).all() and not (a == c).all()


def test_kary_and_chain():
    assert chain_parent(4).tolist() == [-1, 0, 1, 2]
    p = kary_bfs_parent(256, 4)
    assert p[:4].tolist() == [-1] * 4 and p[4] == 0 and p[84] == 20 and p[255] == 62
    assert children_counts(p)[:-1].max() == 4


def test_seeded_values_are_reproducible_bf16_normals():
    w1 = make("tiny_chain", 3)
    w2 = make("tiny_chain", 3)
    for a in ("q", "k", "v", "logits", "draft", "parent"):
        assert np.array_equal(getattr(w1, a), getattr(w2, a))
    assert w1.q.shape == (16, 8, 128) and w1.k.shape == (528, 2, 128)
    assert w1.logits.shape == (16, 4096) and w1.logits.dtype == np.float32
    x = oracle.bf16_bits_to_f64(w1.k)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_peaky_keys_are_exact_powers_of_two():
    w = make("max_256k", 0, parts=("qkv",), L=20000)
    base = make("max_256k", 0, parts=("qkv",), L=20000, peaky=False)
    ratio_rows = 0
    for h in range(w.Hkv):
        a = oracle.bf16_bits_to_f64(w.k[:, h])
        b = oracle.bf16_bits_to_f64(base.k[:, h])
        changed = np.any(a != b, axis=1)
        assert changed[20000:].sum() == 0          # tree keys untouched
        assert changed.sum() == 200                 # ceil(1% of 20000)
        assert np.array_equal(a[changed], 8 * b[changed])
        ratio_rows += changed.sum()
    assert np.array_equal(w.v, base.v)


def test_configs_cover_workloads():
    for name, c in CONFIGS.items():
        assert c["Hq"] % c["Hkv"] == 0
    assert CONFIGS["long_128k"]["L"] == 131072 and CONFIGS["max_256k"]["L"] == 262144


def test_decode_uses_wide_tree_cache():
    d = make("decode_1node", 0, parts=("qkv",), L=300)
    w = make("wide_tree", 0, parts=("qkv",), L=300)
    assert np.array_equal(d.k, w.k[:301]) and np.array_equal(d.q, w.q[:1])


def test_rne_rounding_ties():
    # 1 + 2^-8 is a tie between bf16 neighbours 1 and 1 + 2^-7: even mantissa wins (1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    assert bits.tolist() == [0x3F80, 0x3F82, 0xBF80]
