"""Pins of the oracle's KV commit (accepted path -> rows after the context).

The pin that does not restate the definition: attention of the accepted nodes over the
tree (before the commit) must equal plain causal attention of the same queries over the
committed cache, because an accepted node sees exactly the context and the nodes before
it on its path -- which the commit lays out as consecutive rows.
"""

import numpy as np
import pytest

import oracle
from workloads import chain_parent, random_tree_parent


def _rand(rng, shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("seed", range(12))
def test_commit_then_causal_equals_tree_attention(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 30))
    L = int(rng.integers(0, 40))
    hq, hkv, d = 4, 2, 8
    parent = random_tree_parent(rng, n, max_depth=8, max_branch=3)
    q = _rand(rng, (n, hq, d))
    k = _rand(rng, (L + n, hkv, d))
    v = _rand(rng, (L + n, hkv, d))
    # accept a random eligible path: all nodes match, then take the lowest deepest path
    tok = rng.integers(0, 3, n)
    draft = np.where(rng.random(n) < 0.75, tok, (tok + 1) % 3)
    m, nodes, _, _ = oracle.accept(parent, draft, tok)
    out_tree, lse_tree = oracle.tree_attention(q, k, v, parent, 0.3)
    k2, v2 = oracle.kv_commit(k, v, L, nodes)
    if m == 0:
        assert np.array_equal(k2, k) and np.array_equal(v2, v)
        return
    out_chain, lse_chain = oracle.tree_attention(q[nodes], k2[:L + m], v2[:L + m], chain_parent(m), 0.3)
    np.testing.assert_allclose(out_chain, out_tree[nodes], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_chain, lse_tree[nodes], rtol=0, atol=1e-12)


def test_identity_for_an_accepted_prefix_of_a_chain():
    rng = np.random.default_rng(1)
    k = _rand(rng, (20, 2, 4))
    v = _rand(rng, (20, 2, 4))
    k2, v2 = oracle.kv_commit(k, v, 12, np.arange(5))
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_rows_outside_the_commit_are_untouched_and_bits_are_copied():
    k = np.arange(10 * 3, dtype=np.uint16).reshape(10, 3)
    v = k[::-1].copy()
    k2, v2 = oracle.kv_commit(k, v, 4, [1, 3, 5])
    assert k2[:4].tolist() == k[:4].tolist()
    assert k2[4:7].tolist() == k[[5, 7, 9]].tolist()
    assert v2[4:7].tolist() == v[[5, 7, 9]].tolist()
    assert k2[7:].tolist() == k[7:].tolist() and k2.dtype == np.uint16


def test_rejects_bad_paths():
    k = np.zeros((8, 1))
    for bad in ([2, 1], [0, 0], [-1], [4]):
        with pytest.raises(ValueError):
            oracle.kv_commit(k, k, 4, bad)


def test_mutant_without_reordering_breaks_the_causal_pin():
    """Copying the accepted rows without moving them (or in reverse) fails the pin."""
    rng = np.random.default_rng(5)
    n, L = 6, 5
    parent = np.array([-1, -1, 1, 1, 3, 4], dtype=np.int32)
    q, k, v = _rand(rng, (n, 2, 4)), _rand(rng, (L + n, 1, 4)), _rand(rng, (L + n, 1, 4))
    nodes = np.array([1, 3, 4, 5])
    out_tree, _ = oracle.tree_attention(q, k, v, parent, 0.5)
    for wrong in (nodes[::-1].copy(), np.arange(4)):
        kk, vv = k.copy(), v.copy()
        kk[L:L + 4], vv[L:L + 4] = k[L + wrong], v[L + wrong]
        out_chain, _ = oracle.tree_attention(q[nodes], kk[:L + 4], vv[:L + 4], chain_parent(4), 0.5)
        assert np.abs(out_chain - out_tree[nodes]).max() > 1e-3
