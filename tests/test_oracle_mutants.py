"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of the oracle with one deliberate slip (a dropped term, a
wrong index, a sign, a transposed choice). The test asserts that the independent pins used
in test_oracle_pins.py / test_accept_oracle.py reject every mutant, so a correct result
from the real oracle is evidence rather than coincidence. All of this runs on the CPU.
"""

import math

import numpy as np
import pytest

import oracle
from tests.test_accept_oracle import brute_accept
from tests.test_oracle_pins import all_trees, brute_attention, rand_qkv


def _attn_mutant(kind):
    def f(q, k, v, parent, scale):
        n, hq, d = q.shape
        t, hkv, _ = k.shape
        L = t - n
        g = hq // hkv
        _, anc = oracle.tree_structure(parent)
        mask = np.zeros((n, t), dtype=bool)
        mask[:, :L] = True
        mask[:, L:] = anc
        if kind == "no_self":
            mask[:, L:] &= ~np.eye(n, dtype=bool)
            mask[np.arange(n), L + np.arange(n)] = False
            mask[:, :L] = True
        if kind == "no_tree_keys":
            mask[:, L:] = np.eye(n, dtype=bool)
        if kind == "anc_transposed":
            mask[:, L:] = anc.T
        out = np.empty((n, hq, d))
        lse = np.empty((n, hq))
        for h in range(hq):
            kvh = (h % hkv) if kind == "gqa_interleaved" else h // g
            sc = -scale if kind == "neg_scale" else scale
            s = sc * (q[:, h] @ k[:, kvh].T)
            s = np.where(mask, s, -np.inf)
            mx = s.max(1, keepdims=True)
            p = np.exp(s - mx)
            z = p.sum(1, keepdims=True)
            if kind == "no_normalise":
                z = np.ones_like(z)
            out[:, h] = (p @ v[:, kvh]) / z
            lse[:, h] = mx[:, 0] + np.log(z[:, 0])
        return out, lse
    return f


def _attention_pins_pass(fn):
    rng = np.random.default_rng(99)
    for n in (1, 2, 3):
        for parent in all_trees(n):
            q, k, v = rand_qkv(rng, n, 3, 4, 2, 4)
            o, s = fn(q, k, v, parent, 0.6)
            bo, bs = brute_attention(q.tolist(), k.tolist(), v.tolist(), parent, 0.6)
            if not (np.allclose(o, bo, atol=1e-12, rtol=0) and np.allclose(s, bs, atol=1e-12, rtol=0)):
                return False
    return True


def test_real_oracle_passes():
    assert _attention_pins_pass(oracle.tree_attention)


@pytest.mark.parametrize("kind", ["no_self", "no_tree_keys", "anc_transposed",
                                  "gqa_interleaved", "neg_scale", "no_normalise"])
def test_attention_mutants_rejected(kind):
    assert not _attention_pins_pass(_attn_mutant(kind))


def _accept_mutant(kind):
    def f(parent, draft, tok):
        p = np.asarray(parent)
        n = len(p)
        depth, _ = oracle.tree_structure(p)
        ok = np.asarray(draft) == np.asarray(tok)
        elig = np.zeros(n, dtype=bool)
        for i in range(n):
            if kind == "ignore_parent":
                elig[i] = ok[i]
            else:
                elig[i] = ok[i] and (p[i] < 0 or elig[p[i]])
        if not elig.any():
            return 0, np.array([], dtype=int), np.array([], dtype=int), -1
        if kind == "greedy_first_child":
            # walk from the prefix, always taking the first matching child
            path, u = [], -1
            while True:
                kids = [c for c in range(n) if p[c] == u and ok[c]]
                if not kids:
                    break
                u = kids[0]
                path.append(u)
            nodes = np.array(path)
        else:
            cands = [i for i in range(n) if elig[i] and depth[i] == depth[elig].max()]
            end = max(cands) if kind == "highest_end" else min(cands)
            nodes, u = [], end
            while u >= 0:
                nodes.append(u)
                u = p[u]
            nodes = np.array(nodes[::-1])
        return len(nodes), nodes, np.asarray(draft)[nodes], -1
    return f


def _accept_pins_pass(fn):
    rng = np.random.default_rng(5)
    for _ in range(400):
        n = int(rng.integers(1, 10))
        parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
        draft = rng.integers(0, 2, n)
        tok = rng.integers(0, 2, n)
        got = fn(np.array(parent), draft, tok)
        exp = brute_accept(parent, draft.tolist(), tok.tolist())
        if got[0] != exp[0] or list(got[1]) != exp[1]:
            return False
    return True


def test_real_accept_passes():
    assert _accept_pins_pass(oracle.accept)


@pytest.mark.parametrize("kind", ["ignore_parent", "greedy_first_child", "highest_end"])
def test_accept_mutants_rejected(kind):
    assert not _accept_pins_pass(_accept_mutant(kind))
