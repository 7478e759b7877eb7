"""Pins for the oracle's acceptance walk.

* brute force: enumerate every root-to-node path, keep those whose nodes all match, pick
  the longest (lowest end index on ties) -- on hypothesis-generated trees up to 12 nodes;
* facts: a fully wrong draft accepts nothing; a draft equal to the maxima everywhere
  accepts the full depth; planted workloads accept exactly the planted length;
* hand-worked cases stored in tests/golden/accept_cases.json.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import CONFIGS, accept_trial, chain_parent, kary_bfs_parent, make

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.json")


def brute_accept(parent, draft, tok):
    n = len(parent)
    best_len, best_end = 0, -1
    for u in range(n):
        path = []
        x = u
        while x >= 0:
            path.append(x)
            x = int(parent[x])
        path.reverse()
        if all(draft[a] == tok[a] for a in path):
            if len(path) > best_len:          # strictly longer; equal length keeps lower u
                best_len, best_end = len(path), u
    nodes = []
    x = best_end
    while x >= 0:
        nodes.append(x)
        x = int(parent[x])
    nodes.reverse()
    kids = [c for c in range(n) if parent[c] == best_end]
    bonus = tok[kids[0]] if kids else -1
    return best_len, nodes, [draft[a] for a in nodes], bonus


@st.composite
def tree_and_tokens(draw):
    n = draw(st.integers(1, 12))
    parent = [-1] + [draw(st.integers(-1, i - 1)) for i in range(1, n)]
    tok = draw(st.lists(st.integers(0, 3), min_size=n, max_size=n))
    draft = draw(st.lists(st.integers(0, 3), min_size=n, max_size=n))
    return np.array(parent), np.array(draft), np.array(tok)


@settings(max_examples=600, deadline=None)
@given(tree_and_tokens())
def test_accept_matches_bruteforce(case):
    parent, draft, tok = case
    got = oracle.accept(parent, draft, tok)
    exp = brute_accept(parent.tolist(), draft.tolist(), tok.tolist())
    assert got[0] == exp[0]
    assert got[1].tolist() == exp[1]
    assert got[2].tolist() == exp[2]
    assert got[3] == exp[3]


@pytest.mark.parametrize("parent", [chain_parent(16), kary_bfs_parent(256, 4),
                                    np.array([-1, -1, 0, 1, 1, 4])])
def test_fully_wrong_draft_accepts_nothing(parent):
    n = len(parent)
    tok = np.arange(n)
    draft = tok + 1
    ln, nodes, toks, bonus = oracle.accept(parent, draft, tok)
    assert ln == 0 and nodes.size == 0 and toks.size == 0
    assert bonus == tok[0]          # node 0 is always the first child of the prefix


@pytest.mark.parametrize("parent,depth,end", [(chain_parent(16), 16, 15),
                                              (kary_bfs_parent(256, 4), 4, 84),
                                              (np.array([-1, -1, 0, 1, 1, 4]), 3, 5)])
def test_all_match_accepts_full_depth(parent, depth, end):
    tok = np.arange(len(parent)) * 7
    ln, nodes, toks, bonus = oracle.accept(parent, tok.copy(), tok)
    assert ln == depth and nodes[-1] == end
    assert toks.tolist() == tok[nodes].tolist()


def test_golden_hand_worked_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        ln, nodes, toks, bonus = oracle.accept(c["parent"], c["draft"], c["tok"])
        assert ln == c["accept_len"], c["name"]
        assert nodes.tolist() == c["nodes"], c["name"]
        assert toks.tolist() == c["tokens"], c["name"]
        assert bonus == c["bonus"], c["name"]


@pytest.mark.parametrize("name", ["tiny_chain", "branch_8k", "wide_tree", "budget22",
                                  "max_256k", "decode_1node"])
def test_planted_length_is_accepted(name):
    for trial in range(40):
        parent, draft, tok, plen, pend = accept_trial(name, trial)
        ln, nodes, _, _ = oracle.accept(parent, draft, tok)
        assert ln == plen
        if plen:
            assert nodes[-1] == pend


@pytest.mark.parametrize("name", ["tiny_chain", "budget22"])
def test_planted_logits_give_planted_acceptance(name):
    """With real logits rows the oracle's argmax reproduces the planted path."""
    for trial in range(5):
        w = make(name, trial, parts=("tree", "logits"))
        x = w.logits if w.logits_dtype == "f32" else oracle.bf16_bits_to_f64(w.logits)
        tok = oracle.argmax_rows(x)
        assert (tok[w.matched] == w.draft[w.matched]).all()
        assert (tok[~w.matched] != w.draft[~w.matched]).all()
        ln, nodes, _, _ = oracle.accept(w.parent, w.draft, tok)
        assert ln == w.planted_len


def test_wide_tree_all_match_variant():
    w = make("wide_tree", 0, parts=("tree",), plant="all")
    ln, nodes, _, _ = oracle.accept(w.parent, w.draft, w.draft)
    assert ln == 4 and nodes.tolist() == [0, 4, 20, 84]
    assert CONFIGS["wide_tree"]["N"] == 256
