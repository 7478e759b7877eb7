"""Plain float64 CPU oracle for verifying a speculative draft tree (test infrastructure).

What is computed, and where the pages state it:

* Speculative decoding: a small drafter guesses a block of tokens, the target model checks
  the whole block in one pass, keeps the tokens it agrees with and discards the rest --
  DFlash contributor guide (discosf.com/news/4742660), section "What is DFlash?"; the
  Lucebox-Hub review (aichain-blog.pages.dev), section "2. DFlash".
* The block is a tree (DDTree tree verification) scored by the target in one forward
  pass -- Lucebox-Hub review, section "2. DFlash"; Lucebox Hub tips page
  (d9249.github.io/tips/lucebox-hub), section "Lucebox Hub overview".
* Greedy acceptance compares each draft with the target's temperature-0 sample, which is
  the argmax of the logits -- DFlash contributor guide, section "Coding conventions"
  (``sample(logits, temperature=0.0)``).

The one-pass tree forward is read as masked softmax attention: every draft node attends to
the whole committed context plus itself and its ancestors in the tree. Readings taken where
the pages are silent (each one is pinned by a test under ``tests/``):

* ``parent[i]`` lies in ``[-1, i-1]``; ``-1`` hangs node i under the committed prefix (an
  implicit root that is not a node). Node order is therefore topological.
* The tree nodes' own keys and values follow the context in the cache: rows ``L..L+N-1``.
* Query head h reads KV head ``h // (Hq // Hkv)`` (contiguous grouping).
* Logits row i is the target's distribution for the token at node i; node i matches when
  ``draft[i] == argmax(logits[i])``, ties going to the lowest index.
* The accepted path is the longest root-to-node path whose nodes all match; among equally
  long paths the one ending at the lowest node index wins.
* The optional bonus token is the maximum of the first child row of the accepted end node
  (of the implicit root if nothing is accepted), or -1 when that node has no child.

Everything is float64 except the integer walk. bf16 inputs are widened exactly.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def validate_parent(parent) -> np.ndarray:
    """Return ``parent`` as int64 after checking ``-1 <= parent[i] < i`` for every node."""
    p = np.asarray(parent, dtype=np.int64)
    if p.ndim != 1 or p.size < 1:
        raise ValueError("parent must be a non-empty 1-D array")
    idx = np.arange(p.size)
    bad = (p < -1) | (p >= idx)
    if bad.any():
        raise ValueError(f"parent[{int(np.nonzero(bad)[0][0])}] out of range [-1, i-1]")
    return p


def tree_structure(parent):
    """Depth and ancestor sets of every node.

    ``depth[i]`` counts the nodes on the path from the implicit root to i (1 for a child
    of the committed prefix). ``anc[i, j]`` is True when j is i or an ancestor of i.
    """
    p = validate_parent(parent)
    n = p.size
    depth = np.zeros(n, dtype=np.int64)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if p[i] >= 0:
            anc[i] = anc[p[i]]
            depth[i] = depth[p[i]] + 1
        else:
            depth[i] = 1
        anc[i, i] = True
    return depth, anc


def anc_bitmask_words(parent, words: int = 4) -> np.ndarray:
    """Ancestor sets packed as little-endian 64-bit words: bit j of row i = anc[i, j]."""
    _, anc = tree_structure(parent)
    n = anc.shape[0]
    if n > 64 * words:
        raise ValueError("too many nodes for the word count")
    out = np.zeros((n, words), dtype=np.uint64)
    for i in range(n):
        for j in np.nonzero(anc[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def visibility_mask(parent, L: int) -> np.ndarray:
    """Boolean ``[N, L+N]``: node i sees every context key and the tree keys of anc[i]."""
    _, anc = tree_structure(parent)
    n = anc.shape[0]
    mask = np.zeros((n, L + n), dtype=bool)
    mask[:, :L] = True
    mask[:, L:] = anc
    return mask


def tree_attention(q, k, v, parent, scale: float):
    """Masked softmax attention of N tree nodes over context + tree keys, in float64.

    q: ``[N, Hq, D]``; k, v: ``[L+N, Hkv, D]`` (context rows first, then the tree nodes in
    node order). Returns ``out [N, Hq, D]`` and the natural-log ``lse [N, Hq]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    t, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    L = t - n
    if L < 0:
        raise ValueError("cache shorter than the tree")
    group = hq // hkv
    mask = visibility_mask(parent, L)
    out = np.empty((n, hq, d))
    lse = np.empty((n, hq))
    for h in range(hq):
        kvh = h // group
        s = scale * (q[:, h, :] @ k[:, kvh, :].T)
        s = np.where(mask, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        z = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ v[:, kvh, :]) / z
        lse[:, h] = mx[:, 0] + np.log(z[:, 0])
    return out, lse


def argmax_rows(logits) -> np.ndarray:
    """Index of each row's maximum; the first occurrence wins ties (numpy's rule)."""
    x = np.asarray(logits, dtype=np.float64)
    return np.argmax(x, axis=1).astype(np.int64)


def accept(parent, draft, tok):
    """Longest accepted path of the draft tree.

    Returns ``(accept_len, nodes, tokens, bonus)``: nodes root-to-leaf, tokens the drafts
    on them, bonus as described in the module docstring.
    """
    p = validate_parent(parent)
    draft = np.asarray(draft, dtype=np.int64)
    tok = np.asarray(tok, dtype=np.int64)
    depth, _ = tree_structure(p)
    n = p.size
    eligible = np.zeros(n, dtype=bool)
    for i in range(n):  # parents come first
        eligible[i] = bool(draft[i] == tok[i]) and (p[i] < 0 or bool(eligible[p[i]]))
    if eligible.any():
        best = depth[eligible].max()
        end = int(min(i for i in range(n) if eligible[i] and depth[i] == best))
        nodes = []
        u = end
        while u >= 0:
            nodes.append(u)
            u = int(p[u])
        nodes.reverse()
    else:
        end = -1
        nodes = []
    children = [c for c in range(n) if p[c] == end]
    bonus = int(tok[min(children)]) if children else -1
    nodes = np.array(nodes, dtype=np.int64)
    return len(nodes), nodes, draft[nodes], bonus


def kv_commit(k, v, L: int, nodes):
    """Key/value cache after committing an accepted path.

    The verify rule keeps the drafted tokens the target agreed with and drops the rest
    (DFlash contributor guide, section "What is DFlash?"); on a tree the kept tokens are
    the accepted root-to-node path. Their keys and values therefore move to the rows
    right after the context, in path order: new row ``L + j`` is old row ``L + nodes[j]``
    for ``j < len(nodes)``; every other row is unchanged (rows past ``L + len(nodes)`` are
    no longer part of the committed sequence). ``k``, ``v``: arrays ``[T, ...]`` whose rows
    ``L + i`` hold tree node i; values are copied bit for bit. Returns new arrays.
    """
    nodes = np.asarray(nodes, dtype=np.int64)
    n = k.shape[0] - L
    if nodes.size and (nodes.min() < 0 or nodes.max() >= n or np.any(np.diff(nodes) <= 0)):
        raise ValueError("nodes must be increasing tree node indices")
    k2, v2 = np.array(k, copy=True), np.array(v, copy=True)
    rows = L + nodes
    k2[L:L + nodes.size] = k[rows]
    v2[L:L + nodes.size] = v[rows]
    return k2, v2


def verify(q, k, v, parent, scale, logits, draft):
    """The whole step: attention output, row maxima and the acceptance result."""
    out, lse = tree_attention(q, k, v, parent, scale)
    tok = argmax_rows(logits)
    return out, lse, tok, accept(parent, draft, tok)
