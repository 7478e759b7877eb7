"""Sampled verification (temperature > 0) for the CPU oracle (test infrastructure only).

The target's token for a node is a sample from softmax(logits / T) -- the pages' sampling
call takes a temperature, with 0 meaning the argmax (DFlash contributor guide, section
"Coding conventions"). The sample is drawn with the Gumbel-max construction: the index of
the largest logit / T + G, with G = -ln(-ln u) standard Gumbel noise, is distributed as
softmax(logits / T). The uniforms u come from the counter-based generator Philox-4x32-10
(Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011),
written here from that definition, so that any two implementations draw the same numbers
for the same (seed, counter). Drafts are then accepted exactly as in greedy verification
(longest path of nodes whose draft equals the target's token).

Counter layout: key = (seed low 32 bits, seed high 32 bits); counter = (v // 4, node,
offset low 32 bits, offset high 32 bits); word v % 4 of the output gives the uniform for
vocabulary index v from its top 23 bits: u = ((word >> 9) + 0.5) / 2^23, strictly inside
(0, 1) and exactly representable in float32 (at most 24 significant bits), so every
implementation draws the same u.
"""

from __future__ import annotations

import numpy as np

from .tree_verify import accept

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox-4x32 with 10 rounds on uint32 arrays.

    ``counter``: four arrays (or scalars) c0..c3; ``key``: two arrays k0, k1. Returns the
    four output words as uint64 arrays holding 32-bit values. One round multiplies c0 and
    c2 by the two round constants (full 64-bit products), then outputs
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key is bumped by
    the two Weyl constants between rounds.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in counter)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & MASK32 for k in key)
    for _ in range(10):
        p0 = c0 * np.uint64(PHILOX_M0)        # < 2^64: exact in uint64
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(PHILOX_W0)) & np.uint64(MASK32)
        k1 = (k1 + np.uint64(PHILOX_W1)) & np.uint64(MASK32)
    return c0, c1, c2, c3


def uniforms(n_nodes: int, V: int, seed: int, offset: int) -> np.ndarray:
    """u[i, v] in (0, 1) for node i and vocabulary index v (float64)."""
    v = np.arange(V, dtype=np.uint64)
    out = np.empty((n_nodes, V), dtype=np.float64)
    key = (np.uint64(seed & MASK32), np.uint64((seed >> 32) & MASK32))
    for i in range(n_nodes):
        words = philox4x32_10((v // np.uint64(4), np.uint64(i), np.uint64(offset & MASK32),
                               np.uint64((offset >> 32) & MASK32)), key)
        w = np.choose((v % np.uint64(4)).astype(np.int64), words)
        out[i] = ((w >> np.uint64(9)).astype(np.float64) + 0.5) / 8388608.0
    return out


def sample_rows(logits, temperature: float, seed: int, offset: int) -> np.ndarray:
    """tok[i] = argmax_v(logits[i, v] / T + G[i, v]) with Gumbel noise from Philox."""
    x = np.asarray(logits, dtype=np.float64)
    if not (temperature > 0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")
    u = uniforms(x.shape[0], x.shape[1], seed, offset)
    g = -np.log(-np.log(u))
    return np.argmax(x / temperature + g, axis=1).astype(np.int64)


def sample_accept(parent, draft, logits, temperature: float, seed: int, offset: int):
    """Sampled targets and the accepted path: (tok, (len, nodes, tokens, bonus))."""
    tok = sample_rows(logits, temperature, seed, offset)
    return tok, accept(parent, draft, tok)
