"""CPU side of the seeded branch_8k trials: inputs and the oracle's results for one trial.

Runs in worker processes started with the spawn method, so it imports numpy, the input
generators and the oracle only (no torch, no GPU). The GPU side of each trial stays in the
test process.
"""

from __future__ import annotations

import os

import numpy as np

import oracle
from workloads import make


def init_worker():
    """One BLAS thread per worker: the pool itself supplies the parallelism."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: the environment limit set by the parent applies
        pass
    os.environ.setdefault("OMP_NUM_THREADS", "1")


def branch8k_trial(trial: int) -> dict:
    """Inputs of branch_8k trial ``trial`` and the oracle's attention, argmax and walk."""
    w = make("branch_8k", trial)
    ref, lse = oracle.tree_attention(oracle.bf16_bits_to_f64(w.q), oracle.bf16_bits_to_f64(w.k),
                                     oracle.bf16_bits_to_f64(w.v), w.parent, w.scale)
    tok = oracle.argmax_rows(oracle.bf16_bits_to_f64(w.logits))
    ln, nodes, toks, bonus = oracle.accept(w.parent, w.draft, tok)
    return dict(trial=trial, L=w.L, scale=w.scale, q=w.q, k=w.k, v=w.v, logits=w.logits, parent=w.parent,
                draft=w.draft, planted_len=w.planted_len, planted_end=w.planted_end, ref=ref.astype(np.float64),
                lse=lse, tok=tok, accept_len=ln, nodes=nodes, tokens=toks, bonus=bonus)
