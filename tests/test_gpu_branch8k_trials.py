"""The branch_8k workload's 1000 seeded trials through the real verify path.

Every trial (seed ``SeedSequence([42, 1, trial])``; 42 is the benchmark seed of the DFlash
contributor guide, "Coding conventions") builds its own 64-node tree, 8K-token bf16 cache
and [64, 152064] bf16 logits with a planted path. On the GPU each trial runs

* ``tv_tree_attn`` over the cache: within the attention tolerance of the oracle, and the
  exported log-sum-exp within 1e-3;
* ``tv_argmax_accept`` on the planted logits: tokens, accepted length, path, path tokens
  and bonus bit-exact against ``oracle.argmax_rows`` + ``oracle.accept``, and the accepted
  length equal to the planted one.

The CPU side (inputs and oracle, about 0.75 s per trial on one core) runs in a pool of
spawned worker processes that import no torch; the trials are split into ten tests of 100
so that each reports on its own range.
"""

import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

from tests import trial_worker
from tests.gpu_util import check_attention, dev_bf16, dev_i32, note

pytestmark = pytest.mark.gpu

tv = pytest.importorskip("draft_tree_verification_tv_amd")

TRIALS = 1000
CHUNK = 100


@pytest.fixture(scope="module")
def pool():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()
    workers = max(1, min(12, len(os.sched_getaffinity(0)) - 2))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        p = mp.get_context("spawn").Pool(workers, initializer=trial_worker.init_worker)
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    note(f"branch_8k trials: {workers} CPU workers")
    yield p
    p.close()
    p.join()


def run_trial(c: dict, bufs: dict):
    label = f"branch_8k trial {c['trial']}"
    q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
    parent, draft, logits = dev_i32(c["parent"]), dev_i32(c["draft"]), dev_bf16(c["logits"])
    n, hq = c["q"].shape[0], c["q"].shape[1]
    lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")
    out = tv.tree_attn(q, k, v, parent, L=c["L"], scale=c["scale"], lse=lse, workspace=bufs.get("ws"))
    tok, (ln, nodes, toks, bonus) = tv.argmax_accept(logits, parent, draft, workspace=bufs.get("am_ws"))
    torch.cuda.synchronize()
    check_attention(out, c["ref"], lse, c["lse"], label)
    assert np.array_equal(tok.cpu().numpy(), c["tok"]), f"{label}: argmax"
    got_len = int(ln.item())
    assert got_len == c["accept_len"] == c["planted_len"], f"{label}: accept_len {got_len}"
    g_nodes, g_toks = nodes.cpu().numpy(), toks.cpu().numpy()
    assert g_nodes[:got_len].tolist() == c["nodes"].tolist(), f"{label}: path"
    assert g_toks[:got_len].tolist() == c["tokens"].tolist(), f"{label}: path tokens"
    assert (g_nodes[got_len:] == -1).all() and (g_toks[got_len:] == -1).all(), f"{label}: padding"
    assert int(bonus.item()) == c["bonus"], f"{label}: bonus"
    if got_len:
        assert int(g_nodes[got_len - 1]) == c["planted_end"], f"{label}: end node"
    return got_len


@pytest.mark.parametrize("first", range(0, TRIALS, CHUNK))
def test_branch_8k_trials(pool, first):
    note(f"branch_8k trials {first}..{first + CHUNK - 1}")
    bufs = {}
    lens = []
    for c in pool.imap(trial_worker.branch8k_trial, range(first, first + CHUNK)):
        if not bufs:
            n, hq = c["q"].shape[:2]
            hkv = c["k"].shape[1]
            bufs["ws"] = torch.empty(tv.tree_attn_workspace_size(n, c["L"], hq, hkv), dtype=torch.uint8,
                                     device="cuda")
            bufs["am_ws"] = tv.argmax_workspace(n, c["logits"].shape[1], "cuda")
        lens.append(run_trial(c, bufs))
    # the planted lengths are spread over the tree depths, including empty and long paths
    assert min(lens) == 0 and max(lens) >= 4, lens
