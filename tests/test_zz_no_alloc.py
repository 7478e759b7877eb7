"""The allocation-free tree attention against the workspace entry point it mirrors.

tv_tree_attn_noalloc runs tv_tree_attn's kernels with the split partials in the library's
static per-device buffer instead of a caller workspace, so on the same inputs its outputs
must equal tv_tree_attn's bit for bit (and so meet the oracle's attention tolerance). Two
calls in a row, the second with a smaller input, check that a call does not depend on what
the previous one left in the shared buffer; a request larger than the buffer is refused
before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import check_attention, dev_bf16, dev_i32, note
from workloads import make

pytestmark = pytest.mark.gpu

tv = pytest.importorskip("draft_tree_verification_tv_amd")


def run_both(w, num_splits=0):
    q, k, v, parent = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.parent)
    lse_a = torch.empty((w.N, w.Hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = tv.tree_attn(q, k, v, parent, L=w.L, scale=w.scale, num_splits=num_splits, lse=lse_a)
    b = tv.tree_attn_noalloc(q, k, v, parent, L=w.L, scale=w.scale, num_splits=num_splits, lse=lse_b,
                             dev_error=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    return a, lse_a, b, lse_b


def check_case(w, label, num_splits=0):
    note(f"noalloc {label}: N={w.N} L={w.L} Hq={w.Hq} Hkv={w.Hkv} splits={num_splits}")
    a, lse_a, b, lse_b = run_both(w, num_splits)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{label}: output differs from tv_tree_attn"
    assert torch.equal(lse_a, lse_b), f"{label}: lse differs from tv_tree_attn"
    ref, lse_ref = oracle.tree_attention(oracle.bf16_bits_to_f64(w.q), oracle.bf16_bits_to_f64(w.k),
                                         oracle.bf16_bits_to_f64(w.v), w.parent, w.scale)
    check_attention(b, ref, lse_b, lse_ref, label)


def test_noalloc_matches_workspace_entry_point_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()
    # first call: the 8K branching tree (256 rows per KV head, 256 workgroups of partials);
    # second, smaller: the 22-node budget tree over a ragged 1000-token context
    check_case(make("branch_8k", 7), "branch_8k")
    check_case(make("budget22", 4), "budget22")
    # and back up with a forced split count (more partials than either call above)
    check_case(make("tiny_chain", 3), "tiny_chain", num_splits=9)


def test_noalloc_refuses_more_than_its_buffer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = make("budget22", 0, parts=("tree",))
    L, N, Hq, Hkv = 131072, w.N, 32, 8
    need = tv.tree_attn_workspace_size(N, L, Hq, Hkv, 128, 1024)
    assert need > tv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((N, Hq, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((L + N, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tv.TVError) as ei:
        tv.tree_attn_noalloc(q, kv, kv, dev_i32(w.parent), L=L, num_splits=1024)
    assert ei.value.status == tv.TV_ERR_WORKSPACE
