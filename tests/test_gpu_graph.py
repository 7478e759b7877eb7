"""The verify step captured in a HIP graph: every replay against the oracle and the eager run.

Every entry point only enqueues kernels on the caller's stream (no memsets, no host
synchronisation, no allocation), so a whole verify step -- tree attention for several
layers, argmax + accept, and the KV commit -- can be captured once and replayed. Each
replay must match the CPU oracle (attention within the attention tolerance; tokens, the
accepted path and the committed cache bit for bit) and reproduce the eager outputs bit for
bit; eager work runs between replays.
"""

import numpy as np
import pytest
import torch

import draft_tree_verification_tv_amd as tv
import oracle
from tests.gpu_util import check_attention, dev_bf16, dev_i32, note
from workloads import make


def oracle_step(w, layers):
    """The oracle's results for the captured step: per-layer attention on the rolled
    caches (the same rolls as the device copies), argmax, walk and the committed cache."""
    q = oracle.bf16_bits_to_f64(w.q)
    outs = []
    for i in range(layers):
        k = oracle.bf16_bits_to_f64(np.roll(w.k, i, axis=0))
        v = oracle.bf16_bits_to_f64(np.roll(w.v, 2 * i, axis=0))
        outs.append(oracle.tree_attention(q, k, v, w.parent, w.scale)[0])
    tok = oracle.argmax_rows(oracle.bf16_bits_to_f64(w.logits))
    acc = oracle.accept(w.parent, w.draft, tok)
    kc, vc = oracle.kv_commit(w.k, w.v, w.L, acc[1])  # bit patterns move unchanged
    return outs, tok, acc, kc, vc


def check_against_oracle(got, exp, w, label):
    outs, tok, acc, kc, vc, new_len = got
    e_outs, e_tok, (e_len, e_nodes, e_toks, e_bonus), e_kc, e_vc = exp
    for i, (o, r) in enumerate(zip(outs, e_outs)):
        check_attention(o, r, label=f"{label} layer {i}")
    assert np.array_equal(tok.numpy(), e_tok), f"{label}: tokens"
    ln = int(acc[0].item())
    assert ln == e_len == w.planted_len, f"{label}: accept_len"
    assert acc[1].numpy()[:ln].tolist() == e_nodes.tolist(), f"{label}: path"
    assert acc[2].numpy()[:ln].tolist() == e_toks.tolist(), f"{label}: path tokens"
    assert int(acc[3].item()) == e_bonus, f"{label}: bonus"
    assert np.array_equal(kc.view(torch.int16).numpy().view(np.uint16), e_kc), f"{label}: K commit"
    assert np.array_equal(vc.view(torch.int16).numpy().view(np.uint16), e_vc), f"{label}: V commit"
    assert int(new_len.item()) == w.L + e_len

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["budget22", "branch_8k", "decode_1node"])
def test_graph_replays_match_oracle_and_eager(name):
    w = make(name, 1)
    note(f"graph capture {name}")
    layers = 3
    q = dev_bf16(w.q)
    ks = [dev_bf16(w.k) for _ in range(layers)]
    vs = [dev_bf16(w.v) for _ in range(layers)]
    for i in range(1, layers):          # distinct layers
        ks[i].copy_(torch.roll(ks[0], shifts=i, dims=0))
        vs[i].copy_(torch.roll(vs[0], shifts=2 * i, dims=0))
    parent, draft, logits = dev_i32(w.parent), dev_i32(w.draft), dev_bf16(w.logits)
    outs = [torch.empty((w.N, w.Hq, w.D), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    ws = torch.empty(tv.tree_attn_workspace_size(w.N, w.L, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device="cuda")
    am_ws = tv.argmax_workspace(w.N, w.V, "cuda")
    tok = torch.empty(w.N, dtype=torch.int32, device="cuda")
    acc = tuple(torch.empty(n, dtype=torch.int32, device="cuda") for n in (1, w.N, w.N, 1))
    kc, vc = ks[0].clone(), vs[0].clone()   # cache the commit writes into
    new_len = torch.empty(1, dtype=torch.int32, device="cuda")

    def step():
        for i in range(layers):
            tv.tree_attn(q, ks[i], vs[i], parent, L=w.L, scale=w.scale, out=outs[i], workspace=ws)
        tv.argmax_accept(logits, parent, draft, tok=tok, out=acc, workspace=am_ws)
        tv.kv_commit(kc, vc, w.L, acc[0], acc[1], new_len=new_len)

    def snapshot():
        return ([o.cpu().clone() for o in outs], tok.cpu().clone(), [a.cpu().clone() for a in acc],
                kc.cpu().clone(), vc.cpu().clone(), new_len.cpu().clone())

    def reset_cache():
        kc.copy_(ks[0])
        vc.copy_(vs[0])

    step()                                   # eager (also initialises the library)
    torch.cuda.synchronize()
    ref = snapshot()
    exp = oracle_step(w, layers)
    check_against_oracle(ref, exp, w, f"{name} eager")
    reset_cache()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:                       # scribble over the outputs between replays
            o.fill_(float("nan"))
        tok.fill_(-5)
        reset_cache()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        check_against_oracle(got, exp, w, f"{name} replay {rep}")
        for a, b in zip(got[0], ref[0]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: attention"
        assert torch.equal(got[1], ref[1]), f"replay {rep}: tokens"
        for a, b in zip(got[2], ref[2]):
            assert torch.equal(a, b), f"replay {rep}: accept"
        assert torch.equal(got[3].view(torch.int16), ref[3].view(torch.int16)), f"replay {rep}: K commit"
        assert torch.equal(got[4].view(torch.int16), ref[4].view(torch.int16)), f"replay {rep}: V commit"
        assert torch.equal(got[5], ref[5])
        # eager work between replays
        tv.tree_attn(q, ks[1], vs[1], parent, L=w.L, scale=w.scale)
    assert int(ref[2][0].item()) == w.planted_len
    assert int(ref[5].item()) == w.L + w.planted_len
