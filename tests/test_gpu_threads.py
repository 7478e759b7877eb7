"""First calls from two host threads at once, on two streams of one GPU.

The library keeps per-device state filled in on first use (the compute-unit count and each
attention kernel's large-LDS launch attribute). A fresh process, so that the calls really
are the first ones, starts two threads that meet at a barrier and then call
``tv_tree_attn`` (every kernel variant: one, two, four and eight row-waves, bf16 and FP8
caches) on their own streams at the same time; every output must match the oracle.
"""

import os
import subprocess
import sys
import textwrap

import pytest
import torch

pytestmark = pytest.mark.gpu

SCRIPT = textwrap.dedent(r'''
    import sys, threading
    import numpy as np
    import torch
    import draft_tree_verification_tv_amd as tv
    import oracle
    from tests.gpu_util import check_attention, dev_bf16, dev_i32
    from workloads import make

    # one workload per kernel variant: 8 rows (1 row-wave), 64 (2), 88 (4), 256 (8)
    cases = [("decode_1node", dict(L=4000)), ("tiny_chain", {}), ("budget22", {}), ("branch_8k", dict(L=1500))]
    inputs = []
    for name, ov in cases:
        w = make(name, 2, **ov)
        q, k, v = (oracle.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v))
        ref, _ = oracle.tree_attention(q, k, v, w.parent, w.scale)
        codes_k, e_k = oracle.quantize_kv(w.k)
        codes_v, e_v = oracle.quantize_kv(w.v)
        ref8, _ = oracle.tree_attention(q, oracle.dequantize_kv(codes_k, e_k), oracle.dequantize_kv(codes_v, e_v),
                                        w.parent, w.scale)
        inputs.append((name, w, ref, (codes_k, e_k, codes_v, e_v), ref8))
    dev = [(dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.parent),
            torch.from_numpy(c[0]).cuda(), dev_i32(c[1]), torch.from_numpy(c[2]).cuda(), dev_i32(c[3]))
           for _, w, _, c, _ in inputs]
    torch.cuda.synchronize()
    barrier = threading.Barrier(2)
    results, errors = {}, []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                barrier.wait()
                outs = []
                for (name, w, _, _, _), (q, k, v, p, ck, ek, cv, ev) in zip(inputs, dev):
                    outs.append(tv.tree_attn(q, k, v, p, L=w.L, scale=w.scale))
                    outs.append(tv.tree_attn_fp8(q, ck, cv, ek, ev, p, L=w.L, scale=w.scale))
            s.synchronize()
            results[tid] = outs
        except Exception as exc:  # reported by the main thread
            errors.append(f"thread {tid}: {exc!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for tid in range(2):
        for i, (name, w, ref, _, ref8) in enumerate(inputs):
            check_attention(results[tid][2 * i], ref, label=f"thread {tid} {name} bf16")
            check_attention(results[tid][2 * i + 1], ref8, label=f"thread {tid} {name} fp8")
    print("two-thread first calls ok", flush=True)
''')


def test_concurrent_first_calls_from_two_threads(repo_root):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ)
    env["PYTHONPATH"] = repo_root + os.pathsep + env.get("PYTHONPATH", "")
    res = subprocess.run([sys.executable, "-c", SCRIPT], cwd=repo_root, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "two-thread first calls ok" in res.stdout
