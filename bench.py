#!/usr/bin/env python3
"""Benchmark: one tree-verify step on the 128K-context, 64-node workload, one GPU.

Workload (synthetic, seeded): KV length 131072 + 64 tree rows, 32 q heads / 8 KV heads,
head dim 128, bf16 N(0,1); a 64-node random tree of depth <= 16; logits [64, 152064]
bf16 with a planted path. One step = 64 back-to-back layer-equivalent tree-attention
calls, each on its own KV buffer (64 buffers, 34.4 GB, far beyond the 256 MB Infinity
Cache), then one argmax over the logits and one acceptance walk.

Reported ``value``: microseconds per tree-verify call = mean attention time per
layer-equivalent call + the time of the argmax-and-accept call (HIP events on the stream
the kernels run on). ``roofline`` relates the attention call's algorithmic bytes (K + V + Q +
out) to its measured duration against the 8 TB/s HBM peak. ``cpu_baseline`` times the
float64 CPU oracle on whole verify calls of the same workload (about 10 s of CPU work).

``--workload`` times another configuration of the workload set the same way (a profiling
aid; the default line is the 128K one). A call whose flops per algorithmic byte exceed the
ridge point of the two peaks (2.5 PFLOP/s dense bf16 over 8 TB/s, 312.5 flop/B), as for the
256-node tree, reports an MFMA roofline: 4 * nodes * q heads * keys * head dim flops per
call against the bf16 peak. ``--kv-layout head`` stores the bf16 caches head-major
([Hkv, T, D]) instead of token-major; ``--sweep`` times every configuration's attention
in the three cache formats and both layouts instead of the bench line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
       [--no-check] [--kv-layout token|head] [--sweep]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16, MI355X
LAYERS = 64
WORKLOAD = "long_128k"
CPU_SAMPLE_SECONDS = 10.0

# HBM bytes per tv_tree_attn call on this workload (split + merge kernels), from two
# rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), each calibrated against a 1 GiB device
# copy (read factor 2.0, write factor 1.0); summary in
# profiles/tv_tree_attn_long_128k_hbm_counters.md. Valid only for the kernel sources they
# were taken on (compared through a digest of their code without comments): reported as
# null once that code changes.
TRAFFIC_BYTES_PER_CALL = 572862499
TRAFFIC_SOURCES = ("draft_tree_verification_tv_amd/csrc/tv_attn.hip",
                   "draft_tree_verification_tv_amd/csrc/tv_internal.h")
TRAFFIC_SOURCES_SHA256 = "9a5c140e7d1e013ce8150203dac1510086cc6afb7a068d1ae4b33d9e54cee689"


def code_digest(root, files):
    """SHA-256 of the sources' code with // comments and blank space removed, so that a
    comment edit does not void counters taken on unchanged code."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(root, f)) as fh:
            text = re.sub(r"//[^\n]*", "", fh.read())
        h.update("".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic():
    root = os.path.dirname(os.path.abspath(__file__))
    return TRAFFIC_BYTES_PER_CALL if code_digest(root, TRAFFIC_SOURCES) == TRAFFIC_SOURCES_SHA256 else None


def measure_ceilings(K, Vc, T, Hkv, D, layers, stream, attn_call):
    """Ceilings on this machine, measured with the probe library (include/tv_probe.h):

    * ``hbm_read_gbps``: plain read streams over the layers' K and V caches (HIP events,
      best of three rounds), read (a) as one contiguous range in 4 KB rows and (b) in the
      attention call's own pattern -- one KV head's 256-byte rows every Hkv * 256 bytes,
      one workgroup per (head, key range), K and V caches in turn -- for a few range
      lengths (``kv_pattern``), and at 32 ranges per head, the attention call's grid of
      256 workgroups (``kv_pattern_attn_grid``).
    * ``shader_clock_ghz``: shader-clock cycles over real-time ticks of one spinning wave
      (rate of the real-time counter measured against HIP events while idle), with the
      chip idle, during the read stream and during back-to-back attention calls.
    """
    import numpy as np
    import torch

    from draft_tree_verification_tv_amd import probe

    dev = K.device
    row_b = D * 2
    # the layers' caches after the first (at most 8), or the first alone
    first = 1 if layers > 1 else 0
    nl = max(1, min(layers - 1, 8))
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)

    def timed_bytes(launch, nbytes, rounds=3):
        launch()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return nbytes / best / 1e9

    # (a) contiguous: layers 1 .. nl of K, then of V, 4 KB rows
    span_rows = (nl * T * Hkv * row_b) // 4096
    contiguous = {}
    for grid in (512, 1024, 2048):
        rpw = -(-span_rows // grid)

        def run_contig(rpw=rpw):
            for buf in (K, Vc):
                probe.stream_read(buf[first:first + nl], span_rows, 4096, 4096, 1, rpw, sink)
        contiguous[grid] = timed_bytes(run_contig, 2 * span_rows * 4096)

    # (b) the KV pattern: column = KV head, rows = keys
    pattern = {}
    for ranges in (32, 64, 128):
        rpw = -(-T // ranges)

        def run_kv(rpw=rpw):
            for b in range(first, first + nl):
                probe.stream_read(K[b], T, row_b, Hkv * row_b, Hkv, rpw, sink)
                probe.stream_read(Vc[b], T, row_b, Hkv * row_b, Hkv, rpw, sink)
        pattern[ranges] = timed_bytes(run_kv, 2 * nl * T * Hkv * row_b)

    # shader clock: the real-time counter's rate first (idle, 20 ms spin)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    probe.clock(clk, 2_000_000, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    cyc, ticks = (int(x) for x in clk.cpu())
    rt_hz = ticks / (e0.elapsed_time(e1) * 1e-3)
    idle_ghz = cyc / ticks * rt_hz / 1e9

    def clock_under(work_before, work_after, spin_ticks):
        clk.zero_()
        torch.cuda.synchronize()
        work_before()
        with torch.cuda.stream(side):
            probe.clock(clk, spin_ticks, side)
        work_after()
        torch.cuda.synchronize()
        c, t = (int(x) for x in clk.cpu())
        return c / t * rt_hz / 1e9

    ticks_3ms = int(3e-3 * rt_hz)
    attn_ghz = clock_under(lambda: [attn_call(first + b % nl) for b in range(4)],
                           lambda: [attn_call(first + b % nl) for b in range(4, 44)], ticks_3ms)

    def kv_reads(n):
        for i in range(n):
            b = first + i % nl
            probe.stream_read(K[b], T, row_b, Hkv * row_b, Hkv, -(-T // 64), sink)
            probe.stream_read(Vc[b], T, row_b, Hkv * row_b, Hkv, -(-T // 64), sink)
    read_ghz = clock_under(lambda: kv_reads(2), lambda: kv_reads(30), ticks_3ms)
    del sink
    return {
        "hbm_read_gbps": {"contiguous": round(max(contiguous.values()), 1),
                          "kv_pattern": round(max(pattern.values()), 1),
                          "kv_pattern_attn_grid": round(pattern[32], 1),
                          "contiguous_by_grid": {str(k): round(v, 1) for k, v in contiguous.items()},
                          "kv_pattern_by_ranges_per_head": {str(k): round(v, 1) for k, v in pattern.items()}},
        "shader_clock_ghz": {"idle": round(idle_ghz, 3), "during_attention": round(attn_ghz, 3),
                             "during_kv_read_stream": round(read_ghz, 3), "realtime_counter_mhz": round(rt_hz / 1e6, 3)},
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the parity check (it compares the CPU baseline's oracle results with the GPU's)")
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--workload", default=WORKLOAD,
                    help="configuration to time (profiling aid; the reported metric is long_128k's)")
    ap.add_argument("--splits", type=int, default=0, help="force the KV split count (0 = library choice)")
    ap.add_argument("--kv-layout", choices=("token", "head"), default="token",
                    help="bf16 KV cache storage: token-major [T, Hkv, D] (default) or head-major [Hkv, T, D], "
                         "given to the library through the strides (the read-ceiling probes keep the "
                         "token-major patterns)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: time tv_tree_attn over the bf16, FP8 and 4-bit caches "
                         "at every workload configuration, one JSON line each")
    return ap.parse_args()


def sweep(tv, make, np, torch, dev):
    """Per-configuration attention times: for each workload, distinct KV buffers (at least
    8 and 8 GB of bf16 cache, at most 64) in turn, back to back, HIP events. The FP8 and
    4-bit caches are the same buffers quantised on the GPU. Each format is timed over a
    token-major cache ([T, Hkv, D]) and over the same cache stored head-major ([Hkv, T, D],
    passed through the strides; fields *_hm_*). The six (layout, format) pairs are timed in
    turn within each of five rounds, after a warm-up of every pair; the median round."""
    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    stream = torch.cuda.current_stream()

    def one_config(name):
        w = make(name, 0, parts=("tree", "qkv"))
        N, L, Hq, Hkv, D = w.N, w.L, w.Hq, w.Hkv, w.D
        T, M = L + N, (Hq // Hkv) * N
        per = 2 * T * Hkv * D * 2
        nb = int(min(64, max(8, -(-8e9 // per))))
        K = torch.empty((nb, T, Hkv, D), dtype=torch.bfloat16, device=dev)
        Vc = torch.empty_like(K)
        g = torch.Generator(device=dev)
        g.manual_seed(42)
        K.normal_(generator=g)
        Vc.normal_(generator=g)
        K[0].copy_(to_dev(w.k))
        Vc[0].copy_(to_dev(w.v))
        # the same values, each head's rows contiguous, as [T, Hkv, D] views
        Kh = torch.empty((nb, Hkv, T, D), dtype=torch.bfloat16, device=dev)
        Vh = torch.empty_like(Kh)
        Kh.copy_(K.permute(0, 2, 1, 3))
        Vh.copy_(Vc.permute(0, 2, 1, 3))
        caches = {"": (K, Vc), "_hm": (Kh.permute(0, 2, 1, 3), Vh.permute(0, 2, 1, 3))}
        q = to_dev(w.q)
        parent = torch.from_numpy(w.parent).to(dev)
        out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(tv.tree_attn_workspace_size(N, L, Hq, Hkv, D), dtype=torch.uint8, device=dev)

        def codes(tag, width):
            if tag:
                return torch.empty((Hkv, T, width), dtype=torch.uint8, device=dev).permute(1, 0, 2)
            return torch.empty((T, Hkv, width), dtype=torch.uint8, device=dev)

        calls = {}
        for tag, (kb, vb) in caches.items():
            f8 = [(tv.kv_quantize_fp8(kb[b], codes=codes(tag, D)), tv.kv_quantize_fp8(vb[b], codes=codes(tag, D)))
                  for b in range(nb)]
            f4 = [(tv.kv_quantize_mx4(kb[b], codes=codes(tag, D // 2)),
                   tv.kv_quantize_mx4(vb[b], codes=codes(tag, D // 2))) for b in range(nb)]
            calls["bf16" + tag] = lambda b, kb=kb, vb=vb: tv.tree_attn(q, kb[b], vb[b], parent, L=L, scale=w.scale,
                                                                        out=out, workspace=ws)
            calls["fp8" + tag] = lambda b, f8=f8: tv.tree_attn_fp8(q, f8[b][0][0], f8[b][1][0], f8[b][0][1],
                                                                   f8[b][1][1], parent, L=L, scale=w.scale, out=out,
                                                                   workspace=ws)
            calls["mx4" + tag] = lambda b, f4=f4: tv.tree_attn_mx4(q, f4[b][0][0], f4[b][1][0], f4[b][0][1],
                                                                   f4[b][1][1], parent, L=L, scale=w.scale, out=out,
                                                                   workspace=ws)
        kv_bytes = {"bf16": 2 * T * Hkv * D * 2, "fp8": 2 * T * Hkv * (D + 4), "mx4": 2 * T * Hkv * (D // 2 + 4)}
        reps = max(40, nb)
        for call in calls.values():
            for b in range(2 * nb):
                call(b % nb)
        torch.cuda.synchronize()
        rounds = {key: [] for key in calls}
        for r in range(5):
            # the order of the pairs alternates between rounds
            for key in (list(calls) if r % 2 == 0 else list(calls)[::-1]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for b in range(reps):
                    calls[key](b % nb)
                e1.record(stream)
                torch.cuda.synchronize()
                rounds[key].append(e0.elapsed_time(e1) * 1e3 / reps)
        rec = {"sweep": name, "L": L, "N": N, "Hq": Hq, "Hkv": Hkv, "rows_per_kv_head": M, "kv_buffers": nb}
        for key in calls:
            t = float(np.median(rounds[key]))
            rec[f"{key}_us"] = round(t, 2)
            rec[f"{key}_kv_tbps"] = round(kv_bytes[key.split("_")[0]] / t / 1e6, 3)
        rec["bf16_tflops"] = round(4.0 * N * Hq * T * D / rec["bf16_us"] / 1e6, 1)
        return rec

    for name in ("tiny_chain", "budget22", "branch_8k", "long_128k", "max_256k", "wide_tree", "decode_1node"):
        print(json.dumps(one_config(name)), flush=True)
        torch.cuda.empty_cache()  # the configuration's buffers died with one_config


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the verify step is measured per device; a "
              "multi-GPU layout (KV heads split across GPUs, no exchange) is not built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_tree_verification_tv_amd as tv
    from workloads import make

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tv.lib()
    if args.sweep:
        sweep(tv, make, np, torch, dev)
        return

    log("generating the seeded workload (CPU)")
    w = make(args.workload, 0)
    N, L, Hq, Hkv, D, V = w.N, w.L, w.Hq, w.Hkv, w.D, w.V
    T = L + N

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    layers = args.layers
    log(f"allocating {layers} KV buffers ({2 * layers * T * Hkv * D * 2 / 1e9:.1f} GB)")
    if args.kv_layout == "head":
        # each head's rows side by side; K[b] and Vc[b] are [T, Hkv, D] views of the storage
        K_store = torch.empty((layers, Hkv, T, D), dtype=torch.bfloat16, device=dev)
        V_store = torch.empty((layers, Hkv, T, D), dtype=torch.bfloat16, device=dev)
        K, Vc = K_store.permute(0, 2, 1, 3), V_store.permute(0, 2, 1, 3)
    else:
        K = K_store = torch.empty((layers, T, Hkv, D), dtype=torch.bfloat16, device=dev)
        Vc = V_store = torch.empty((layers, T, Hkv, D), dtype=torch.bfloat16, device=dev)
    K[0].copy_(to_dev(w.k))
    Vc[0].copy_(to_dev(w.v))
    g = torch.Generator(device=dev)
    g.manual_seed(42)
    for b in range(1, layers):
        K[b].normal_(generator=g)
        Vc[b].normal_(generator=g)
    q = to_dev(w.q)
    parent = torch.from_numpy(w.parent).to(dev)
    draft = torch.from_numpy(w.draft).to(dev)
    logits = to_dev(w.logits)
    out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(tv.tree_attn_workspace_size(N, L, Hq, Hkv, D, args.splits), dtype=torch.uint8, device=dev)
    am_ws = tv.argmax_workspace(N, V, dev)
    tok = torch.empty(N, dtype=torch.int32, device=dev)
    acc = (torch.empty(1, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.int32, device=dev),
           torch.empty(N, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # Kernels go to the current stream: `stream` when eager, the capture stream while a
        # graph is being recorded. ev[b] .. ev[b+1] brackets attention call b; the last pair
        # brackets argmax + accept.
        if ev:
            ev[0].record(stream)
        for b in range(layers):
            tv.tree_attn(q, K[b], Vc[b], parent, L=L, scale=w.scale, num_splits=args.splits, out=out, workspace=ws)
            if ev:
                ev[b + 1].record(stream)
        # argmax over the vocabulary and the accept walk: one call, two launches
        tv.argmax_accept(logits, parent, draft, tok=tok, out=acc, workspace=am_ws)
        if ev:
            ev[layers + 1].record(stream)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + written once")
        del src, dst

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(layers + 2)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # The same step captured once as a HIP graph and replayed (every call only enqueues
    # kernels on the stream, so the whole step is capturable).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms_per_step = g0.elapsed_time(g1) / args.steps
    del graph

    # Next-row calls on the same inputs, timed alone (not part of `value`): sampled
    # verification at temperature 1 and the KV commit of the accepted path (on layer 1's
    # cache, whose values do not matter for the timing).
    # The first few dozen calls on freshly written buffers run up to 15 % slow, so each
    # timing warms up first and reports the median of five rounds.
    def timed(fn, reps=20, warm=8):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        rounds = []
        for _ in range(5):
            t0e.record(stream)
            for _ in range(reps):
                fn()
            t1e.record(stream)
            torch.cuda.synchronize()
            rounds.append(t0e.elapsed_time(t1e) * 1e3 / reps)
        return float(np.median(rounds))

    sample_us = timed(lambda: tv.sample_accept(logits, parent, draft, 1.0, 1234, 0, tok=tok, out=acc,
                                               workspace=am_ws))
    tv.argmax_accept(logits, parent, draft, tok=tok, out=acc, workspace=am_ws)
    commit_us = timed(lambda: tv.kv_commit(K[1], Vc[1], L, acc[0], acc[1]))

    # FP8 cache: the caches of the first four layers quantised on the GPU (together larger
    # than the last-level cache), then the tree attention over them in turn.
    nf8 = min(layers, 4)
    f8 = [(tv.kv_quantize_fp8(K[b]), tv.kv_quantize_fp8(Vc[b])) for b in range(nf8)]
    quant_us = timed(lambda: tv.kv_quantize_fp8(K[1], codes=f8[1][0][0], exps=f8[1][0][1]))
    f8_turn = [0]

    def fp8_call():
        (kc, ke), (vc, ve) = f8[f8_turn[0] % nf8]
        f8_turn[0] += 1
        tv.tree_attn_fp8(q, kc, vc, ke, ve, parent, L=L, scale=w.scale, num_splits=args.splits, out=out,
                         workspace=ws)
    fp8_us = timed(fp8_call, reps=8 * nf8, warm=4 * nf8)
    del f8

    # 4-bit cache: the same four layers quantised on the GPU, then the tree attention over
    # them in turn.
    mx = [(tv.kv_quantize_mx4(K[b]), tv.kv_quantize_mx4(Vc[b])) for b in range(nf8)]
    mx_quant_us = timed(lambda: tv.kv_quantize_mx4(K[1], codes=mx[1][0][0], exps=mx[1][0][1]))
    mx_turn = [0]

    def mx4_call():
        (kc, ke), (vc, ve) = mx[mx_turn[0] % nf8]
        mx_turn[0] += 1
        tv.tree_attn_mx4(q, kc, vc, ke, ve, parent, L=L, scale=w.scale, num_splits=args.splits, out=out,
                         workspace=ws)
    mx4_us = timed(mx4_call, reps=8 * nf8, warm=4 * nf8)
    del mx

    # Streaming reference on this machine: a plain 1 GiB device-to-device copy (read and
    # write counted), the best of five; context for the roofline fraction.
    cp_n = 1 << 30
    cp_src = torch.empty(cp_n, dtype=torch.uint8, device=dev).fill_(3)
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    cp_best = float("inf")
    for _ in range(5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        cp_dst.copy_(cp_src)
        c1.record(stream)
        torch.cuda.synchronize()
        cp_best = min(cp_best, c0.elapsed_time(c1) * 1e-3)
    copy_gbps = 2 * cp_n / cp_best / 1e9
    del cp_src, cp_dst

    # the probes read the caches' storage in the token-major patterns whatever the layout
    ceilings = measure_ceilings(K_store, V_store, T, Hkv, D, layers, stream,
                                lambda b: tv.tree_attn(q, K[b], Vc[b], parent, L=L, scale=w.scale,
                                                       num_splits=args.splits, out=out, workspace=ws))

    # Every attention call timed on its own (steps x layers repetitions): median, p10, p90.
    attn_ms = np.array([e[b].elapsed_time(e[b + 1]) for e in events for b in range(layers)])
    tokens_ms = np.array([e[layers].elapsed_time(e[layers + 1]) for e in events])
    t_attn_us = float(np.median(attn_ms) * 1e3)
    t_attn_mean_us = float(np.mean(attn_ms) * 1e3)  # the roofline uses the average duration
    t_tokens_us = float(np.median(tokens_ms) * 1e3)
    call_us = t_attn_us + t_tokens_us
    ms_per_step = wall * 1e3 / args.steps

    kv_bytes = 2 * T * Hkv * D * 2
    qo_bytes = 2 * N * Hq * D * 2
    algo_bytes = kv_bytes + qo_bytes
    achieved = algo_bytes / (t_attn_mean_us * 1e-6) / 1e9
    flops = 4 * N * Hq * T * D
    # The roofline that bounds the call: HBM for long contexts, MFMA for wide trees
    # (arithmetic intensity above the 312 flop/B ridge of 2.5 PFLOP/s over 8 TB/s).
    mfma_bound = flops / algo_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(flops / (t_attn_mean_us * 1e-6) / 1e12, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(flops / (t_attn_mean_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None, "kernel": "tv_tree_attn (split + merge)", "algorithmic_flops": flops}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": (measured_traffic() if args.workload == WORKLOAD and args.kv_layout == "token"
                                else None),
                    "kernel": "tv_tree_attn (split + merge)", "algorithmic_bytes": algo_bytes,
                    "traffic_unit": "bytes per call"}
    kv_gbps = kv_bytes / (t_attn_us * 1e-6) / 1e9
    log(f"attn {t_attn_us:.1f} us/call ({kv_gbps:.0f} GB/s KV, {kv_gbps / HBM_PEAK_GBS:.1%} of peak), "
        f"argmax+accept {t_tokens_us:.1f} us, step {ms_per_step:.2f} ms (graph replay {graph_ms_per_step:.2f} ms)")

    parity = None
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = len(os.sched_getaffinity(0))
        log(f"CPU oracle baseline: whole verify calls (attention over all heads, argmax, accept) for "
            f"about {CPU_SAMPLE_SECONDS:.0f} s ({threads} cores)")
        qf = oracle.bf16_bits_to_f64(w.q)
        kf = oracle.bf16_bits_to_f64(w.k)
        vf = oracle.bf16_bits_to_f64(w.v)
        lf = oracle.bf16_bits_to_f64(w.logits)
        reps = 0
        t0 = time.perf_counter()
        while True:
            ref, _ = oracle.tree_attention(qf, kf, vf, w.parent, w.scale)
            etok = oracle.argmax_rows(lf)
            eacc = oracle.accept(w.parent, w.draft, etok)
            reps += 1
            if time.perf_counter() - t0 >= CPU_SAMPLE_SECONDS:
                break
        cpu_us = (time.perf_counter() - t0) / reps * 1e6
        del qf, kf, vf, lf
        if not args.no_check:
            # The oracle's own results from the timed calls against the GPU's on buffer 0:
            # attention for every head, argmax and the acceptance walk.
            log("parity check of KV buffer 0 against the oracle results just timed")
            tv.tree_attn(q, K[0], Vc[0], parent, L=L, scale=w.scale, num_splits=args.splits, out=out, workspace=ws)
            tv.argmax_accept(logits, parent, draft, tok=tok, out=acc, workspace=am_ws)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            err = float(np.abs(got - ref).max())
            excess = float((np.abs(got - ref) - (1e-2 + 2e-2 * np.abs(ref))).max())
            rel = float((np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)).max())
            eln, enodes, etoks, ebonus = eacc
            got_nodes = acc[1].cpu().numpy()
            accept_ok = (int(acc[0].item()) == eln and got_nodes[:eln].tolist() == enodes.tolist()
                         and acc[2].cpu().numpy()[:eln].tolist() == etoks.tolist() and int(acc[3].item()) == ebonus)
            parity = {"attn_max_abs": err, "attn_row_rel": rel,
                      "argmax_exact": bool((tok.cpu().numpy() == etok).all()), "accept_exact": bool(accept_ok),
                      "accept_len": int(eln)}
            ok = excess <= 0 and rel <= 2e-2 and parity["argmax_exact"] and parity["accept_exact"]
            log(f"parity {'OK' if ok else 'FAILED'}: {parity}")
            if not ok:
                sys.exit(1)
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
        except OSError:
            pass
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max((d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"),
                               default=None)
        except Exception:  # threadpoolctl missing or unable to inspect the BLAS
            blas_threads = None
        cpu = {"value": round(cpu_us, 1), "unit": "us per tree-verify call", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model, "blas_threads": blas_threads,
               "sample": f"float64 numpy oracle on KV buffer 0 of the same workload: {reps} whole verify "
                         f"call(s) (tree attention of {N} nodes x {Hq} q heads over {T} keys, argmax of the "
                         f"[{N}, {V}] logits, accept walk), mean time per call; bf16->float64 input "
                         f"widening not timed"}
        log(f"CPU oracle: {cpu_us / 1e3:.1f} ms per call over {reps} call(s)")

    rec = {
        "metric": "µs per tree-verify call (attn+argmax+accept) and KV GB/s vs HBM peak",
        "value": round(call_us, 2),
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("long_128k: KV 131072 + 64-node tree (depth<=16), 32 q / 8 KV heads, D=128, "
                                "bf16; logits [64,152064] bf16; 64 layer-equivalent attention calls on distinct "
                                "KV buffers + argmax + accept per step") if args.workload == WORKLOAD else
                               (f"{args.workload}: KV {L} + {N} nodes, {Hq} q / {Hkv} KV heads, D={D}, bf16; logits "
                                f"[{N},{V}]; {layers} layer-equivalent attention calls on distinct KV buffers + "
                                f"argmax + accept per step"),
                   "kv_len": L, "nodes": N, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V,
                   "layers_per_step": layers, "kv_layout": args.kv_layout, "parallelism": "none (1 GPU)"},
        "breakdown_us": {"attn_per_call": round(t_attn_us, 2), "attn_mean": round(t_attn_mean_us, 2),
                         "attn_calls_timed": int(attn_ms.size), "argmax_accept": round(t_tokens_us, 2),
                         "attn_p10": round(float(np.percentile(attn_ms, 10) * 1e3), 2),
                         "attn_p90": round(float(np.percentile(attn_ms, 90) * 1e3), 2)},
        "graph_ms_per_step": round(graph_ms_per_step, 3),
        "next_rows_us": {"sample_accept_T1": round(sample_us, 2), "kv_commit": round(commit_us, 2),
                         "tree_attn_fp8": round(fp8_us, 2), "kv_quantize_fp8_one_tensor": round(quant_us, 2),
                         "tree_attn_mx4": round(mx4_us, 2), "kv_quantize_mx4_one_tensor": round(mx_quant_us, 2)},
        "kv_gbps": round(kv_gbps, 1),
        "kv_hbm_frac": round(kv_gbps / HBM_PEAK_GBS, 4),
        "hbm_copy_gbps": round(copy_gbps, 1),
        "hbm_read_gbps": ceilings["hbm_read_gbps"],
        "shader_clock_ghz": ceilings["shader_clock_ghz"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
