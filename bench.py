#!/usr/bin/env python3
"""Decode throughput of the routed-expert MoE layer on one MI355X (gfx950).

The default workload is the GLM-scale decode stack (hidden 6144, 256 experts of
intermediate 2048, top-8, shared expert 2048, 40 layers, 218 GB of records in
HBM, Zipf(1.1) routing); --workload gemma_a4b_h2816_e128_l30 runs the
Gemma-4-A4B-scale 30-layer stack.  A step is one decode token (batch 1)
through every layer of the workload's stack: router + exact top-8 + gates, the 8 selected experts' dequant-fused
SwiGLU, the shared expert and the weighted combine, layer after layer on one
stream (layer l+1 starts after layer l's output is written).  Inputs are
synthetic and seeded (synth/): random 4-bit records filled on the GPU, int8
routers, N(0,1) bf16 activations, a distinct input for each of the workload's
decode steps.  Timed: exactly --steps steps, replayed as hipGraphs of up to
--graph-chunk steps (the largest divisor of --steps not above it), bracketed
by synchronisations.

Printed (stdout, one JSON line): decode tokens/s per MoE layer (value), the
whole-stack tokens/s, achieved HBM GB/s on algorithmic bytes (router + 8
selected records + shared record per token-layer) against the 8 TB/s peak,
a roofline entry for the dominant kernel (gate/up) from a live per-kernel
pass (dispatch-stamped hipEvents), a plain streaming read of one token-layer's
bytes timed in the same run (the achievable HBM rate the layer is set
against), and the CPU oracle timed on this host's cores (one thread and all
cores).

--workload glm_prefill_h6144_e256_t128 measures the grouped (prefill) path
instead: a step is one 128-token chunk through one layer, cycling over
--prefill-layers layers of distinct weights; the roofline entry is the grouped
gate/up kernel's, with its MFMA utilisation.  --workload
offload_h2816_e256_l40_lfu16 measures the out-of-core decode with the HBM
slot cache.  --bits 2 runs any workload on 2-bit records of the same affine
group-64 format.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs (profiles/*_counters.md), each scaled by the same counter's
# reading for a 1 GiB device copy (FETCH x2.0, WRITE x1.0).  Valid only for the
# kernel sources they were taken on (first 16 hex digits of the sha256 of the
# kernel file followed by the two device headers it includes); None once any
# of them changes.
KERNEL_HEADERS = ("moe_device.h", "moe_internal.h")
TRAFFIC = {
    # FETCH_SIZE 62870.48 KiB x 2.00 + WRITE_SIZE 160.84 KiB x 1.00 per launch
    ("glm_h6144_e256_l40_zipf", "k_gate_up"): (128918532, "moe_kernels.hip", "f321826cbb94aa76"),
    # FETCH_SIZE 12344.51 KiB x 2.00 + WRITE_SIZE 41.88 KiB x 1.00 per launch (the launch
    # also runs the router)
    ("gemma_a4b_h2816_e128_l30", "k_gate_up"): (25323475, "moe_kernels.hip", "f321826cbb94aa76"),
    # FETCH_SIZE 1833452.71 KiB x 2.00 + WRITE_SIZE 5756.12 KiB x 1.00 per launch (mean over
    # the bench's 32 distinct chunks)
    ("glm_prefill_h6144_e256_t128", "k_gu_grouped"): (3760662184, "moe_prefill.hip", "5f90596f37f6cfc7"),
}


def source_digest(src):
    import hashlib
    h = hashlib.sha256()
    for name in (src, *KERNEL_HEADERS):
        with open(os.path.join(ROOT, "bit_routed_expert_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload, kernel, bits=4):
    ent = TRAFFIC.get((workload if bits == 4 else f"{workload}/bits{bits}", kernel))
    if ent is None:
        return None
    nbytes, src, digest = ent
    return nbytes if source_digest(src) == digest else None


METRIC = "decode tokens/s per MoE layer + achieved HBM GB/s vs peak (batch 1, top-8)"


def chunk_len(K: int, cap: int) -> int:
    """Steps per graph: the largest divisor of K not above cap, so that exactly K
    steps are replayed in whole graphs."""
    return max(d for d in range(1, max(1, min(K, cap)) + 1) if K % d == 0)


def graph_units(run_step, S: int, G: int, n: int):
    """n replay callables; the i-th runs steps (i*G + j) mod S, j < G, captured
    as one hipGraph (graphs over the same steps are shared)."""
    import torch
    made, units = {}, []
    for i in range(n):
        c0 = (i * G) % S
        if c0 not in made:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(G):
                    run_step((c0 + j) % S)
            made[c0] = g.replay
        units.append(made[c0])
    return units


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gu_bytes(H, I, bits=4):
    """gate+up part of a record: codes 2*I*H*bits/8 bytes + scale/bias I*H/8 bytes."""
    return H * I * bits // 4 + H * I // 8


def down_bytes(H, I, bits=4):
    """down part: codes H*I*bits/8 bytes + scale/bias H*I/16 bytes."""
    return H * I * bits // 8 + H * I // 16


def launch_bytes(wl, bits, T, fused_route):
    """Algorithmic bytes per launch of the per-token path's kernels for T
    tokens: the router (int8 rows + fp16 scales), the gate/up halves and the
    down halves of the k routed records plus the shared one.  With
    fused_route the router runs inside the gate/up launch, which then reads
    both."""
    H, E, I, k, Is = wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter
    rt = T * (E * H + 2 * E)
    gu = T * (k * gu_bytes(H, I, bits) + (gu_bytes(H, Is, bits) if Is else 0))
    dn = T * (k * down_bytes(H, I, bits) + (down_bytes(H, Is, bits) if Is else 0))
    return {"route": rt, "gate_up": gu + (rt if fused_route else 0), "down_combine": dn}


def token_layer_bytes(wl, bits):
    """Algorithmic HBM bytes of one decode token through one layer: the router,
    the top_k selected records and the shared record."""
    from bit_routed_expert_moe_amd import record_bytes
    rbs = record_bytes(wl.hidden, wl.shared_inter, bits) if wl.shared_inter else 0
    return wl.router_bytes + wl.top_k * record_bytes(wl.hidden, wl.inter, bits) + rbs


def dtype_desc(bits):
    return f"u{bits} weights x f16 activations -> f32"


def make_inputs(wl, layer, S):
    """[S][T][H] activations for one layer (float64) from the seeded generator."""
    import synth
    if wl.routing in ("zipf", "uniform"):
        q, rs = synth.router(wl.seed, layer, wl.n_experts, wl.hidden)
        W = q.astype(np.float64) * rs.view(np.float16).astype(np.float64)[:, None]
        zr = synth.ZipfRealiser(W, wl.zipf_s, wl.seed, layer)
        return zr.activations_batch(range(S))[:, None, :]
    return np.stack([synth.activations(wl.seed, layer, s, wl.hidden, wl.n_tokens) for s in range(S)])


def kernel_timed_pass(run_steps, capacity):
    """Per-launch timings of run_steps(): while the library's profiler is on it
    dispatches each kernel with hipExtLaunchKernelGGL and a start/stop hipEvent
    pair on the launch stream, stamped by that dispatch itself (its begin and
    end, as a kernel trace reports them).  Returns [(name, ms)]."""
    import torch
    from bit_routed_expert_moe_amd import KernelTimer
    run_steps()  # warm pass
    torch.cuda.synchronize()
    with KernelTimer(capacity=capacity) as kt:
        run_steps()
    recs = kt.read()
    torch.cuda.synchronize()
    return recs


STREAM_BLOCKS = (1024, 2048, 4096)  # workgroup counts tried for the plain read


def stream_reference(pools, nbytes, steps):
    """A plain streaming read (moe_stream_read) of one token-layer's bytes,
    timed in this run: for each of `steps` steps and each layer, nbytes from
    that layer's pool at an offset that moves with the step (so, like the
    layer's own reads, no read is served from a cache), dispatch-timed.
    Returns the best workgroup count's rate and every count's."""
    import torch
    from bit_routed_expert_moe_amd import KernelTimer, stream_read
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = nbytes // 256 * 256
    res = {}
    for nb in STREAM_BLOCKS:
        def run():
            for s in range(steps):
                for pool, _, _ in pools:
                    span = pool.numel() - n
                    off = (s * 7919 * 256 * 64) % max(span, 1) // 256 * 256
                    stream_read(pool, off, n, nb, sink)
        recs = kernel_timed_pass(run, steps * len(pools) + 16)
        ms = np.array([m for name, m in recs if name == "stream_read"])
        res[nb] = {"launches": int(ms.size), "avg_us": round(float(ms.mean()) * 1e3, 3),
                   "gbps": round(n / (float(ms.mean()) * 1e-3) / 1e9, 1)}
    best = max(res, key=lambda b: res[b]["gbps"])
    return {"gbps": res[best]["gbps"], "bytes_per_launch": n, "best_blocks": best,
            "kernel": "k_stream_read (16-byte nontemporal loads, 256 threads, 8 in flight each)",
            "by_blocks": {str(b): v for b, v in res.items()}}


SIGMOID_SCALE = 2.5  # routed scaling factor of the sigmoid-router runs


def gate_kwargs(args, wl, layer, dev):
    """Layer keyword arguments for the chosen gate; the bias is seeded per layer."""
    import synth
    import torch
    if args.gate == "softmax":
        return {}
    b = synth.selection_bias(wl.seed, layer, wl.n_experts)
    return dict(gate="sigmoid", routed_scale=SIGMOID_SCALE, selection_bias=torch.from_numpy(b).to(dev))


def gate_desc(args):
    return "softmax" if args.gate == "softmax" else f"sigmoid (bias U(-0.05, 0.05), scale {SIGMOID_SCALE})"


def oracle_route(orc, args, wl, layer, rq, rs, xd):
    import synth
    if args.gate == "softmax":
        return orc.route(rq, rs, xd, wl.top_k)
    b = synth.selection_bias(wl.seed, layer, wl.n_experts).astype(np.float64)
    return orc.route(rq, rs, xd, wl.top_k, gate="sigmoid", bias=b, scale=SIGMOID_SCALE)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, xs_host, seconds, args, pools):
    """The CPU oracle on the first token-layers of the same inputs (steps in
    order, layers in order), in two modes: one thread, then every core of this
    process's affinity set (OpenMP over output rows), each for about seconds/2
    of oracle compute.  The selected records are read back from the device
    pools (filled by the seeded generator) outside the timed region; only the
    oracle's own compute is timed."""
    import oracle
    orc = oracle.default()
    H, I, Is, k = wl.hidden, wl.inter, wl.shared_inter, wl.top_k
    S, L = xs_host.shape[0], xs_host.shape[1]
    routers = {}

    def record(l, e):
        pool, shared, rb = pools[l]
        if e < 0:
            return shared.cpu().numpy()
        return pool[e * rb:(e + 1) * rb].cpu().numpy()

    def run(threads, budget):
        used = orc.set_threads(threads)
        spent, n = 0.0, 0
        for s in range(S):
            for l in range(L):
                if l not in routers:
                    import synth
                    routers[l] = synth.router(wl.seed, l, wl.n_experts, H)
                rq, rs = routers[l]
                for t in range(wl.n_tokens):
                    xd = orc.act_to_f64(wl.act, xs_host[s, l, t])
                    t0 = time.perf_counter()
                    ids, w, _ = oracle_route(orc, args, wl, l, rq, rs, xd)
                    spent += time.perf_counter() - t0
                    recs = [record(l, int(e)) for e in ids]
                    shared = record(l, -1) if Is else None
                    t0 = time.perf_counter()
                    yr = np.stack([orc.expert_ffn(H, I, r, xd, bits=args.bits) for r in recs])
                    ys = orc.expert_ffn(H, Is, shared, xd, bits=args.bits) if Is else None
                    orc.combine(w, yr, ys)
                    spent += time.perf_counter() - t0
                    n += 1
                if spent >= budget:
                    return n, spent, used
        return n, spent, used

    all_cores = len(os.sched_getaffinity(0))
    n1, t1, u1 = run(1, seconds / 2)
    na, ta, ua = run(all_cores, seconds / 2)
    return {"value": round(na / ta, 3), "unit": "tok/s per layer", "cores": ua, "kind": "oracle",
            "sample": f"{na} token-layers (steps 0.., layers in order) of the same inputs; fp64 "
                      f"plain-loop oracle, OpenMP over output rows on {ua} threads; records read "
                      f"back from the device pools outside the timing; {ta:.1f} s of oracle compute",
            "single_thread": {"value": round(n1 / t1, 3), "unit": "tok/s per layer", "cores": u1,
                              "sample": f"{n1} token-layers, the same ones first; {t1:.1f} s"},
            "cpu_model": cpu_model(), "host_cores": all_cores,
            "stack_tok_s": round(na / ta / L, 4)}


LOOKAHEAD_RECALL = 0.716  # top-8 recall of the lookahead router on a real model (Colibri README)


def topk_sets(W, X, k):
    """Top-k expert sets (by float64 logit) of the rows of X under router W [E][H]."""
    lg = X @ W.T
    return [set(np.argpartition(-row, k)[:k].tolist()) for row in lg]


def lookahead_hints(wl, xs_host, rho):
    """[S][L][1][H] hints, layer l's from its own input (layer 0's unused)."""
    import synth
    S, L = xs_host.shape[0], xs_host.shape[1]
    return np.stack([np.stack([synth.lookahead_hint(wl.seed, l, s, xs_host[s, l], rho)
                               for l in range(L)]) for s in range(S)])


def lookahead_recall(wl, routers, xs_host, rho, steps):
    """Mean |top-k(hint) & top-k(x)| / k over the given steps and layers 1..L-1."""
    import synth
    k, L = wl.top_k, xs_host.shape[1]
    hit = n = 0
    for l in range(1, L):
        X = xs_host[steps, l, 0]
        Hh = np.stack([synth.lookahead_hint(wl.seed, l, s, xs_host[s, l], rho)[0] for s in steps])
        for a, b in zip(topk_sets(routers[l], X, k), topk_sets(routers[l], Hh, k)):
            hit += len(a & b)
            n += k
    return hit / n


def calibrate_rho(wl, routers, xs_host, target, steps):
    """The rho whose hints reach the target recall on these steps (bisection;
    the recall grows with rho)."""
    lo, hi = 0.0, 1.0
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        if lookahead_recall(wl, routers, xs_host, mid, steps) < target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def run_cached(args, wl):
    """Out-of-core decode: each layer keeps wl.n_slots HBM slots filled from a
    pinned host pool of all its experts (--cache-policy, default LFU; with
    --pin N the N experts used most during the warm-up steps are pinned per
    layer before the timed steps; with --lookahead N each layer l+1 prefetches
    the top N experts of a hint derived from its input before layer l runs, the
    hints' noise set so that their top-8 recall is the pages' 71.6 %).
    Launched eagerly: every layer synchronises the host on its expert ids."""
    import torch
    import synth
    import synth.gpu
    from bit_routed_expert_moe_amd import Layer, record_bytes

    H, E, I, k, Is, L = wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.n_layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    bits = args.bits
    rb = record_bytes(H, I, bits)
    t_setup = time.time()
    layers, keep = [], []
    staging = torch.empty(E * rb, dtype=torch.uint8, device=dev)
    for l in range(L):
        rq, rs = synth.router(wl.seed, l, E, H)
        synth.gpu.fill_records(staging, H, I, wl.seed, l, 0, E, bits=bits)
        host = torch.empty(E * rb, dtype=torch.uint8, pin_memory=True)
        host.copy_(staging)
        shared = torch.empty(record_bytes(H, Is, bits), dtype=torch.uint8, device=dev)
        synth.gpu.fill_records(shared, H, Is, wl.seed, l, -1, 1, bits=bits)
        slots = torch.zeros(wl.n_slots * rb, dtype=torch.uint8, device=dev)
        layers.append(Layer(H, E, I, k, Is, torch.from_numpy(rq).to(dev),
                            torch.from_numpy(rs.view(np.float16)).to(dev), None, shared,
                            act=wl.act, n_slots=wl.n_slots, host_pool=host, slots=slots,
                            cache_policy=args.cache_policy, bits=bits,
                            **gate_kwargs(args, wl, l, dev)))
    del staging
    S = wl.steps
    xs_host = np.stack([make_inputs(wl, l, S) for l in range(L)], axis=1)  # [S][L][1][H]
    xs = torch.from_numpy(synth.quantize_act(xs_host, wl.act).view(np.int16)).to(dev).view(torch.bfloat16)
    ws = layers[0].workspace(1)
    W = min(args.warmup, S)
    K = min(args.steps, S - W)
    la = None
    if args.lookahead:
        routers = []
        for l in range(L):
            q, rs_ = synth.router(wl.seed, l, E, H)
            routers.append(q.astype(np.float64) * rs_.view(np.float16).astype(np.float64)[:, None])
        rho = calibrate_rho(wl, routers, xs_host, LOOKAHEAD_RECALL, list(range(min(32, S))))
        hs = torch.from_numpy(synth.quantize_act(lookahead_hints(wl, xs_host, rho), wl.act)
                              .view(np.int16)).to(dev).view(torch.bfloat16)
        pid = torch.empty(L, 1, k, dtype=torch.int32, device=dev)
        pw = torch.empty(L, 1, k, dtype=torch.float32, device=dev)
        ph = torch.empty(L, k, dtype=torch.int32, pin_memory=True)
        la = {"n_predict": args.lookahead, "mode": args.lookahead_mode, "hint_rho": round(rho, 4),
              "recall_target": LOOKAHEAD_RECALL,
              "recall_timed": round(lookahead_recall(wl, routers, xs_host, rho,
                                                     list(range(W, W + K))), 4)}
        del routers
    ids = torch.empty(L, 1, k, dtype=torch.int32, device=dev)
    w = torch.empty(L, 1, k, dtype=torch.float32, device=dev)
    y = torch.empty(L, 1, H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f} s: {L} layers x {E} experts in pinned host memory "
        f"({L * E * rb / 1e9:.2f} GB), {wl.n_slots} slots per layer")

    def run_step(s):
        for l in range(L):
            nxt = la is not None and l + 1 < L  # layer l+1's experts from its hint, ahead of layer l
            if nxt and args.lookahead_mode == "call":
                layers[l + 1].cache_prefetch(hs[s, l + 1, 0], args.lookahead, ws)
            elif nxt:  # route the hint now, read the ids once layer l's call has synchronised
                layers[l + 1].route(hs[s, l + 1], ws, out=(pid[l + 1], pw[l + 1]))
                ph[l + 1].copy_(pid[l + 1, 0], non_blocking=True)
            layers[l].forward(xs[s, l], ws, out=(ids[l], w[l], y[l]))
            if nxt and args.lookahead_mode == "ids":
                layers[l + 1].cache_prefetch_ids(ph[l + 1, :args.lookahead].tolist())

    # pinned host -> device bandwidth in the same run (1 GiB, the bound's denominator)
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_gbs = 4 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    counts = np.zeros((L, E), dtype=np.int64)  # expert selections per layer over the warm-up
    for s in range(W):
        run_step(s)
        if args.pin:
            for l, row in enumerate(ids.cpu().numpy()[:, 0]):
                np.add.at(counts[l], row, 1)
    torch.cuda.synchronize()
    if args.pin:
        for l in range(L):
            if args.pin_source == "learned":  # the layer's own usage heatmap
                if layers[l].cache_usage() != counts[l].tolist():
                    raise RuntimeError(f"layer {l}: usage heatmap differs from the warm-up's selections")
                layers[l].cache_pin_hottest(args.pin)
            else:
                top = sorted(range(E), key=lambda e: (-counts[l, e], e))[:args.pin]
                layers[l].cache_pin(top)
        torch.cuda.synchronize()
    h0 = sum(l_.cache_stats()[0] for l_ in layers)
    m0 = sum(l_.cache_stats()[1] for l_ in layers)
    p0 = [sum(l_.prefetch_stats()[i] for l_ in layers) for i in (0, 1)]
    t0 = time.perf_counter()
    for s in range(W, W + K):
        run_step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h1 = sum(l_.cache_stats()[0] for l_ in layers)
    m1 = sum(l_.cache_stats()[1] for l_ in layers)
    p1 = [sum(l_.prefetch_stats()[i] for l_ in layers) for i in (0, 1)]
    ms_per_step = wall * 1e3 / K
    hit_timed = (h1 - h0) / max(1, (h1 - h0) + (m1 - m0))
    hit_all = h1 / max(1, h1 + m1)
    miss_bytes_step = (m1 - m0) / K * rb
    pref_bytes_step = (p1[0] - p0[0]) / K * rb
    h2d_bytes_step = miss_bytes_step + pref_bytes_step
    hbm_bytes_step = L * token_layer_bytes(wl, bits) + h2d_bytes_step  # reads + slot writes
    bound_ms = max(hbm_bytes_step / (PEAK_HBM_GBS * 1e9), h2d_bytes_step / (h2d_gbs * 1e9)) * 1e3
    if la:
        la["prefetch_per_step"] = round((p1[0] - p0[0]) / K, 2)
        la["prefetch_used_frac"] = round((p1[1] - p0[1]) / max(1, p1[0] - p0[0]), 4)
    out = {
        "metric": METRIC, "value": round(L / (ms_per_step * 1e-3), 1), "unit": "tok/s per layer",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_desc(bits), "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "n_experts": E, "inter": I, "top_k": k,
                   "shared_inter": Is, "layers": L, "batch": 1, "act": wl.act, "bits": bits,
                   "routing": wl.routing, "gate": gate_desc(args), "n_slots": wl.n_slots,
                   "cache_policy": args.cache_policy, "pinned_per_layer": args.pin,
                   "lookahead": args.lookahead,
                   "pin_source": (f"expert counts over the {W} warm-up steps" + (
                       ", from each layer's usage heatmap" if args.pin_source == "learned" else ""))
                   if args.pin else None},
        "stack_tok_s": round(1e3 / ms_per_step, 2),
        "hit_rate_timed": round(hit_timed, 4), "hit_rate_all_steps": round(hit_all, 4),
        "miss_bytes_per_step": int(miss_bytes_step), "h2d_bytes_per_step": int(h2d_bytes_step),
        "h2d_gbps": round(h2d_gbs, 1), "lookahead": la,
        "roofline": {"bound": "pcie", "achieved": round(h2d_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
                     "peak": round(h2d_gbs, 1), "unit": "GB/s",
                     "frac": round(bound_ms / ms_per_step, 4), "traffic": None,
                     "note": "frac = max(HBM bytes / 8 TB/s, H2D bytes (misses + prefetches) / "
                             "measured H2D) / step time"},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def run_prefill(args, wl):
    """Prefill chunks: a step is one chunk of wl.n_tokens tokens through one layer
    (router, top-k, grouping by expert, grouped gate/up and down, combine).
    Steps cycle over --prefill-layers layers of distinct weights, so a layer's
    records are not served from a cache between its steps."""
    import torch
    import synth
    import synth.gpu
    from bit_routed_expert_moe_amd import Layer, record_bytes

    H, E, I, k, Is, T = wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.n_tokens
    NL, C = args.prefill_layers, args.prefill_chunks
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    bits = args.bits
    rb, rbs = record_bytes(H, I, bits), (record_bytes(H, Is, bits) if Is else 0)
    t_setup = time.time()
    layers, pools = [], []
    for l in range(NL):
        rq, rs = synth.router(wl.seed, l, E, H)
        pool = torch.empty(E * rb, dtype=torch.uint8, device=dev)
        synth.gpu.fill_records(pool, H, I, wl.seed, l, 0, E, bits=bits)
        shared = None
        if Is:
            shared = torch.empty(rbs, dtype=torch.uint8, device=dev)
            synth.gpu.fill_records(shared, H, Is, wl.seed, l, -1, 1, bits=bits)
        pools.append((pool, shared, rq, rs))
        layers.append(Layer(H, E, I, k, Is, torch.from_numpy(rq).to(dev),
                            torch.from_numpy(rs.view(np.float16)).to(dev), pool, shared, act=wl.act,
                            bits=bits, **gate_kwargs(args, wl, l, dev)))
    S = NL * C  # distinct (layer, chunk) steps
    xs_host = np.empty((S, T, H))
    for l in range(NL):
        if wl.routing in ("zipf", "uniform"):
            rq, rs = pools[l][2], pools[l][3]
            W = rq.astype(np.float64) * rs.view(np.float16).astype(np.float64)[:, None]
            zr = synth.ZipfRealiser(W, wl.zipf_s, wl.seed, l)
            for c in range(C):
                xs_host[c * NL + l] = np.concatenate([zr.activations(c * T + t) for t in range(T)])
        else:
            for c in range(C):
                xs_host[c * NL + l] = synth.activations(wl.seed, l, c, H, T)
    xs_q = synth.quantize_act(xs_host, wl.act)
    xs = (torch.from_numpy(xs_q.view(np.int16)).to(dev).view(torch.bfloat16) if wl.act == "bf16"
          else torch.from_numpy(xs_q).to(dev))
    ws = layers[0].workspace(T)
    ids = torch.empty(S, T, k, dtype=torch.int32, device=dev)
    w = torch.empty(S, T, k, dtype=torch.float32, device=dev)
    y = torch.empty(S, T, H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f} s: {NL} layers x {E} experts of {rb} B, "
        f"{S} distinct chunks of {T} tokens")

    def run_step(s):
        j = s % S
        layers[j % NL].forward(xs[j], ws, out=(ids[j], w[j], y[j]))

    for s in range(S):
        run_step(s)
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    G = 1 if args.no_graph else chunk_len(K, args.graph_chunk)
    start = (W + G - 1) // G
    if args.no_graph:
        units = [(lambda s=s: run_step(s)) for s in range(start + K)]
    else:
        units = graph_units(run_step, S, G, start + K // G)
    for i in range(start):
        units[i]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(K // G):
        units[start + i]()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / K
    log(f"timed {K} steps in {ms_per_step * K:.2f} ms (wall {wall * 1e3:.2f} ms), graphs of {G} steps")

    # bytes and MFMA work of each distinct step, from the selections it made
    ids_h = ids.cpu().numpy()
    uniq = np.array([len(np.unique(ids_h[j])) for j in range(S)])
    tiles = np.array([int(sum((c + 15) // 16 for c in np.bincount(ids_h[j].ravel(), minlength=E) if c))
                      for j in range(S)])
    steps_j = [(start * G + i) % S for i in range(K)]  # distinct step of each timed step
    router_b, act_b = E * H + 2 * E, T * H * (2 if wl.act == "bf16" else 4) + T * H * 4
    step_bytes = uniq * rb + rbs + router_b + act_b
    mean_bytes = float(np.mean(step_bytes[steps_j]))
    gbps = mean_bytes / (ms_per_step * 1e-3) / 1e9
    useful_flops = 2.0 * T * 3 * H * (k * I + Is)
    shared_tiles = (T + 15) // 16 if Is else 0
    exec_flops = 2.0 * 16 * 3 * H * (tiles * I + shared_tiles * Is)
    mfma_peak = 2.5e15  # dense fp16 MFMA, MI355X
    mean_exec = float(np.mean(exec_flops[steps_j]))

    # live per-kernel pass over the S distinct steps (dispatch-stamped hipEvents)
    def profiled_steps():
        for s in range(S):
            run_step(s)

    recs = kernel_timed_pass(profiled_steps, S * 8 + 64)
    per_step_bytes = {"grouped_gate_up": uniq * gu_bytes(H, I, bits) + (gu_bytes(H, Is, bits) if Is else 0),
                      "grouped_down": uniq * down_bytes(H, I, bits) + (down_bytes(H, Is, bits) if Is else 0)}
    kernels = {}
    for name in sorted({r[0] for r in recs}):
        ms = np.array([m for n_, m in recs if n_ == name])
        ent = {"launches": int(ms.size), "avg_us": round(float(ms.mean()) * 1e3, 3),
               "p50_us": round(float(np.median(ms)) * 1e3, 3)}
        if name in per_step_bytes and ms.size == S:
            b = per_step_bytes[name]
            ent["alg_bytes_mean"] = int(b.mean())
            ent["gbps"] = round(float(b.sum()) / (float(ms.sum()) * 1e-3) / 1e9, 1)
        kernels[name] = ent
    gu = kernels["grouped_gate_up"]
    gu_flops = float(np.mean(2.0 * 16 * 2 * H * (tiles * I + shared_tiles * Is)))
    roofline = {"bound": "hbm", "achieved": gu["gbps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gu["gbps"] / PEAK_HBM_GBS, 4), "traffic": traffic_for(wl.name, "k_gu_grouped", bits),
                "kernel": "k_gu_grouped", "alg_bytes_per_launch": gu["alg_bytes_mean"],
                "avg_launch_us": gu["avg_us"], "timing": "hipExtLaunchKernelGGL start/stop events",
                "mfma_util": round(gu_flops / (gu["avg_us"] * 1e-6) / mfma_peak, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = prefill_cpu_baseline(wl, pools[0], xs_q[0], args.cpu_seconds, args)

    out = {
        "metric": "prefill tokens/s per MoE layer + achieved HBM GB/s vs peak (128-token chunk, top-8)",
        "value": round(T / (ms_per_step * 1e-3), 1), "unit": "tok/s per layer",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_desc(bits) + " (MFMA)", "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "n_experts": E, "inter": I, "top_k": k,
                   "shared_inter": Is, "chunk_tokens": T, "act": wl.act, "routing": wl.routing, "gate": gate_desc(args),
                   "bits": bits,
                   "weight_sets": NL, "distinct_chunks": S, "graph_chunk": G},
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBS, 4),
        "alg_bytes_per_chunk": int(mean_bytes), "unique_experts_mean": round(float(uniq.mean()), 2),
        "mfma_util_useful": round(useful_flops / (ms_per_step * 1e-3) / mfma_peak, 5),
        "mfma_util_executed": round(mean_exec / (ms_per_step * 1e-3) / mfma_peak, 5),
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def prefill_cpu_baseline(wl, pool, x_chunk, seconds, args):
    """The CPU oracle, token by token, on the first chunk of layer 0 (records read
    from that layer's generated pool), until about `seconds` of oracle compute."""
    import oracle
    orc = oracle.default()
    threads = orc.set_threads(len(os.sched_getaffinity(0)))
    dpool, dshared, rq, rs = pool
    H, I, Is, k = wl.hidden, wl.inter, wl.shared_inter, wl.top_k
    host = dpool.cpu().numpy()
    shared = dshared.cpu().numpy() if dshared is not None else None
    rb = host.size // wl.n_experts
    spent, n = 0.0, 0
    for t in range(x_chunk.shape[0]):
        xd = orc.act_to_f64(wl.act, x_chunk[t])
        t0 = time.perf_counter()
        ids, w, _ = oracle_route(orc, args, wl, 0, rq, rs, xd)
        yr = np.stack([orc.expert_ffn(H, I, host[int(e) * rb:(int(e) + 1) * rb], xd, bits=args.bits)
                       for e in ids])
        ys = orc.expert_ffn(H, Is, shared, xd, bits=args.bits) if Is else None
        orc.combine(w, yr, ys)
        spent += time.perf_counter() - t0
        n += 1
        if spent >= seconds:
            break
    return {"value": round(n / spent, 3), "unit": "tok/s per layer", "cores": threads, "kind": "oracle",
            "sample": f"{n} tokens of the first chunk (layer 0), one by one; fp64 plain-loop oracle, "
                      f"OpenMP over rows; {spent:.1f} s of oracle compute"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="glm_h6144_e256_l40_zipf")
    ap.add_argument("--graph-chunk", type=int, default=32,
                    help="most steps per hipGraph (the largest divisor of --steps not above it)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of hipGraphs")
    ap.add_argument("--profile-steps", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-layers", type=int, default=8,
                    help="prefill workloads: layers of distinct weights cycled over")
    ap.add_argument("--prefill-chunks", type=int, default=4,
                    help="prefill workloads: distinct input chunks per layer")
    ap.add_argument("--gate", choices=("softmax", "sigmoid"), default="softmax",
                    help="router gate: renormalised softmax (default) or the sigmoid router "
                         "(selection bias U(-0.05, 0.05) per expert, routed scale 2.5)")
    ap.add_argument("--cache-policy", choices=("lfu", "lru"), default="lfu",
                    help="slot-cache workloads: replacement policy")
    ap.add_argument("--pin", type=int, default=0,
                    help="slot-cache workloads: pin this many experts per layer, the most used "
                         "during the warm-up steps")
    ap.add_argument("--pin-source", choices=("stats", "learned"), default="stats",
                    help="slot-cache workloads: the --pin set counted on the host from the warm-up's "
                         "selections (stats) or taken by each layer from its own usage heatmap (learned)")
    ap.add_argument("--lookahead", type=int, default=0, metavar="N",
                    help="slot-cache workloads: prefetch each next layer's top N experts "
                         "from a hint (router lookahead); 0 = off")
    ap.add_argument("--lookahead-mode", choices=("ids", "call"), default="ids",
                    help="ids: route the hint with moe_route_topk and prefetch the ids after the "
                         "current layer's call (no extra host wait); call: moe_cache_prefetch")
    ap.add_argument("--bits", type=int, choices=(4, 2), default=4,
                    help="width of the expert weight codes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling the "
                         "FETCH_SIZE/WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU hot path only; runs on more than one GPU are "
              "not part of this build (see the sharding note in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    import synth
    import synth.gpu
    from bit_routed_expert_moe_amd import Layer, record_bytes, stack_forward

    wl = synth.WORKLOADS[args.workload]
    if wl.n_slots:
        return run_cached(args, wl)
    if wl.n_tokens != 1:
        return run_prefill(args, wl)
    H, E, I, k, Is, L, T = (wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter,
                            wl.n_layers, wl.n_tokens)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t_setup = time.time()
    bits = args.bits
    rb = record_bytes(H, I, bits)
    layers, pools = [], []
    for l in range(L):
        rq, rs = synth.router(wl.seed, l, E, H)
        pool = torch.empty(E * rb, dtype=torch.uint8, device=dev)
        synth.gpu.fill_records(pool, H, I, wl.seed, l, 0, E, bits=bits)
        shared = None
        if Is:
            shared = torch.empty(record_bytes(H, Is, bits), dtype=torch.uint8, device=dev)
            synth.gpu.fill_records(shared, H, Is, wl.seed, l, -1, 1, bits=bits)
        pools.append((pool, shared, rb))
        layers.append(Layer(H, E, I, k, Is, torch.from_numpy(rq).to(dev),
                            torch.from_numpy(rs.view(np.float16)).to(dev), pool, shared, act=wl.act,
                            bits=bits, **gate_kwargs(args, wl, l, dev)))
    S = wl.steps
    xs_host = np.stack([make_inputs(wl, l, S) for l in range(L)], axis=1)  # [S][L][T][H]
    xs_q = synth.quantize_act(xs_host, wl.act)
    if wl.act == "bf16":
        xs = torch.from_numpy(xs_q.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        xs = torch.from_numpy(xs_q).to(dev)
    ws = layers[0].workspace(T)
    ids = torch.empty(S, L, T, k, dtype=torch.int32, device=dev)
    w = torch.empty(S, L, T, k, dtype=torch.float32, device=dev)
    y = torch.empty(S, L, T, H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f} s: {L} layers, {E} experts of {rb} B, "
        f"{S} distinct steps")

    def run_step(s):
        stack_forward(layers, xs[s], ws, out=(ids[s], w[s], y[s]))

    run_step(0)
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    G = 1 if args.no_graph else chunk_len(K, args.graph_chunk)
    start = (W + G - 1) // G
    if args.no_graph:  # callables, each running G consecutive steps
        units = [(lambda s=s: run_step(s % S)) for s in range(start + K)]
    else:
        units = graph_units(run_step, S, G, start + K // G)
    for i in range(start):
        units[i]()
    torch.cuda.synchronize()

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K // G + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(K // G):
        units[start + i]()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = evs[0].elapsed_time(evs[-1])
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) / G for i in range(K // G)])
    ms_per_step = total_ms / K
    log(f"timed {K} steps in {total_ms:.2f} ms (wall {wall * 1e3:.2f} ms), graphs of {G} steps")

    tl_bytes = token_layer_bytes(wl, bits)
    sel_bytes = wl.top_k * record_bytes(H, I, bits)
    step_bytes = L * T * tl_bytes
    layer_tok_s = L * T / (ms_per_step * 1e-3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    # live per-kernel pass over the same steps (dispatch-stamped hipEvents)
    P = min(args.profile_steps, S)

    def profiled_steps():
        for s in range(P):
            run_step(s)

    recs = kernel_timed_pass(profiled_steps, P * L * 4 + 64)
    # up to hidden 4096 the resident forward routes inside the gate/up launch
    # (no route launch): that launch then also reads the router
    fused_route = "route" not in {r[0] for r in recs}
    kbytes = launch_bytes(wl, bits, T, fused_route)
    kernels = {}
    for name in sorted({r[0] for r in recs}):
        ms = np.array([m for n_, m in recs if n_ == name])
        net = float(ms.mean())
        ent = {"launches": int(ms.size), "avg_us": round(net * 1e3, 3),
               "p50_us": round(float(np.median(ms)) * 1e3, 3)}
        if name in kbytes:
            ent["alg_bytes"] = int(kbytes[name])
            ent["gbps"] = round(kbytes[name] / (net * 1e-3) / 1e9, 1)
        kernels[name] = ent
    kfn = "k_gate_up"
    gu = kernels["gate_up"]
    roofline = {"bound": "hbm", "achieved": gu["gbps"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gu["gbps"] / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(wl.name, kfn, bits),
                "kernel": kfn, "alg_bytes_per_launch": gu["alg_bytes"], "routing_in_launch": fused_route,
                "avg_launch_us": gu["avg_us"], "timing": "hipExtLaunchKernelGGL start/stop events"}

    achievable = stream_reference(pools, tl_bytes, P)
    roofline["achievable"] = achievable["gbps"]
    roofline["frac_of_achievable"] = round(gu["gbps"] / achievable["gbps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, xs_q, args.cpu_seconds, args, pools)

    out = {
        "metric": METRIC, "value": round(layer_tok_s, 1), "unit": "tok/s per layer",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_desc(bits), "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "n_experts": E, "inter": I, "top_k": k,
                   "shared_inter": Is, "layers": L, "batch": T, "act": wl.act, "bits": bits,
                   "routing": wl.routing, "gate": gate_desc(args), "graph_chunk": G},
        "stack_tok_s": round(T / (ms_per_step * 1e-3), 2),
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBS, 4),
        "alg_bytes_per_token_layer": tl_bytes,
        # the selected records alone (no router, no shared record)
        "selected_bytes_per_token_layer": sel_bytes,
        "hbm_gbps_selected_only": round(L * T * sel_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_ms_percentiles_over": f"{K // G} timed graph replays of {G} steps (per-step means)",
        "step_ms_p50": round(float(np.percentile(per_step, 50)), 5),
        "step_ms_p95": round(float(np.percentile(per_step, 95)), 5),
        "step_ms_p99": round(float(np.percentile(per_step, 99)), 5),
        "hbm_frac_of_achievable": round(gbps / achievable["gbps"], 4),
        "stream_reference": achievable,
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
