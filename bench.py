#!/usr/bin/env python3
"""Benchmark of the kernelized linear-attention hot path on one MI355X.

A step is one causal forward plus one causal backward (la_forward_causal +
la_backward_causal through the C ABI, the backward reading the carried state
the forward saved, as a training step would) over the workload B=4, H=16, N=4096,
d=64, bf16 inputs ~ N(0,1)/sqrt(d), chunk 64.  W untimed warmup steps, then K
steps timed back to back between two device synchronisations.  Inputs are
resident in HBM before the timed region; the step rotates over several input
sets whose total exceeds the 256 MB last-level cache, so each step starts with
its inputs in HBM, not in cache.  Before the W warmup steps, untimed steps run
for 0.5 s of GPU time: the first milliseconds of work after start-up run while
the GPU clock ramps up and read about 5-10% slow, which a short run (K = 20)
would otherwise time.  Launches are eager; with
--graph each input set's step is captured once into a HIP graph and the timed
region replays the graphs (every graph's replays are first checked bitwise
against eager steps; on this stack replays measure a few microseconds slower
per step).  The per-kernel event times come from a second, eager run of the
same K steps right after the timed one.

The JSON line also carries
  * roofline    : the dominant kernel's algorithmic bytes per launch over its
                  average duration (HIP events around every launch, recorded
                  on the library's stream over a second run of the timed steps) against the
                  8 TB/s HBM peak; step_frac / step_achieved inside it: the whole
                  step (22 d bytes per token-head) over the timed step time;
  * step_roofline: the same for the whole step (22 d bytes per token-head);
  * calls       : the other measured calls (non-causal forward, non-causal
                  forward + backward, and the causal forward on FAVOR+ random
                  features, at the same size; the long and very-long
                  causal workloads; 512 decode steps one per call, 16 per
                  call, and 16 per call with 32 query heads on 4 shared
                  key/value states), each with its throughput and roofline
                  fraction;
  * cpu_baseline: the fp64 CPU oracle timed on this host on repeated full
                  steps of the same workload (bounded to about 10 s); each
                  entry of calls carries the same for its own workload
                  (cpu_oracle: about 1.5 s on a sample of heads or steps).

The roofline's "traffic" is the dominant kernel's measured HBM bytes per
launch: FETCH_SIZE and WRITE_SIZE from two rocprofv3 counter passes over this
script, each divided by the factor the same counter reads for a plain copy of
known size (`--copy-probe`).  They are read from profiles/<kernel>_traffic.txt,
which records a hash of the kernel sources; when the sources have changed since
the counters were taken the field is null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-calls] [--no-cpu] [--graph]
       python bench.py --copy-probe      (a 256 MiB device copy, for counter calibration)
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LLC_BYTES = 256 * 2**20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-calls", action="store_true", help="skip the other calls")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--graph", action="store_true", help="time HIP-graph replays of the steps instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true", help="only run 5 device copies of 256 MiB")
    return ap.parse_args()


COPY_PROBE_BYTES = 256 * 2**20


def copy_probe(torch):
    """Five copies of COPY_PROBE_BYTES between two device buffers (counter calibration)."""
    src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 5}), flush=True)


def kernel_source_hash():
    """sha256 over the HIP sources and headers the library is built from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/<kernel>_traffic.txt, or None if
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def kernel_stats(entries):
    """{name: (launches, total ms)} from the library's per-launch events."""
    out = {}
    for name, ms in entries:
        n, t = out.get(name, (0, 0.0))
        out[name] = (n + 1, t + ms)
    return out


def unit_bytes(B, H, N, d, esize=2):
    return B * H * N * d * esize


# Algorithmic bytes per launch of each kernel, in [B,H,N,d] tensors read or
# written through the ABI (workspace traffic is not algorithmic).
# The fused backward reads q, k, v, dO and writes dq, dk, dv: 7 units (its second
# sweep's re-reads of the segment are not algorithmic traffic).
KERNEL_UNITS = {"seg_state": 2, "causal_fwd": 4, "causal_fwd_fused": 4, "noncausal_fwd": 2, "bwd_prefix": 5, "bwd_suffix": 6, "bwd_fused": 7,
                "ncbwd_q": 3, "ncbwd_kv": 4}


def sequence_roofline(stats, B, H, N, d, steps):
    name = max(stats, key=lambda k: stats[k][1])
    n, tot = stats[name]
    avg_s = tot / n * 1e-3
    units = KERNEL_UNITS.get(name)
    if units is None:
        return name, None
    alg = units * unit_bytes(B, H, N, d)
    ach = alg / avg_s / 1e9
    return name, {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                  "kernel": name, "launches": n, "avg_us": round(avg_s * 1e6, 2),
                  "alg_bytes_per_launch": alg}


PREWARM_S = 0.5


def prewarm(run, nsets, torch, seconds=PREWARM_S):
    """Untimed steps for `seconds` of GPU time before the warmup steps: the first
    milliseconds of work after start-up run while the GPU clock ramps up, and a run
    of a few dozen steps would otherwise be timed on the ramp."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            run(i % nsets)
            i += 1
        torch.cuda.synchronize()
    return i


def time_steps(fn, nsets, warmup, steps, la, torch, timed_fn=None, warm_s=0.0):
    """Wall time of `steps` back-to-back steps, then per-kernel event times over a second run of them.

    timed_fn (default fn) is what the timed region runs per step, e.g. the replay of
    a captured graph of fn; the per-kernel event run always calls fn itself.
    warm_s: seconds of untimed steps before the warmup steps."""
    run = timed_fn or fn
    if warm_s > 0:
        prewarm(run, nsets, torch, warm_s)
    for i in range(warmup):
        run(i % nsets)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i % nsets)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    la.profile_enable(True)
    for i in range(steps):
        fn(i % nsets)
    torch.cuda.synchronize()
    stats = kernel_stats(la.profile_entries())
    la.profile_enable(False)
    return dt, stats


def capture_graphs(step, nsets, outputs, torch):
    """One HIP graph per input set of step(i) (all its kernel launches), or None.

    Every graph is replayed twice, with the eager step of another set and a
    synchronisation between the replays, and each replay's outputs must equal
    the eager step's outputs bitwise (the kernels are deterministic); otherwise
    the bench keeps eager launches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsets):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(nsets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(nsets):
        step(i)
        ref = [t.clone() for t in outputs]
        for _ in range(2):
            step((i + 1) % nsets)
            torch.cuda.synchronize()
            graphs[i].replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outputs, ref)):
                return None
    return graphs


def bench_mid(args, la, inp, torch):
    w = inp.MID
    B, H, N, d = w.B, w.H, w.N, w.d
    per_set = 4 * unit_bytes(B, H, N, d)
    nsets = max(2, math.ceil(2 * LLC_BYTES / per_set))
    sets = [inp.workload_inputs(w, seed=s, device="cuda", with_dout=True) for s in range(nsets)]
    o = torch.empty_like(sets[0][0])
    grads = tuple(torch.empty_like(sets[0][0]) for _ in range(3))
    wsf = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, B, H, N, d, w.dtype), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(la.workspace_size(la.LA_OP_BWD_CAUSAL, B, H, N, d, w.dtype), dtype=torch.uint8, device="cuda")
    saved = la.new_saved_state(sets[0][0])

    def step(i):
        q, k, v, do = sets[i]
        la.la_forward_causal(q, k, v, out=o, workspace=wsf, saved_state=saved)
        la.la_backward_causal(q, k, v, do, out=grads, workspace=wsb, saved_state=saved)

    graphs = capture_graphs(step, nsets, (o,) + grads, torch) if args.graph else None
    replay = None if graphs is None else (lambda i: graphs[i].replay())
    dt, stats = time_steps(step, nsets, args.warmup, args.steps, la, torch, timed_fn=replay, warm_s=PREWARM_S)
    T = B * H * N
    step_s = dt / args.steps
    step_bytes = 11 * unit_bytes(B, H, N, d)
    flops = 14 * d * d * T
    kname, roof = sequence_roofline(stats, B, H, N, d, args.steps)
    if roof is not None:
        # the whole step beside the dominant kernel: 11 units (22 d bytes per token-head)
        roof["step_achieved"] = round(step_bytes / step_s / 1e9, 1)
        roof["step_frac"] = round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4)
        roof["step_alg_bytes"] = step_bytes
    return {
        "value": B * N * args.steps / dt,
        "ms_per_step": step_s * 1e3,
        "roofline": roof,
        "step_roofline": {"bound": "hbm", "alg_bytes": step_bytes,
                          "achieved": round(step_bytes / step_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                          "frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                          "alg_tflops": round(flops / step_s / 1e12, 2),
                          "mfma_frac": round(flops / step_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
        "kernels_us": {k: round(t / n * 1e3, 2) for k, (n, t) in sorted(stats.items())},
        "input_sets": nsets,
        "launch": "hip_graph" if graphs is not None else "eager",
    }, sets


def bench_call(name, fn, warmup, steps, tokens, alg_bytes, la, torch, nsets=1):
    dt, stats = time_steps(fn, nsets, warmup, steps, la, torch)
    s = dt / steps
    return {"tokens_per_s": round(tokens / s, 1), "ms": round(s * 1e3, 4),
            "alg_bytes": alg_bytes, "achieved_GBs": round(alg_bytes / s / 1e9, 1),
            "hbm_frac": round(alg_bytes / s / 1e9 / HBM_PEAK_GBS, 4),
            "kernels_us": {k: round(t / n * 1e3, 2) for k, (n, t) in sorted(stats.items())}}


def bench_calls(args, la, inp, torch, mid_sets):
    calls = {}
    w = inp.MID
    # The Mid calls rotate over the headline step's input sets (together larger than
    # the last-level cache), so each call reads its inputs from HBM.
    nsets = len(mid_sets)
    q0 = mid_sets[0][0]
    o = torch.empty_like(q0)
    ws = torch.empty(la.workspace_size(la.LA_OP_FWD_NONCAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                     device="cuda")

    def nc_fwd(i):
        q, k, v, _ = mid_sets[i]
        la.la_forward_noncausal(q, k, v, out=o, workspace=ws)

    calls["mid_noncausal_fwd"] = bench_call("noncausal", nc_fwd, 100, 400, w.B * w.N,
                                            4 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    # Non-causal training step: forward saving the key aggregates, backward reading them
    # (the forward reads q, k, v and writes o; the backward reads q, k, v, dout and writes dq, dk, dv: 11 units).
    g = tuple(torch.empty_like(q0) for _ in range(3))
    wsb = torch.empty(la.workspace_size(la.LA_OP_BWD_NONCAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")
    saved = la.new_saved_state(q0)

    def nc_step(i):
        q, k, v, do = mid_sets[i]
        la.la_forward_noncausal(q, k, v, out=o, workspace=ws, saved_state=saved)
        la.la_backward_noncausal(q, k, v, do, out=g, workspace=wsb, saved_state=saved)

    calls["mid_noncausal_fwd_bwd"] = bench_call("noncausal_step", nc_step, 100, 400, w.B * w.N,
                                                11 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    del o, ws, g, wsb, saved

    # Causal forward on FAVOR+ random features (m = d) at the Mid shape: the feature
    # kernel on q and k, then the causal forward on the features.  Algorithmic bytes:
    # q, k, v read and o written (4 units); the two feature passes add 4 more.
    fsets = [inp.favor_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=s, device="cuda") for s in range(nsets)]
    om = inp.favor_omega(w.d, seed=0, device="cuda")
    fq, fk = torch.empty_like(q0), torch.empty_like(q0)
    o = torch.empty_like(q0)
    wsf = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")

    def favor_fwd(i):
        q, k, v = fsets[i]
        la.favor_features(q, om, out=fq)
        la.favor_features(k, om, out=fk)
        la.la_forward_causal_features(fq, fk, v, out=o, workspace=wsf)

    calls["mid_favor_causal_fwd"] = bench_call("favor", favor_fwd, 100, 400, w.B * w.N,
                                               4 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    del fq, fk, wsf

    # The same with m = 2d random features (two feature blocks per head): algorithmic
    # bytes q, k, v read and o written (4 units); the features add 2 x (1 + 2) units.
    m = 2 * w.d
    om2 = inp.favor_omega(w.d, seed=0, device="cuda", m=m)
    fq = torch.empty((w.B, w.H, 2, w.N, w.d), dtype=w.dtype, device="cuda")
    fk = torch.empty_like(fq)
    wsf = torch.empty(la.features_workspace_size(True, w.B, w.H, w.N, w.d, m, w.dtype), dtype=torch.uint8,
                      device="cuda")

    def favor_fwd_m2(i):
        q, k, v = fsets[i]
        la.favor_features_blocks(q, om2, out=fq)
        la.favor_features_blocks(k, om2, out=fk)
        la.la_forward_causal_features_blocks(fq, fk, v, out=o, workspace=wsf)

    calls["mid_favor_m128_causal_fwd"] = bench_call("favor_m2", favor_fwd_m2, 100, 400, w.B * w.N,
                                                    4 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    # Its backward on the features (m = 2d): the head's g from the forward's output, the blocks' sweeps.
    # Algorithmic bytes: q, k features (2 units each), v, dout read; their gradients written (8 units).
    o2, den2 = la.la_forward_causal_features_blocks(fq, fk, fsets[0][2], return_den=True)
    g2 = (torch.empty_like(fq), torch.empty_like(fk), torch.empty_like(q0))
    dos2 = [inp.normal((w.B, w.H, w.N, w.d), inp.generator(60 + s, "cuda"), w.dtype, 1.0, "cuda") for s in range(nsets)]
    wsb2 = torch.empty(la.features_workspace_size(3, w.B, w.H, w.N, w.d, m, w.dtype), dtype=torch.uint8, device="cuda")

    def favor_bwd_m2(i):
        la.la_backward_causal_features_blocks(fq, fk, fsets[i][2], dos2[i], den2, o=o2, out=g2, workspace=wsb2)

    calls["mid_favor_m128_causal_bwd"] = bench_call("favor_m2_bwd", favor_bwd_m2, 100, 400, w.B * w.N,
                                                    8 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    # A non-causal FAVOR+ training step with m = 2d: block features of q and k, the forward, its
    # backward on the features, the feature map's backward.  Algorithmic bytes: the 8 units of the
    # attention's own inputs and gradients (q, k, v, dout read; o, dq, dk, dv written).
    wsn = torch.empty(la.features_workspace_size(False, w.B, w.H, w.N, w.d, m, w.dtype), dtype=torch.uint8,
                      device="cuda")
    wsn_b = torch.empty(la.features_workspace_size(4, w.B, w.H, w.N, w.d, m, w.dtype), dtype=torch.uint8,
                        device="cuda")
    dq2, dk2 = torch.empty_like(q0), torch.empty_like(q0)

    def favor_train_nc_m2(i):
        q, k, v = fsets[i]
        la.favor_features_blocks(q, om2, out=fq)
        la.favor_features_blocks(k, om2, out=fk)
        la.la_forward_noncausal_features_blocks(fq, fk, v, out=o, workspace=wsn, den_out=den2)
        la.la_backward_noncausal_features_blocks(fq, fk, v, dos2[i], den2, o=o, out=g2, workspace=wsn_b)
        la.favor_features_blocks_backward(q, om2, fq, g2[0], out=dq2)
        la.favor_features_blocks_backward(k, om2, fk, g2[1], out=dk2)

    calls["mid_favor_m128_noncausal_fwd_bwd"] = bench_call("favor_m2_nc_train", favor_train_nc_m2, 50, 200, w.B * w.N,
                                                           8 * unit_bytes(w.B, w.H, w.N, w.d), la, torch,
                                                           nsets=nsets)
    del fq, fk, wsf, o2, den2, g2, dos2, wsb2, wsn, wsn_b, dq2, dk2

    # A FAVOR+ training step (m = d): features of q and k, the causal forward on them, its
    # backward on the features, and the gradient through the feature map for q and k.
    # Algorithmic bytes: q, k, v, dout read and o, dq, dk, dv written (8 units).
    fq, fk = torch.empty_like(q0), torch.empty_like(q0)
    gfe = tuple(torch.empty_like(q0) for _ in range(3))
    dq, dk = torch.empty_like(q0), torch.empty_like(q0)
    dos = [inp.normal((w.B, w.H, w.N, w.d), inp.generator(50 + s, "cuda"), w.dtype, 1.0, "cuda") for s in range(nsets)]
    wsf = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(la.workspace_size(la.LA_OP_BWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")

    def favor_step(i):
        q, k, v = fsets[i]
        la.favor_features(q, om, out=fq)
        la.favor_features(k, om, out=fk)
        la.la_forward_causal_features(fq, fk, v, out=o, workspace=wsf)
        la.la_backward_causal_features(fq, fk, v, dos[i], out=gfe, workspace=wsb)
        la.favor_features_backward(q, om, fq, gfe[0], out=dq)
        la.favor_features_backward(k, om, fk, gfe[1], out=dk)

    calls["mid_favor_causal_fwd_bwd"] = bench_call("favor_step", favor_step, 100, 400, w.B * w.N,
                                                   8 * unit_bytes(w.B, w.H, w.N, w.d), la, torch, nsets=nsets)
    del fsets, fq, fk, o, wsf, wsb, gfe, dq, dk, dos

    w = inp.LONG
    q, k, v, do = inp.workload_inputs(w, seed=0, device="cuda", with_dout=True)
    o = torch.empty_like(q)
    g = tuple(torch.empty_like(q) for _ in range(3))
    wsf = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(la.workspace_size(la.LA_OP_BWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")
    saved = la.new_saved_state(q)

    def long_step(i):
        la.la_forward_causal(q, k, v, out=o, workspace=wsf, saved_state=saved)
        la.la_backward_causal(q, k, v, do, out=g, workspace=wsb, saved_state=saved)

    calls["long_causal_fwd_bwd"] = bench_call("long", long_step, 2, 10, w.B * w.N,
                                              11 * unit_bytes(w.B, w.H, w.N, w.d), la, torch)
    del q, k, v, do, o, g, wsf, wsb, saved

    w = inp.VERYLONG
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    q, k, v = inp.workload_inputs(w, seed=0, device="cuda", with_dout=False)
    o = torch.empty_like(q)
    wsf = torch.empty(la.workspace_size(la.LA_OP_FWD_CAUSAL, w.B, w.H, w.N, w.d, w.dtype), dtype=torch.uint8,
                      device="cuda")
    r = bench_call("verylong", lambda i: la.la_forward_causal(q, k, v, out=o, workspace=wsf), 2, 10, w.B * w.N,
                   4 * unit_bytes(w.B, w.H, w.N, w.d), la, torch)
    r["peak_mem_bytes"] = int(torch.cuda.max_memory_allocated() - base)
    r["workspace_bytes"] = int(wsf.numel())
    r["state_bytes_per_head"] = (w.d * w.d + w.d) * 4
    r["softmax_matrix_bytes_per_head_bf16"] = w.N * w.N * 2
    calls["verylong_causal_fwd"] = r
    del q, k, v, o, wsf

    w = inp.DECODE
    B, H, d = w.batch, w.H, w.d
    S = torch.empty(B, H, d, d, device="cuda")
    z = torch.empty(B, H, d, device="cuda")
    nb = 32
    for b0 in range(0, B, nb):
        pq, pk, pv = inp.qkv(nb, H, w.prefix, d, w.dtype, seed=1000 + b0, device="cuda")
        _, Sb, zb = la.la_forward_causal(pq, pk, pv, return_state=True)
        S[b0:b0 + nb].copy_(Sb)
        z[b0:b0 + nb].copy_(zb)
        del pq, pk, pv
    sq, sk, sv = inp.decode_tokens(B, H, d, w.steps, w.dtype, seed=2, device="cuda")
    od = torch.empty(B, H, d, dtype=w.dtype, device="cuda")

    def span(i):
        for t in range(w.steps):
            la.la_decode_step(S, z, sq[t], sk[t], sv[t], out=od)

    step_bytes = B * H * (2 * 4 * d * d + 2 * 4 * d + 4 * 2 * d)
    r = bench_call("decode", span, 1, 3, B * w.steps, step_bytes * w.steps, la, torch)
    r["tokens_per_s"] = r.pop("tokens_per_s")
    r["us_per_step"] = round(r["ms"] * 1e3 / w.steps, 2)
    r["alg_bytes_per_step"] = step_bytes
    calls["decode_512_steps"] = r

    # The same 512 tokens per sequence through la_decode_steps, TPC tokens per call:
    # the state moves once per call (2 * 4 d^2 + 2 * 4 d bytes per head) plus TPC
    # tokens of q, k, v, o (4 * 2 d bytes each).
    TPC = 16
    calls_n = w.steps // TPC
    blocks = [tuple(t[c * TPC:(c + 1) * TPC].permute(1, 2, 0, 3).contiguous() for t in (sq, sk, sv))
              for c in range(calls_n)]
    ob = torch.empty(B, H, TPC, d, dtype=w.dtype, device="cuda")

    def span_multi(i):
        for c in range(calls_n):
            bq, bk, bv = blocks[c]
            la.la_decode_steps(S, z, bq, bk, bv, out=ob)

    call_bytes = B * H * (2 * 4 * d * d + 2 * 4 * d + TPC * 4 * 2 * d)
    r = bench_call("decode_steps", span_multi, 1, 3, B * calls_n * TPC, call_bytes * calls_n, la, torch)
    r["tokens_per_call"] = TPC
    r["us_per_call"] = round(r["ms"] * 1e3 / calls_n, 2)
    r["us_per_token_step"] = round(r["ms"] * 1e3 / (calls_n * TPC), 2)
    r["alg_bytes_per_call"] = call_bytes
    calls[f"decode_512_steps_{TPC}_per_call"] = r

    # Grouped heads: the same 32 query heads per sequence read 4 shared key/value states
    # (8 query heads per state), so a call moves a quarter of the state bytes.
    HKV = 4
    Sg = S[:, :HKV].contiguous()
    zg = z[:, :HKV].contiguous()
    gblocks = [(bq, bk[:, :HKV].contiguous(), bv[:, :HKV].contiguous()) for bq, bk, bv in blocks]

    def span_grouped(i):
        for c in range(calls_n):
            bq, bk, bv = gblocks[c]
            la.la_decode_steps(Sg, zg, bq, bk, bv, out=ob)

    gcall_bytes = B * (HKV * (2 * 4 * d * d + 2 * 4 * d + TPC * 2 * 2 * d) + H * TPC * 2 * 2 * d)
    r = bench_call("decode_steps_gqa", span_grouped, 1, 3, B * calls_n * TPC, gcall_bytes * calls_n, la, torch)
    r["tokens_per_call"] = TPC
    r["kv_heads"] = HKV
    r["us_per_call"] = round(r["ms"] * 1e3 / calls_n, 2)
    r["us_per_token_step"] = round(r["ms"] * 1e3 / (calls_n * TPC), 2)
    r["alg_bytes_per_call"] = gcall_bytes
    calls[f"decode_512_steps_{TPC}_per_call_{H}q_{HKV}kv"] = r
    return calls


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_share():
    """Host threads the oracle may use: every core this process may run on, within the
    thread count the host grants the job (OMP_NUM_THREADS, when set)."""
    n = len(os.sched_getaffinity(0))
    try:
        omp = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        omp = 0
    return min(n, omp) if omp > 0 else n


def cpu_baseline(args, inp, torch, mid_set):
    import oracle

    w = inp.MID
    q, k, v, do = (inp.to_f64(t) for t in mid_set)
    # the host's share of cores, capped at the heads (the oracle's parallelism)
    cores = min(cpu_share(), w.B * w.H)
    oracle.set_threads(cores)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward_causal(q, k, v)
        oracle.backward_causal(q, k, v, do)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(reps * w.B * w.N / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"{reps} full causal fwd+bwd steps of B4 H16 N4096 d64 (all 64 heads), fp64, "
                      f"{dt:.1f} s wall"}


def call_oracles(args, inp, torch):
    """The fp64 oracle timed on a bounded sample of each call's workload (a few heads, or
    a few decode steps), as tokens/s of the whole workload: sample token-heads per
    second divided by the workload's heads per token."""
    import oracle

    cores = cpu_share()
    f64 = inp.to_f64

    def rate(fn, token_heads, heads_per_token, budget=1.5):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        return round(reps * token_heads / heads_per_token / dt, 1), reps, dt

    out = {}

    def record(name, fn, token_heads, heads_per_token, threads, what):
        # all affinity cores, capped at the sample's heads (the oracle's parallelism)
        oracle.set_threads(min(cores, threads))
        v, reps, dt = rate(fn, token_heads, heads_per_token)
        out[name] = {"value": v, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
                     "cpu": cpu_model(), "sample": f"{reps} x {what}, fp64, {dt:.1f} s wall"}

    w = inp.MID
    hs = 8
    q, k, v, do = (f64(t) for t in inp.qkv(1, hs, w.N, w.d, torch.float32, seed=90, with_dout=True))
    record("mid_noncausal_fwd", lambda: oracle.forward_noncausal(q, k, v), hs * w.N, w.H,
           hs, f"non-causal forward of {hs} of the 64 Mid heads")
    record("mid_noncausal_fwd_bwd", lambda: (oracle.forward_noncausal(q, k, v), oracle.backward_noncausal(q, k, v, do)),
           hs * w.N, w.H, hs, f"non-causal forward + backward of {hs} Mid heads")
    fq, fk, fv = (f64(t) for t in inp.favor_qkv(1, hs, w.N, w.d, torch.float32, seed=91))
    om = f64(inp.favor_omega(w.d, seed=0))
    record("mid_favor_causal_fwd",
           lambda: oracle.forward_features(oracle.favor_features(fq, om), oracle.favor_features(fk, om), fv, True),
           hs * w.N, w.H, hs, f"FAVOR+ features + causal forward of {hs} Mid heads")
    fdo = f64(inp.normal((1, hs, w.N, w.d), inp.generator(94), torch.float32, 1.0))

    def favor_train():
        rfq, rfk = oracle.favor_features(fq, om), oracle.favor_features(fk, om)
        oracle.forward_features(rfq, rfk, fv, True)
        gq, gk, _ = oracle.backward_features(rfq, rfk, fv, fdo, True)
        oracle.favor_features_backward(fq, om, gq)
        oracle.favor_features_backward(fk, om, gk)

    record("mid_favor_causal_fwd_bwd", favor_train, hs * w.N, w.H, hs,
           f"FAVOR+ features, causal forward and backward, feature-map backward of {hs} Mid heads")
    om2 = f64(inp.favor_omega(w.d, seed=0, m=2 * w.d))
    def favor_m2_bwd():
        rfq, rfk = oracle.favor_features(fq, om2), oracle.favor_features(fk, om2)
        oracle.backward_features(rfq, rfk, fv, fdo, True)

    record("mid_favor_m128_causal_bwd", favor_m2_bwd, hs * w.N, w.H, hs,
           f"FAVOR+ features (m = 2d) and the causal backward on them, {hs} Mid heads")

    def favor_m2_nc_train():
        rfq, rfk = oracle.favor_features(fq, om2), oracle.favor_features(fk, om2)
        oracle.forward_features(rfq, rfk, fv, False)
        gq, gk, _ = oracle.backward_features(rfq, rfk, fv, fdo, False)
        oracle.favor_features_backward(fq, om2, gq)
        oracle.favor_features_backward(fk, om2, gk)

    record("mid_favor_m128_noncausal_fwd_bwd", favor_m2_nc_train, hs * w.N, w.H, hs,
           f"FAVOR+ features (m = 2d), non-causal forward and backward, feature-map backward of {hs} Mid heads")
    record("mid_favor_m128_causal_fwd",
           lambda: oracle.forward_features(oracle.favor_features(fq, om2), oracle.favor_features(fk, om2), fv, True),
           hs * w.N, w.H, hs, f"FAVOR+ features (m = 2d) + causal forward of {hs} Mid heads")
    L = inp.LONG
    hl = 4
    q, k, v, do = (f64(t) for t in inp.qkv(1, hl, L.N, L.d, torch.float32, seed=92, with_dout=True))
    record("long_causal_fwd_bwd", lambda: (oracle.forward_causal(q, k, v), oracle.backward_causal(q, k, v, do)),
           hl * L.N, L.H, hl, f"causal forward + backward of {hl} of the 128 Long heads")
    V = inp.VERYLONG
    q, k, v = (f64(t) for t in inp.qkv(1, 2, V.N // 8, V.d, torch.float32, seed=93))
    record("verylong_causal_fwd", lambda: oracle.forward_causal(q, k, v), 2 * (V.N // 8), V.H,
           2, f"causal forward of 2 heads over the first {V.N // 8} tokens of a Very long head")
    D = inp.DECODE
    hd, steps = 64, 32
    S0 = np.abs(np.random.default_rng(94).standard_normal((hd, D.d, D.d))) + 1.0
    z0 = np.abs(np.random.default_rng(95).standard_normal((hd, D.d))) * 100 + 100.0
    sq, sk, sv = (f64(t) for t in inp.decode_tokens(1, hd, D.d, steps, torch.float32, seed=96))

    def dec():
        S, z = S0, z0
        for t in range(steps):
            _, S, z = oracle.decode_step(S, z, sq[t, 0], sk[t, 0], sv[t, 0])

    record("decode", dec, hd * steps, D.H, hd, f"{steps} decode steps of {hd} head-states")
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(torch)
        return

    import la_inputs as inp
    import linear_attention_02_amd as la

    la.load_library()
    torch.cuda.set_device(0)
    res, mid_sets = bench_mid(args, la, inp, torch)
    calls = None if args.no_calls else bench_calls(args, la, inp, torch, mid_sets)
    cpu = None if args.no_cpu else cpu_baseline(args, inp, torch, mid_sets[0])
    if calls is not None and not args.no_cpu:
        orc = call_oracles(args, inp, torch)
        for name, r in calls.items():
            key = "decode" if name.startswith("decode") else name
            if key in orc:
                r["cpu_oracle"] = orc[key]
    line = {
        "metric": "causal LA fwd+bwd tokens/s, B4 H16 N4096 d64 bf16; % of HBM/MFMA roofline",
        "value": round(res["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal linear attention fwd+bwd, B4 H16 N4096 d64, bf16 in / fp32 accumulate, "
                               "phi = elu+1, chunk 64", "global_batch": 4, "seq_len": 4096, "heads": 16,
                   "head_dim": 64, "parallelism": "single GPU", "launch": res["launch"]},
        "roofline": res["roofline"],
        "step_roofline": res["step_roofline"],
        "kernels_us": res["kernels_us"],
        "calls": calls,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
