#!/usr/bin/env python3
"""Throughput of the MoE feed-forward layer on one MI355X.

A step is one pass of the whole layer over one batch of seeded synthetic
input resident in HBM: one moe_layer call (route and permute -> routed
experts -> combine, with the shared expert on a side stream beside them); for
the Refill-RMS workload: route with the 11th expert -> permute -> routed
experts (fp32 rows) -> refill score -> keep-set.  Steps cycle through
several independently generated weight copies so that the weights do not stay
in the 256 MB on-die cache between steps.

Prints one JSON line: tokens/s; the roofline position of the dominant kernel
(the routed grouped-expert call, timed with HIP events on its stream inside
the timed region); the roofline position of the whole layer (its algorithmic
flops or bytes over the wall time of a step); the same figures for the
16-token W4A16 decode layer, measured in the same process; and the oracle's
CPU throughput on a bounded sample.

The default workload is the expert-pruned W4A16 layer over one packed row of
32768 tokens (256 of 512 experts kept, top-10, hidden 2560, width 640), the
largest configuration that fits one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) / MFMA TFLOP/s (prefill), % of peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
EV_EVERY = 8                 # timed steps between two recorded pairs of routed-call events

# bytes of one expert's weights (gate + up + down)
def expert_bytes(w, fmt):
    n = 3 * w.H * w.F
    if fmt == "bf16":
        return 2 * n
    if fmt == "fp8":  # one byte per weight + an fp32 scale per 128 x 128 block
        return n + 4 * (n // (128 * 128))
    if fmt == "nvfp4":  # 4-bit codes + an E4M3 scale per 16 weights + 3 fp32 global scales
        return n // 2 + n // 16 + 3 * 4
    # AWQ g32: 4-bit codes + fp16 scale per (group, column) + 4-bit zero per (group, column)
    return n // 2 + 2 * (n // 32) + (n // 32) // 2


def source_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_expert_router_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="pruned_awq",
                   help="tiny_bf16, decode_bf16, decode_awq, decode_fp8, decode_nvfp4, prefill_awq, "
                        "prefill_fp8, prefill_nvfp4, pruned_awq, refill_bf16")
    p.add_argument("--copies", type=int, default=0, help="weight copies to cycle (0: auto)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of the oracle CPU-baseline sample (0 disables it)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--graph", choices=["on", "off"], default="off",
                   help="replay each layer step from one HIP graph (captured moe_layer call, side "
                        "stream included); the roofline events then bracket the whole replay")
    p.add_argument("--shared-stream", choices=["on", "off"], default="on",
                   help="run the shared expert on a side stream beside the routed path (on) or on "
                        "the main stream before it (off)")
    p.add_argument("--secondary", default="decode_awq",
                   help="a second workload measured in the same process ('none' skips it)")
    p.add_argument("--secondary-steps", type=int, default=200)
    p.add_argument("--awq-layout", choices=["om", "awq"], default="om",
                   help="AWQ code layout: om = output-major (converted once at setup; the MFMA GEMV "
                        "for decode batches, the MFMA GEMM for prefill), awq = the AWQ GEMM packing as "
                        "stored (its streaming GEMV for decode; prefill-sized calls run the older GEMM)")
    return p.parse_args()


def roofline(bytes_, flops, ms):
    """Roofline position of `bytes_` algorithmic bytes and `flops` algorithmic
    flops done in `ms` milliseconds, against whichever MI355X peak bounds them."""
    hbm_bound = bytes_ / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12)
    if hbm_bound:
        achieved = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}


def use_output_major(w, layout):
    """AWQ banks run on output-major codes (converted once at setup) unless
    the AWQ layout is asked for."""
    return w.fmt == "awq" and layout == "om"


def measure(moe, w, steps, warmup, copies_arg, seed, graph, layout="om", side_stream=True):
    """Times `steps` layer steps of workload `w` (after `warmup` untimed ones).
    Returns the figures of the JSON line and the first weight copy's inputs."""
    import numpy as np
    import torch

    import workloads

    dev = torch.device("cuda:0")
    # ---- inputs: independent weight copies, each > 256 MB unless tiny
    per_copy = w.E * expert_bytes(w, w.fmt)
    copies = copies_arg or (1 if per_copy < 64e6 else max(2, int(np.ceil(1.2e9 / per_copy))))
    copies = min(copies, 8)
    sets = []
    for c in range(copies):
        d = workloads.generate(w, seed=seed, device=dev, copy=c)
        if w.E_base:
            keep = d["keep_idx"].to(dev)
            wr, ex = moe.prune_slice(keep, d["router"], d["experts"])
            d["router"], d["experts"] = wr, ex
        if use_output_major(w, layout):
            d["experts"] = moe.awq_to_output_major(d["experts"])
        sets.append(d)
    torch.cuda.synchronize()
    ws = moe.Workspace(dev)
    stream = torch.cuda.current_stream()
    # the shared expert needs only x: moe_layer runs it on a side stream
    # (default priority) beside routing and the routed experts
    side = torch.cuda.Stream(dev)

    if w.refill:
        stats = [(torch.zeros(w.E, dtype=torch.float32, device=dev),
                  torch.zeros(w.E, dtype=torch.int32, device=dev)) for _ in sets]

    calls = []
    if not w.refill:
        for d in sets:
            calls.append(moe.LayerCall(d["x"], d["router"], w.k, d["experts"], d["shared"],
                                       side_stream=side if side_stream else None, ws=ws))

    def step(i, ev=None):
        d = sets[i % copies]
        x = d["x"]
        if w.refill:
            idx, tl, gate, _ = moe.route(x, d["router"], w.k, extra=1, ws=ws)
            off, sp, p2r = moe.permute(idx, w.E, ws=ws)
            if ev: ev[0].record(stream)
            rows = moe.grouped_ffn(x, w.k + 1, d["experts"], off, sp, out_dtype=moe.OUT_F32, ws=ws)
            if ev: ev[1].record(stream)
            s, c = stats[i % copies]
            moe.refill_score(rows, off, sp, p2r, tl, s, c, ws=ws)
            moe.refill_finalize(s, c, w.H, w.keep)
            return idx
        return calls[i % copies](ev)

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:  # torch creates the HIP events on first record; the library records them
        a.record(stream)
        b.record(stream)
    if graph:
        step = graph_steps(w, calls, step)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        # the routed-call events are recorded on every EV_EVERY-th step only:
        # an event record costs the stream a few microseconds of idle time
        step(i, evs[i] if i % EV_EVERY == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ffn_ms = float(np.mean([a.elapsed_time(b) for i, (a, b) in enumerate(evs) if i % EV_EVERY == 0]))
    ms_per_step = 1e3 * elapsed / steps

    # ---- algorithmic work of the dominant call (routed grouped experts), per call
    kk = w.k + (1 if w.refill else 0)
    P = w.T * kk
    touched = []
    for c in range(copies):
        d = sets[c]
        idx, _, _, _ = moe.route(d["x"], d["router"], w.k, extra=1 if w.refill else 0, ws=ws)
        touched.append(int(torch.unique(idx).numel()))
    torch.cuda.synchronize()
    n_touched = float(np.mean(touched))
    out_bytes = 4 if w.refill else 2
    bytes_call = n_touched * expert_bytes(w, w.fmt) + w.T * w.H * 2 + P * w.H * out_bytes
    flops_call = 2.0 * P * 3 * w.H * w.F
    roof = roofline(bytes_call, flops_call, ffn_ms)
    roof["kernel"] = ("whole layer (one graph replay; the events bracket the replay)" if graph
                      else "moe_grouped_ffn (routed): gate/up + down kernels")
    roof["avg_ms"] = round(ffn_ms, 4)
    roof["algorithmic_bytes"] = int(bytes_call)
    roof["algorithmic_flops"] = int(flops_call)
    roof["traffic"] = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("source_hash") == source_hash():
            roof["traffic"] = t.get("bytes_per_call")

    # ---- the whole layer: router, routed experts, shared expert (not in the
    # Refill-RMS pass, where it cancels), activations in and out
    layer_flops = 2.0 * w.T * w.E * w.H + flops_call
    layer_bytes = n_touched * expert_bytes(w, w.fmt) + w.E * w.H * 2 + w.T * w.H * 2
    if not w.refill:
        layer_flops += 2.0 * w.T * 3 * w.H * w.Fs
        layer_bytes += 3 * w.H * w.Fs * 2 + w.T * w.H * 2
    layer = roofline(layer_bytes, layer_flops, ms_per_step)
    layer["ms"] = round(ms_per_step, 4)
    layer["algorithmic_bytes"] = int(layer_bytes)
    layer["algorithmic_flops"] = int(layer_flops)

    config = {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E,
              "experts_base": w.E_base or w.E, "top_k": w.k, "expert_width": w.F,
              "shared_width": w.Fs, "weights": w.fmt, "weight_copies": copies,
              "touched_experts": n_touched, "hip_graphs": bool(graph),
              "shared_expert_stream": ("side" if side_stream else "main") if not w.refill else None,
              "awq_codes": ("output-major" if use_output_major(w, layout) else "awq") if w.fmt == "awq" else None}
    out = {"value": round(w.T * steps / elapsed, 1), "ms_per_step": round(ms_per_step, 4),
           "config": config, "roofline": roof, "layer_roofline": layer}
    first = sets[0]
    del sets
    return out, first


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is measured on "
              "a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_moe_expert_router_amd as moe
    import workloads

    w = workloads.get(args.workload)
    torch.cuda.set_device(torch.device("cuda:0"))
    moe.lib()

    main_fig, first = measure(moe, w, args.steps, args.warmup, args.copies, args.seed, args.graph == "on",
                              args.awq_layout, args.shared_stream == "on")
    result = {"metric": METRIC, "value": main_fig["value"], "unit": "tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_fig["ms_per_step"],
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": {"bf16": "bf16", "awq": "w4a16_g32/bf16", "fp8": "w8a16_e4m3_block128/bf16",
                        "nvfp4": "w4a4_nvfp4_g16/bf16"}[w.fmt],
              "data": "synthetic (seeded)",
              "config": main_fig["config"],
              "roofline": main_fig["roofline"],
              "layer_roofline": main_fig["layer_roofline"]}

    # ---- the 16-token W4A16 decode layer, in the same process
    if args.secondary != "none" and args.secondary != w.name:
        sw = workloads.get(args.secondary)
        sec, _ = measure(moe, sw, args.secondary_steps, args.warmup, 0, args.seed, False, args.awq_layout,
                         args.shared_stream == "on")
        torch.cuda.empty_cache()
        result["secondary"] = {"workload": sw.name, "steps": args.secondary_steps,
                               "tokens_per_s": sec["value"], "ms_per_step": sec["ms_per_step"],
                               "config": sec["config"], "roofline": sec["roofline"],
                               "layer_roofline": sec["layer_roofline"]}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, first, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def graph_steps(w, calls, eager_step):
    """Steps replayed from HIP graphs: one captured moe_layer call (side
    stream included) per weight copy.  Event records captured inside a graph
    do not time the replayed work, so in this mode the events bracket the
    whole replay.  Capture follows an eager pass, so the workspace has its
    final size."""
    import torch
    if w.refill:
        raise ValueError("the Refill-RMS pass is not replayed from graphs")
    for i in range(len(calls)):
        eager_step(i)
    torch.cuda.synchronize()
    graphs = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c()
        graphs.append(g)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev: ev[0].record(stream)
        graphs[i % len(graphs)].replay()
        if ev: ev[1].record(stream)
    return step


def cpu_baseline(w, d, seconds):
    import numpy as np

    import oracle as O
    import workloads
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    xb_all = workloads.bits(d["x"])
    wr = workloads.bits(d["router"])
    # sample size from a first small timing
    n = min(w.T, 8)
    tokens_done, t_total = 0, 0.0
    reps = 0
    while t_total < seconds and reps < 64:
        lo = (tokens_done) % w.T
        n_now = min(n, w.T - lo)
        xb = xb_all[lo:lo + n_now]
        t0 = time.perf_counter()
        logits, _ = O.router_logits(xb, wr)
        kk = w.k + (1 if w.refill else 0)
        idx = O.rank(logits, kk)
        used = np.unique(idx)
        import torch
        sel = torch.as_tensor(used, dtype=torch.long, device=d["x"].device)
        bank = O.bank_from_tensors({k: (v if isinstance(v, (str, float)) else workloads.bits(v.index_select(0, sel)))
                                    for k, v in d["experts"].items()})
        local = np.searchsorted(used, idx).astype(np.int32)
        if w.refill:
            s = np.zeros(len(used))
            c = np.zeros(len(used), np.int64)
            # experts outside `used` never appear in this sample's top-(k+1) lists
            lg = np.full((n_now, len(used)), -np.inf, np.float32)
            for t in range(n_now):
                lg[t, local[t]] = logits[t, idx[t]]
            O.refill_accumulate(xb, lg, w.k, bank, None, s, c)
        else:
            g = O.gates(logits, idx, w.k)
            rows = O.pair_outputs(xb, local, bank)
            shared = O.bank_from_tensors(workloads.bank_numpy(d["shared"]))
            sv = O.shared_outputs(xb, shared)
            O.combine(rows, g, sv)
        t_total += time.perf_counter() - t0
        tokens_done += n_now
        reps += 1
        if reps == 1:  # size the remaining batches from the first one
            per_tok = t_total / n_now
            n = int(max(1, min(w.T, (seconds - t_total) / per_tok / 4)))
    return {"value": round(tokens_done / t_total, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{tokens_done} tokens of the same workload (first copy) in {reps} batches, "
                      f"{t_total:.1f} s wall; the fp64 C oracle (exact logits, per-pair SwiGLU, combine"
                      + (", full Refill-RMS re-evaluation" if w.refill else "") + ")"}


if __name__ == "__main__":
    main()
