#!/usr/bin/env python3
"""Throughput of the MoE feed-forward layer on one MI355X.

A step is one pass of the whole layer over one batch of seeded synthetic
input resident in HBM: route and permute (one call) -> routed experts -> combine, with the
shared expert on a second stream beside them (for the Refill-RMS workload: route with the 11th expert -> permute ->
routed experts (fp32 rows) -> refill score -> keep-set).  Steps cycle through
several independently generated weight copies so that the weights do not stay
in the 256 MB on-die cache between steps.

Prints one JSON line: tokens/s, the roofline position of the dominant kernel
(the routed grouped-expert call, timed with HIP events on its stream inside
the timed region) and the oracle's CPU throughput on a bounded sample.
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
    p.add_argument("--workload", default="decode_bf16",
                   help="tiny_bf16, decode_bf16, decode_awq, decode_fp8, decode_nvfp4, prefill_awq, "
                        "prefill_fp8, prefill_nvfp4, pruned_awq, refill_bf16")
    p.add_argument("--copies", type=int, default=0, help="weight copies to cycle (0: auto)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of the oracle CPU-baseline sample (0 disables it)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--graph", choices=["on", "off"], default="off",
                   help="replay each step from HIP graphs ([route, permute], [routed experts], "
                        "[combine]; the shared expert stays on its side stream)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is measured on "
              "a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_moe_expert_router_amd as moe
    import workloads

    w = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()

    # ---- inputs: independent weight copies, each > 256 MB unless tiny
    per_copy = w.E * expert_bytes(w, w.fmt)
    copies = args.copies or (1 if per_copy < 64e6 else max(2, int(np.ceil(1.2e9 / per_copy))))
    copies = min(copies, 8)
    sets = []
    for c in range(copies):
        d = workloads.generate(w, seed=args.seed, device=dev, copy=c)
        if w.E_base:
            keep = d["keep_idx"].to(dev)
            wr, ex = moe.prune_slice(keep, d["router"], d["experts"])
            d["router"], d["experts"] = wr, ex
        sets.append(d)
    torch.cuda.synchronize()
    ws = moe.Workspace(dev)
    stream = torch.cuda.current_stream()
    # the shared expert needs only x: it runs on a second stream (default
    # priority) beside routing and the routed experts, with its own workspace
    side, side_ws = torch.cuda.Stream(dev), moe.Workspace(dev)

    if w.refill:
        stats = [(torch.zeros(w.E, dtype=torch.float32, device=dev),
                  torch.zeros(w.E, dtype=torch.int32, device=dev)) for _ in sets]

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
            moe.refill_score(rows, off, sp, p2r, idx, tl, s, c, ws=ws)
            moe.refill_finalize(s, c, w.H, w.keep)
            return idx
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            s = moe.grouped_ffn(x, 1, d["shared"], ws=side_ws)
        idx, tl, gate, off, sp, p2r = moe.route_permute(x, d["router"], w.k, ws=ws)
        if ev: ev[0].record(stream)
        rows = moe.grouped_ffn(x, w.k, d["experts"], off, sp, ws=ws)
        if ev: ev[1].record(stream)
        stream.wait_stream(side)
        s.record_stream(stream)
        moe.combine(rows, p2r, gate, s)
        return idx

    use_graph = args.graph == "on"
    if use_graph:
        step = graph_steps(moe, w, sets, ws, side, side_ws, stream, step)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ms_per_step = 1e3 * elapsed / args.steps
    value = w.T * args.steps / elapsed

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
    hbm_bound = bytes_call / (PEAK_HBM_GBS * 1e9) >= flops_call / (PEAK_BF16_TFLOPS * 1e12)
    if hbm_bound:
        achieved = bytes_call / (ffn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops_call / (ffn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["kernel"] = "moe_grouped_ffn (routed): gate/up + down kernels"
    roof["avg_ms"] = round(ffn_ms, 4)
    roof["algorithmic_bytes"] = int(bytes_call)
    roof["algorithmic_flops"] = int(flops_call)
    roof["traffic"] = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("source_hash") == source_hash():
            roof["traffic"] = t.get("bytes_per_call")

    result = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": {"bf16": "bf16", "awq": "w4a16_g32/bf16", "fp8": "w8a16_e4m3_block128/bf16",
                        "nvfp4": "w4a4_nvfp4_g16/bf16"}[w.fmt],
              "data": "synthetic (seeded)",
              "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E,
                         "experts_base": w.E_base or w.E, "top_k": w.k, "expert_width": w.F,
                         "shared_width": w.Fs, "weights": w.fmt, "weight_copies": copies,
                         "touched_experts": n_touched, "hip_graphs": use_graph},
              "roofline": roof}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, sets[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def graph_steps(moe, w, sets, ws, side, side_ws, stream, eager_step):
    """Steps replayed from HIP graphs, one set per weight copy: [route and permute],
    [routed experts], [combine] captured separately so that the HIP events
    around the routed call are recorded between replays.  The shared expert
    runs on the side stream as in the eager step.  Capture happens after an
    eager pass, so every workspace already has its final size."""
    import torch
    for i in range(len(sets)):
        eager_step(i)
    torch.cuda.synchronize()
    graphs = []
    for d in sets:
        x = d["x"]
        if w.refill:
            raise ValueError("the Refill-RMS pass is not replayed from graphs")
        s_buf = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=x.device)
        g1, g2, g3 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            idx, tl, gate, off, sp, p2r = moe.route_permute(x, d["router"], w.k, ws=ws)
        with torch.cuda.graph(g2):
            rows = moe.grouped_ffn(x, w.k, d["experts"], off, sp, ws=ws)
        with torch.cuda.graph(g3):
            y = moe.combine(rows, p2r, gate, s_buf)
        graphs.append((g1, g2, g3, s_buf, (idx, tl, gate, off, sp, p2r, rows, y)))
    torch.cuda.synchronize()

    def step(i, ev=None):
        d = sets[i % len(sets)]
        g1, g2, g3, s_buf, keep = graphs[i % len(sets)]
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            moe.grouped_ffn(d["x"], 1, d["shared"], ws=side_ws, rows=s_buf)
        g1.replay()
        if ev: ev[0].record(stream)
        g2.replay()
        if ev: ev[1].record(stream)
        stream.wait_stream(side)
        g3.replay()
        return keep[0]
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
