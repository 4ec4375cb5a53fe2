#!/usr/bin/env python3
"""Benchmark one MoE layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one call of moe_layer_forward (router, dispatch, batch-union expert
FFN, combine) over one batch of synthetic tokens, with the layer's weights
already resident in HBM. The default workload is the 512-expert
Qwen-Next-class layer (d_model 2048, expert intermediate 512, top-10 of 512
plus one ungated shared expert, int4 group-32 experts, Q8_0 activations) at a
prefill of 4096 tokens with Zipf(1.1)-skewed routing. Steps rotate through
enough device copies of the experts that the bytes one call touches, times
the copies, exceed 2 GB: repeated calls cannot be served from the 256 MB
Infinity Cache.

Prints one JSON line: MoE-layer tokens/s, plus the roofline of the dominant
kernel (its average duration measured with HIP events attached to its own
dispatch on the launch stream, inside the eager timed region), ceilings
measured in the same run, and the oracle's rate on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix cores (5.0 POPS)
F16_PEAK_TFLOPS = 2500.0       # MI355X dense f16 matrix cores (2.5 PFLOP/s): the integer products run here
GEMV_MAX_T = 16                # Q8_0 batches up to this many tokens run on the GEMV
MALL_DEFEAT_BYTES = 2 << 30    # copies x bytes touched per call must exceed this
COPY_MEMORY_CAP = 96 << 30     # at most this much HBM for the copies
STREAM_BYTES = 4 << 30         # the streaming-read reference reads this much per launch
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_prefill")
    ap.add_argument("--copies", type=int, default=0,
                    help="device copies of the experts (0 = enough that copies x bytes touched >= 2 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time the oracle sample aims at")
    return ap.parse_args()


def measured_traffic(kernel_key: str, sources):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(kernel_key)
    except (OSError, ValueError):
        return None
    from quantized_expert_ffn_amd.profiling import source_digest
    if not rec or rec.get("source_digest") != source_digest(sources):
        return None
    return rec.get("bytes_per_launch")


def stream_read_ceiling(dev, reps: int = 5) -> float:
    """What a plain streaming read reaches on this GPU (include/moe_calib.h):
    best of `reps` launches over a 4 GiB buffer, GB/s."""
    import torch
    import quantized_expert_ffn_amd as qe
    buf = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    blocks = 256 * 16
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    qe.moe_calib_stream_read(buf, sink, blocks)          # first touch
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        qe.moe_calib_stream_read(buf, sink, blocks)
        e1.record()
        torch.cuda.synchronize(dev)
        best = max(best, STREAM_BYTES / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    return best


def prefill_mix_ceiling(dev, reps: int = 5) -> float:
    """What the prefill GEMM's inner loop reaches with its operands resident in
    LDS (include/moe_calib.h): best of `reps` launches of 512 blocks of eight
    waves (two per CU, as the GEMM runs), useful int8 TOPS."""
    import torch
    import quantized_expert_ffn_amd as qe
    blocks, stages = 512, 300
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    qe.moe_calib_prefill_mix(blocks, stages, sink)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops = qe.moe_calib_prefill_mix(blocks, stages, sink)
        e1.record()
        torch.cuda.synchronize(dev)
        best = max(best, ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def cpu_baseline(wl, target_s: float):
    """The oracle (plain numpy) on the whole batch of the same workload, on
    this host's cores, repeated until about target_s of CPU time (at most 5
    runs); the experts it needs are quantised beforehand, untimed."""
    import synth
    from oracle import ffn as offn
    from oracle import layer as olayer
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:           # threadpoolctl missing: numpy's own default
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    shape = wl.layer
    bits = synth.weight_bits(shape)
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = offn.QuantExpert.from_fp32(synth.expert_weight(shape, e, "gate"),
                                                  synth.expert_weight(shape, e, "up"),
                                                  synth.expert_weight(shape, e, "down"), bits,
                                                  synth.weight_per_row(shape))
        return cache[e]

    spec = olayer.RouterSpec(mode=shape.router, top_k=shape.top_k, renormalize=shape.renormalize,
                             n_group=shape.n_group, topk_group=shape.topk_group,
                             routed_scaling_factor=shape.routed_scaling_factor, bias=synth.score_bias(shape),
                             top_p=wl.top_p or shape.top_p, shared_gate=synth.shared_gate_weight(shape))
    wg = synth.gate_weight(shape)
    shared = expert(shape.n_experts) if shape.shared_expert else None
    n_tok = wl.tokens
    if wl.block:
        x = synth.block_states(shape, wl.tokens)
        gamma = synth.norm_weight(shape)
        run = lambda: olayer.block_forward(x, gamma, 1e-5, wg, spec, expert, shared, wl.act_mode)  # noqa: E731
    else:
        x = synth.activations(shape, wl.tokens)
        run = lambda: olayer.layer_forward(x, wg, spec, expert, shared, wl.act_mode)  # noqa: E731
    # quantise the experts the batch routes to (weight preparation, not the layer)
    from oracle import dispatch as odispatch
    xr = x if not wl.block else olayer.rmsnorm(x, gamma, 1e-5).astype(np.float32)
    counts = odispatch.dispatch(olayer.route(xr, wg, spec)[0], shape.n_experts)[0]
    for e in np.nonzero(counts)[0]:
        expert(int(e))
    runs, elapsed = 0, 0.0
    while runs < 1 or (elapsed < target_s and runs < 5):
        t0 = time.perf_counter()
        run()
        elapsed += time.perf_counter() - t0
        runs += 1
    return {"value": round(n_tok * runs / elapsed, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"all {n_tok} tokens of {wl.name}, {runs} oracle layer_forward run(s) ({elapsed:.1f} s) with "
                      f"{threads} BLAS threads; the {int((counts > 0).sum())} routed experts (+ shared) quantised "
                      "beforehand, untimed"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the MoE layer here runs on a "
              f"single MI355X; expert-parallel sharding is a design note, not a measured path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import quantized_expert_ffn_amd as qe
    from quantized_expert_ffn_amd import accounting as acc
    from quantized_expert_ffn_amd import device_layer as dl

    wl = synth.workload(args.workload)
    shape = wl.layer
    act = qe.ACT_MODES[wl.act_mode]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    qe.load()
    T = wl.tokens
    d, I, fmt = shape.d_model, shape.d_ff, shape.wformat

    print(f"[bench] {wl.name}: quantising the layer on the GPU", file=sys.stderr, flush=True)
    layer = dl.build(shape, dev, copies=1)
    params = qe.with_top_p(layer.params, wl.top_p) if wl.top_p else layer.params
    if wl.block:
        x = torch.from_numpy(synth.block_states(shape, T)).to(dev)
        norm_w = torch.from_numpy(synth.norm_weight(shape)).to(dev)
    else:
        x = dl.activations(shape, T, dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    ws = qe.workspace(T, shape.top_k, shape.n_experts, d, I, act, shape.shared_expert, dev)

    # the routing of this batch (the same every step): distinct experts, for the
    # byte count and for the number of copies that defeats the caches
    idx = torch.empty((T, shape.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, shape.top_k), dtype=torch.float32, device=dev)
    x_route = x
    if wl.block:   # a block routes its normalised states (recomputed by torch only to count experts)
        x_route = (x * torch.rsqrt((x * x).mean(dim=1, keepdim=True) + 1e-5) * norm_w).contiguous()
    qe.moe_route(x_route, layer.gate_w, params, idx, wts, ws)
    counts = torch.empty(shape.n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(shape.n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * shape.top_k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * shape.top_k, dtype=torch.int32, device=dev)
    qe.moe_dispatch(idx, shape.n_experts, counts, offsets, perm, inv)
    counts_h = counts.cpu().numpy()
    touched = acc.layer_bytes(counts_h, T, d, I, fmt, shape.n_experts, shape.shared_expert, shape.has_bias)
    per_copy = acc.expert_bytes(d, I, fmt) * (shape.n_experts + shape.shared_expert)
    copies = args.copies or max(1, min(-(-MALL_DEFEAT_BYTES // touched), COPY_MEMORY_CAP // per_copy))
    dl.add_copies(layer, copies)
    print(f"[bench] {copies} device copies of the experts ({per_copy / 1e6:.1f} MB each; {touched / 1e6:.1f} MB "
          f"touched per call)", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)

    def step(i, evs=None):
        c = i % copies
        if wl.block:
            qe.moe_block_forward(x, norm_w, 1e-5, layer.gate_w, params, layer.routed[c], layer.shared[c], act, out, ws,
                                 evs)
            return
        if evs is None:
            qe.moe_layer_forward(x, layer.gate_w, params, layer.routed[c], layer.shared[c], act, out, ws)
        else:
            qe.moe_layer_forward_timed(x, layer.gate_w, params, layer.routed[c], layer.shared[c], act, out,
                                       ws, evs)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # (1) eager steps with HIP events on the launch stream: the gate/up and
    # down kernels carry theirs on the dispatch itself, the other stages are
    # bracketed by event records
    stage_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * qe.MOE_STAGE_COUNT)]
                 for _ in range(args.steps)]
    for evs in stage_evs:          # torch creates an event on its first record; do that before timing
        for e in evs:
            e.record()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, stage_evs[i])
    torch.cuda.synchronize(dev)
    eager_elapsed = time.perf_counter() - t0
    stage_us = {}
    for si, name in enumerate(qe.STAGES):
        # a stage that does not run for this batch keeps the events recorded
        # before the step: its start then precedes the step's first event
        ran = si == 0 or all(e[0].elapsed_time(e[2 * si]) >= 0.0 for e in stage_evs)
        if ran:
            stage_us[name] = round(float(np.mean([e[2 * si].elapsed_time(e[2 * si + 1]) for e in stage_evs])) * 1e3, 2)
    kernel_ms = stage_us["gateup"] * 1e-3
    print(f"[bench] eager {args.steps} steps: {eager_elapsed * 1e6 / args.steps:.1f} us/step, stages (us) "
          f"{stage_us}", file=sys.stderr, flush=True)

    # (2) the same step captured once per weight copy in a HIP graph and replayed
    elapsed = eager_elapsed
    if not args.no_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for c in range(copies):
            graphs[c].replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize(dev)
        elapsed = time.perf_counter() - t0
        print(f"[bench] graph {args.steps} steps: {elapsed * 1e6 / args.steps:.1f} us/step", file=sys.stderr,
              flush=True)
    ms_per_step = elapsed * 1e3 / args.steps

    # (3) the per-step spread: the same steps once more, each between two
    # events on the launch stream (not part of the timed region above)
    step_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize(dev)
    step_evs[0].record()
    for i in range(args.steps):
        if args.no_graph:
            step(args.warmup + i)
        else:
            graphs[i % copies].replay()
        step_evs[i + 1].record()
    torch.cuda.synchronize(dev)
    per_step = np.array([step_evs[i].elapsed_time(step_evs[i + 1]) * 1e3 for i in range(args.steps)])
    step_pct = {q: round(float(np.percentile(per_step, v)), 2) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    # (4) the references measured in the same run
    stream_gbs = stream_read_ceiling(dev)
    mix_tops = prefill_mix_ceiling(dev)
    print(f"[bench] streaming read: {stream_gbs:.0f} GB/s; prefill GEMM inner loop alone: {mix_tops:.0f} TOPS",
          file=sys.stderr, flush=True)

    # the kernel the library launches for the gate/up stage of this workload:
    # the GEMV for decode and for Q8_0 batches of up to 16 tokens (HBM bound),
    # the tiled matrix-core GEMM for prefill (matrix-core bound)
    gemv = wl.act_mode == "f32" or T <= GEMV_MAX_T
    if gemv:
        kfiles, kname = ("gemv.hip", "f16codes.h"), ("gateup_gemv" if wl.act_mode == "f32" else "gateup_gemv_q8")
    else:
        kfiles, kname = ("mfma_gemm.hip", "q8_stage.h", "f16codes.h"), "gateup_q8_mfma"
    # the files the kernel is built from: a traffic record taken on other code is not used
    kernel_sources = [os.path.join(ROOT, "quantized_expert_ffn_amd", "csrc", f) for f in kfiles]
    kbytes = acc.gateup_kernel_bytes(counts_h, T, shape.top_k, d, I, fmt, shape.shared_expert, wl.act_mode)
    if gemv:
        achieved = kbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(kbytes)}
    else:
        ops = acc.gateup_ops(counts_h, T, d, I, shape.shared_expert)
        achieved = ops / (kernel_ms * 1e-3) / 1e12
        # integer products counted as int8 multiply-adds (2 ops each) over the
        # routed rows only, priced against the int8 matrix-core peak; they run
        # (exactly) on the f16 matrix cores, whose peak is half of it
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "ops": "int8 multiply-adds x 2, routed rows only",
                "algorithmic_ops": int(ops), "frac_of_f16_peak": round(achieved / F16_PEAK_TFLOPS, 4),
                "algorithmic_bytes": int(kbytes),
                "hbm_gbs_at_achieved": round(kbytes / (kernel_ms * 1e-3) / 1e9, 1)}
    roof["kernel"] = f"{kname}_{wl.name}"
    roof["kernel_us"] = round(kernel_ms * 1e3, 2)
    roof["traffic"] = measured_traffic(roof["kernel"], kernel_sources)
    if roof["traffic"]:
        roof["traffic_over_algorithmic_bytes"] = round(roof["traffic"] / kbytes, 3)
    roof["ceiling_stream_read_gbs"] = round(stream_gbs, 1)
    if gemv:
        roof["frac_of_stream_read"] = round(achieved / stream_gbs, 4)
    else:
        roof["ceiling_instr_mix_tops"] = round(mix_tops, 1)
        roof["frac_of_instr_mix"] = round(achieved / mix_tops, 4)

    line = {
        "metric": "MoE-layer tokens/s at 1 GPU (decode HBM GB/s or prefill int8 TOPS vs peak in roofline)",
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"f32 activations as f16 hi/lo pairs (22 significant bits under a power of two shared per "
                  f"32-column group: over the batch for X, per row for H), {fmt} weights, f32 accumulate"
                  if wl.act_mode == "f32"
                  else f"i8 ({fmt} weight codes x Q8_0 activation codes): exact integer group dots on the f16 "
                       "matrix cores, f32 group scales and accumulation"),
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantised on the GPU)",
        "config": {"workload": wl.name, "tokens": T, "d_model": d, "n_experts": shape.n_experts, "d_ff": I,
                   "top_k": shape.top_k, "router": shape.router,
                   "weights": (f"{fmt[:4]} per-row scales" if fmt.endswith("_row") else f"{fmt} group 32"),
                   "act_mode": wl.act_mode, "shared_expert": shape.shared_expert, "shared_gate": shape.shared_gate,
                   "zipf_s": shape.zipf_s, "distinct_experts": int((counts_h > 0).sum()),
                   "routed_rows": int(counts_h.sum()), "max_expert_rows": int(counts_h.max()),
                   "top_p": wl.top_p or shape.top_p, "block": wl.block, "device_copies": copies,
                   "bytes_touched_per_call": int(touched), "copies_x_touched": int(copies * touched)},
        "roofline": roof,
        "timing": {"launch": "eager" if args.no_graph else "hip_graph",
                   "step_us": step_pct,
                   "eager_ms_per_step": round(eager_elapsed * 1e3 / args.steps, 5),
                   "kernel_timing": "HIP events attached to the gate/up kernel dispatch (hipExtLaunchKernel), "
                                    "mean over the eager steps",
                   "eager_stage_us": stage_us},
    }
    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
