#!/usr/bin/env python3
"""Benchmark one MoE layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one call of moe_layer_forward (router, dispatch, batch-union expert
FFN, combine) over one batch of synthetic tokens, with the layer's weights
already resident in HBM. The default workload is the OLMoE-1B-7B-shaped int8
layer at a decode batch of 16 tokens. Steps rotate through several device
copies of the experts so that repeated calls cannot be served from the
256 MB Infinity Cache.

Prints one JSON line: MoE-layer tokens/s, plus the roofline of the dominant
kernel (its average duration measured with HIP events on the launch stream
inside the timed region) and the oracle's rate on the host cores.
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
GEMV_MAX_T = 16               # Q8_0 batches up to this many tokens run on the GEMV
F16_PEAK_TFLOPS = 2500.0       # MI355X dense f16 matrix cores (2.5 PFLOP/s): the prefill products run here
MALL_DEFEAT_BYTES = 2 << 30    # rotate through at least this much weight memory
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="olmoe_b16")
    ap.add_argument("--copies", type=int, default=0, help="device copies of the experts (0 = enough for 2 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
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


def copy_bandwidth(dev, mib: int = 1024, reps: int = 5) -> float:
    """Achievable HBM rate on this GPU as a reference beside the vendor peak:
    a device-to-device copy of `mib` MiB (read + write), best of `reps`, GB/s."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize(dev)
        best = max(best, 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def cpu_baseline(wl, target_s: float):
    """The oracle (plain numpy) on the same workload, on this host's cores."""
    import synth
    from oracle import ffn as offn
    from oracle import layer as olayer
    try:
        import threadpoolctl
        threads = min(16, os.cpu_count() or 1)
        ctl = threadpoolctl.threadpool_limits(threads)
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:           # threadpoolctl missing: numpy's own default
        ctl, cores = None, os.cpu_count() or 1
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
    # sample: the whole batch for decode; a prefix of tokens for prefill
    n_tok = wl.tokens if wl.tokens <= 16 else 64
    if wl.block:
        x = synth.block_states(shape, wl.tokens)[:n_tok]
        gamma = synth.norm_weight(shape)
        run = lambda: olayer.block_forward(x, gamma, 1e-5, wg, spec, expert, shared, wl.act_mode)  # noqa: E731
    else:
        x = synth.activations(shape, wl.tokens)[:n_tok]
        run = lambda: olayer.layer_forward(x, wg, spec, expert, shared, wl.act_mode)  # noqa: E731
    # untimed pass to quantise the experts the sample needs (weight preparation, not the layer)
    run()
    runs, elapsed = 0, 0.0
    while elapsed < target_s and runs < 50:
        t0 = time.perf_counter()
        run()
        elapsed += time.perf_counter() - t0
        runs += 1
    if ctl is not None:
        ctl.unregister() if hasattr(ctl, "unregister") else None
    return {"value": round(n_tok * runs / elapsed, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tok} of the {wl.tokens} tokens of {wl.name}, {runs} oracle layer_forward runs "
                      f"({elapsed:.1f} s), experts quantised beforehand"}


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

    per_copy = acc.expert_bytes(shape.d_model, shape.d_ff, shape.wformat) * (shape.n_experts + shape.shared_expert)
    copies = args.copies or max(1, min(16, -(-MALL_DEFEAT_BYTES // per_copy)))
    print(f"[bench] {wl.name}: building {copies} device copies of the layer "
          f"({per_copy / 1e6:.1f} MB each)", file=sys.stderr, flush=True)
    layer = dl.build(shape, dev, copies=copies)
    params = qe.with_top_p(layer.params, wl.top_p) if wl.top_p else layer.params
    T = wl.tokens
    if wl.block:
        x = torch.from_numpy(synth.block_states(shape, T)).to(dev)
        norm_w = torch.from_numpy(synth.norm_weight(shape)).to(dev)
    else:
        x = dl.activations(shape, T, dev)
    out = torch.empty((T, shape.d_model), dtype=torch.float32, device=dev)
    ws = qe.workspace(T, shape.top_k, shape.n_experts, shape.d_model, shape.d_ff, act, shape.shared_expert, dev)
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
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, stage_evs[i])
    torch.cuda.synchronize(dev)
    eager_elapsed = time.perf_counter() - t0
    stage_us = {}
    for si, name in enumerate(qe.STAGES):
        if name == "quant_x" and wl.act_mode == "f32":
            name = "split_x"
        if stage_evs[0][2 * si].query() and stage_evs[0][2 * si + 1].query():
            try:
                stage_us[name] = round(float(np.mean([e[2 * si].elapsed_time(e[2 * si + 1]) for e in stage_evs])) * 1e3, 2)
            except RuntimeError:
                pass
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

    # the routing of this batch (identical every step): distinct experts for the byte count
    idx = torch.empty((T, shape.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, shape.top_k), dtype=torch.float32, device=dev)
    # (a block routes its normalised states; torch recomputes them here only
    # to count the experts the timed steps read)
    x_route = x
    if wl.block:
        x_route = (x * torch.rsqrt((x * x).mean(dim=1, keepdim=True) + 1e-5) * norm_w).contiguous()
    qe.moe_route(x_route, layer.gate_w, params, idx, wts, ws)
    counts = torch.empty(shape.n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(shape.n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * shape.top_k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * shape.top_k, dtype=torch.int32, device=dev)
    qe.moe_dispatch(idx, shape.n_experts, counts, offsets, perm, inv)
    counts_h = counts.cpu().numpy()

    d, I, fmt = shape.d_model, shape.d_ff, shape.wformat
    # the kernel the library launches for the gate/up stage of this workload:
    # the GEMV for decode and for Q8_0 batches of up to 16 tokens (HBM bound),
    # the tiled matrix-core GEMM for prefill (matrix-core bound)
    gemv = wl.act_mode == "f32" or T <= GEMV_MAX_T
    if gemv:
        kfile, kname = "gemv.hip", ("gateup_gemv" if wl.act_mode == "f32" else "gateup_gemv_q8")
    else:
        kfile, kname = "mfma_gemm.hip", "gateup_q8_mfma"
    kernel_sources = [os.path.join(ROOT, "quantized_expert_ffn_amd", "csrc", kfile)]
    if gemv:
        algo = acc.gateup_kernel_bytes(counts_h, T, shape.top_k, d, I, fmt, shape.shared_expert, wl.act_mode)
        achieved = algo / (kernel_ms * 1e-3) / 1e9
        copy_gbs = copy_bandwidth(dev)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "achievable_copy": round(copy_gbs, 1),
                "frac_of_achievable": round(achieved / copy_gbs, 4)}
        kkey = f"{kname}_{wl.name}"
    else:
        ops = acc.gateup_ops(counts_h, T, d, I, shape.shared_expert)
        achieved = ops / (kernel_ms * 1e-3) / 1e12
        # the integer codes are multiplied on the f16 matrix cores (exactly), so
        # the peak of that unit bounds the kernel; the int8 figure is given too
        # attainable = min(int8 peak, the kernel's intensity x HBM peak)
        kbytes = acc.gateup_kernel_bytes(counts_h, T, shape.top_k, d, I, fmt, shape.shared_expert, wl.act_mode)
        attainable = min(INT8_PEAK_TOPS, ops / kbytes * HBM_PEAK_GBS / 1e3)
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / F16_PEAK_TFLOPS, 4), "frac_of_int8_peak": round(achieved / INT8_PEAK_TOPS, 4),
                "attainable_int8": round(attainable, 1), "frac_of_attainable": round(achieved / attainable, 4)}
        kkey = f"{kname}_{wl.name}"
    roof["kernel"] = kkey
    roof["traffic"] = measured_traffic(kkey, kernel_sources)

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
        "dtype": (f"f32 (activations f32 as exact f16 pairs, {fmt} weights, f32 accumulate)" if wl.act_mode == "f32"
                  else f"i8 codes ({fmt} weights x Q8_0 activations) on f16 matrix cores: exact integer group dots, "
                       "f32 scales"),
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantised on the GPU)",
        "config": {"workload": wl.name, "tokens": T, "d_model": d, "n_experts": shape.n_experts, "d_ff": I,
                   "top_k": shape.top_k, "router": shape.router, "weights": (f"{fmt[:4]} per-row scales" if fmt.endswith("_row") else f"{fmt} group 32"),
                   "act_mode": wl.act_mode, "shared_expert": shape.shared_expert, "shared_gate": shape.shared_gate,
                   "distinct_experts": int((counts_h > 0).sum()), "routed_rows": int(counts_h.sum()),
                   "top_p": wl.top_p or shape.top_p, "block": wl.block, "device_copies": copies},
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
