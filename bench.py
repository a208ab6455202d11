#!/usr/bin/env python3
"""Benchmark of the MXFP8 grouped-MLP training step on one MI355X (gfx950).

One step = the whole hot path on one batch of seeded synthetic input:
grouped_mlp_fwd in training mode (quantize X, W1, W2 in both layouts; grouped
GEMM1 with the fused ScaledSwiGLU / routing-weight / requantize epilogue;
grouped GEMM2) followed by grouped_mlp_bwd (quantize dY; dgrad2 with the
fused SwiGLU-backward epilogue; dprobs; wgrad2; dgrad1; wgrad1 accumulated
into fp32 main grads). Default workload: the Mixtral-8x7B-shaped MoE MLP
fwd+bwd (4096 tokens, top-2 of 8 experts = 8192 routed rows, hidden 4096,
ffn 14336). Inputs are resident in HBM before the timed region; no host
transfer or allocation happens inside it.

Prints ONE JSON line: metric/value (GEMM FLOP of the step per second, the
backward's wgrad GEMMs overlapping dgrad on the library's side stream),
per-stage times from a second pass with HIP events recorded on the launch
stream (stages in order), the roofline of the dominant kernel, the step on
weights cast once into the weight cache (qinit-style), the standalone
quantize GB/s (16384 x 4096 bf16, both layouts), token dispatch / combine and
the MoE block forward (8192 tokens, top-2 of 8), the forward-only Llama-3.1-8B
dense and Mixtral-shaped MLPs, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 grouped-MLP TFLOP/s (fwd+bwd) and % of MXFP8 MFMA peak; quantize GB/s"
PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 / MXFP8 MFMA
PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0         # MI355X dense FP4 / MXFP4 MFMA
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E
NOMINAL_SCLK_MHZ = 2400.0         # the clock the MFMA peak is quoted at
GEMM_KERNEL_SRC = os.path.join(ROOT, "mxfp8_block_scaled_mx_amd", "csrc", "mx_gemm.hip")
QUANT_KERNEL_SRC = os.path.join(ROOT, "mxfp8_block_scaled_mx_amd", "csrc", "mx_quantize.hip")
# headers compiled into both kernels (device helpers, argument structs)
KERNEL_HEADERS = [os.path.join(ROOT, "mxfp8_block_scaled_mx_amd", "csrc", h) for h in ("mx_device.h", "mx_internal.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stage_flops(R, H, F):
    """Algorithmic GEMM FLOP of each GEMM stage (actual routed rows, no padding)."""
    return {
        "gemm1_swiglu": 4.0 * R * H * F, "gemm2": 2.0 * R * H * F,
        "dgrad2_swiglu_bwd": 2.0 * R * H * F, "wgrad2": 2.0 * R * H * F,
        "dgrad1": 4.0 * R * H * F, "wgrad1": 4.0 * R * H * F,
    }


def stage_bytes(E, R, P, H, F):
    """Algorithmic HBM bytes of each stage: every operand read once, every
    output written once (MXFP8 = 1 byte per code + 1 per 32 codes; the
    columnwise layouts hold P = sum of per-expert row counts padded to 32;
    fp32 main grads are read and written)."""
    mx8 = 1.0 + 1.0 / 32
    return {
        "quantize_x": 2 * R * H + mx8 * (R * H + H * P),
        "quantize_w1": 2 * E * 2 * F * H + 2 * mx8 * E * 2 * F * H,
        "quantize_w2": 2 * E * H * F + 2 * mx8 * E * H * F,
        "gemm1_swiglu": mx8 * (R * H + E * 2 * F * H) + 4 * R + 2 * R * 2 * F + mx8 * (R * F + F * P),
        "gemm2": mx8 * (R * F + E * H * F) + 2 * R * H,
        "quantize_dy": 2 * R * H + mx8 * (R * H + H * P),
        "dgrad2_swiglu_bwd": mx8 * (R * H + E * F * H) + 2 * R * 2 * F + 4 * R
                             + mx8 * (R * 2 * F + 2 * F * P) + 4 * R * (F // 256),
        "dprobs_reduce": 4 * R * (F // 256) + 4 * R,
        "wgrad2": mx8 * (H * P + F * P) + 2 * 4 * E * H * F,
        "dgrad1": mx8 * (R * 2 * F + E * H * 2 * F) + 2 * R * H,
        "wgrad1": mx8 * (2 * F * P + H * P) + 2 * 4 * E * 2 * F * H,
    }


def traffic_from_profiles(workload, stage):
    """Measured HBM bytes per launch of one stage from the committed rocprofv3
    counter summary, only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    for key, src in (("source_sha256", GEMM_KERNEL_SRC), ("quantize_source_sha256", QUANT_KERNEL_SRC)):
        if vals.get(key) != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
    if vals.get("headers_sha256") != hashlib.sha256(b"".join(open(h, "rb").read() for h in KERNEL_HEADERS)).hexdigest():
        return None
    try:
        return float(vals[f"{stage}.hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def oracle_sample(inp, wl, rows=256, ffn_cols=1024):
    """A bounded slice of one MLP workload for timing the oracle: the first
    `rows` routed rows of its largest expert and the first `ffn_cols` ffn
    columns of that expert (gate rows [0, Fs), up rows [F, F + Fs) of W1, the
    columns [0, Fs) of W2). The sliced MLP is the same computation at a
    smaller F, so its algorithmic FLOP rate stands for the workload's."""
    import numpy as np
    split = inp["split_sizes"]
    e = int(np.argmax(split))
    r0 = int(split[:e].sum())
    S = int(min(rows, split[e]))
    F, Fs = wl.ffn, min(ffn_cols, wl.ffn)
    w1 = inp["w1"][e]
    out = {"x": inp["x"][r0:r0 + S].copy(), "probs": inp["probs"][r0:r0 + S].copy(),
           "w1": np.ascontiguousarray(np.concatenate([w1[:Fs], w1[F:F + Fs]])[None]),
           "w2": np.ascontiguousarray(inp["w2"][e][:, :Fs][None]), "rows": S, "ffn": Fs, "expert": e,
           "hidden": wl.hidden}
    if "dy" in inp:
        out["dy"] = inp["dy"][r0:r0 + S].copy()
    return out


def cpu_baseline(samples, tiny, c2_rows, reps=3):
    """The oracle (float64 numpy, per-expert loops) as it stands, timed on the
    host: median of `reps` wall times per configuration, on all BLAS threads;
    the tiny MoE forward and the quantize sample also on one thread.

    samples: oracle_sample() slices of the Llama dense forward, the
    Mixtral-shaped forward and the Mixtral-shaped forward+backward; tiny: the
    whole tiny MoE workload; c2_rows: the first rows of the 16384 x 4096
    quantize tensor (bf16 bits), both layouts."""
    import numpy as np
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                              # threadpoolctl missing: report the core count
        threadpool_limits, threads = None, os.cpu_count()

    def med(fn):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def single(fn):
        if threadpool_limits is None:
            return None
        with threadpool_limits(limits=1):
            return med(fn)

    res = {}
    # tiny MoE MLP forward, whole workload
    fl = 6.0 * tiny["x"].shape[0] * tiny["w1"].shape[2] * (tiny["w1"].shape[1] // 2)
    f1 = lambda: orc.mlp_forward(tiny["x"], tiny["probs"], tiny["w1"], tiny["w2"], tiny["split_sizes"])
    t, t1 = med(f1), single(f1)
    res["tiny_moe_fwd"] = {"sample": "whole workload (512 routed rows, 4 experts, H=256, F=512)",
                           "seconds": round(t, 4), "gflops": round(fl / t / 1e9, 3),
                           "single_thread_seconds": None if t1 is None else round(t1, 4),
                           "single_thread_gflops": None if t1 is None else round(fl / t1 / 1e9, 3)}
    # standalone quantize, both layouts
    nb = c2_rows.shape[0] * c2_rows.shape[1] * (2 + 2 * (1 + 1 / 32))
    xq = orc.bf16_bits_to_f64(c2_rows)
    f2 = lambda: (orc.quantize_rowwise(xq), orc.quantize_colwise(xq))
    t, t1 = med(f2), single(f2)
    res["quantize_16384x4096"] = {"sample": f"rows 0..{c2_rows.shape[0] - 1} of the tensor, both layouts",
                                  "seconds": round(t, 4), "gbps": round(nb / t / 1e9, 4),
                                  "single_thread_seconds": None if t1 is None else round(t1, 4),
                                  "single_thread_gbps": None if t1 is None else round(nb / t1 / 1e9, 4)}
    for name, smp in samples.items():
        S, H, Fs = smp["rows"], smp["hidden"], smp["ffn"]
        bwd = "dy" in smp

        def fn(smp=smp, bwd=bwd):
            f = orc.mlp_forward(smp["x"], smp["probs"], smp["w1"], smp["w2"], [smp["rows"]])
            if bwd:
                orc.mlp_backward(smp["x"], smp["probs"], smp["w1"], smp["w2"], [smp["rows"]], smp["dy"], f)

        fl = (18.0 if bwd else 6.0) * S * H * Fs
        t = med(fn)
        res[name] = {"sample": f"{'fwd+bwd' if bwd else 'fwd'} of expert {smp['expert']} on its first {S} "
                               f"routed rows, H={H}, ffn columns 0..{Fs - 1}",
                     "seconds": round(t, 4), "gflops": round(fl / t / 1e9, 3)}
    head = res["mixtral_moe_fwd_bwd"]
    return {"value": round(head["gflops"] / 1e3, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": head["sample"] + f" (median of {reps}); per-configuration samples under 'configs'",
            "configs": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_moe_fwd_bwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--no-qinit", action="store_true", help="skip the cached-weight (qinit-style) step")
    ap.add_argument("--no-moe", action="store_true", help="skip token dispatch / combine")
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the shader clock")
    ap.add_argument("--no-gemm-fp4", action="store_true", help="skip the MXFP4 GEMM")
    ap.add_argument("--no-fp4-step", action="store_true", help="skip the MXFP4 MLP step")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the forward-only Llama dense and Mixtral-shaped workloads")
    ap.add_argument("--quantize-only", action="store_true",
                    help="only time the standalone 16384 x 4096 quantize (for profiling it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of a known size (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "sharding over several GPUs (expert parallelism) is designed but not run here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as wlmod
    import mxfp8_block_scaled_mx_amd as mx

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mx.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(mx, torch, dev)
        return
    if args.quantize_only:
        q, _ = measure_quantize(mx, torch, np, wlmod, dev)
        print(json.dumps({"quantize": q}), flush=True)
        return
    wl = wlmod.WORKLOADS[args.workload]
    if not wl.backward:
        raise SystemExit("bench.py times the fwd+bwd step; pick a workload with a backward pass")

    log(f"generating inputs for {wl.name} (seed {wl.seed})")
    t0 = time.perf_counter()
    inp = wlmod.make_mlp_inputs(wl)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; split_sizes={inp['split_sizes'].tolist()}")

    def to_dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w1, w2, dy = (to_dev_bf16(inp[k]) for k in ("x", "w1", "w2", "dy"))
    probs = torch.from_numpy(inp["probs"]).to(dev)
    E, R, H, F = wl.experts, wl.rows, wl.hidden, wl.ffn
    split = inp["split_sizes"].tolist()
    runner = mx.MLPRunner(E, R, H, F, split, device=dev)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device=dev)
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        runner.forward(x, probs, w1, w2, training=True)
        runner.backward(dy, probs, dw1, dw2, accumulate=True)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    nf, nb = len(mx.FWD_STAGES) + 1, len(mx.BWD_STAGES) + 1
    ev_f = [[torch.cuda.Event(enable_timing=True) for _ in range(nf)] for _ in range(args.steps)]
    ev_b = [[torch.cuda.Event(enable_timing=True) for _ in range(nb)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for evs in ev_f + ev_b:          # torch creates the HIP event on first record
        for e in evs:
            e.record()
    log(f"timing {args.steps} steps")
    # one event before each step and one after the last, on the launch stream
    ev_step = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in ev_step:
        e.record()
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        ev_step[i].record()
        step()
    ev_step[args.steps].record()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    per_step = [ev_step[i].elapsed_time(ev_step[i + 1]) for i in range(args.steps)]
    # per-stage times: the same steps with stage events set, which runs every
    # stage on the launch stream in order (no side-stream overlap)
    log(f"timing {args.steps} steps stage by stage")
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        mx.set_stage_events(ev_f[i])
        runner.forward(x, probs, w1, w2, training=True)
        mx.set_stage_events(ev_b[i])
        runner.backward(dy, probs, dw1, dw2, accumulate=True)
    end.record()
    mx.set_stage_events(None)
    torch.cuda.synchronize()
    serial_ms = start.elapsed_time(end) / args.steps

    stages = {}
    for names, evs in ((mx.FWD_STAGES, ev_f), (mx.BWD_STAGES, ev_b)):
        for j, name in enumerate(names):
            stages[name] = float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
    flops = stage_flops(R, H, F)
    P = int(sum((m + 31) // 32 * 32 for m in split))
    nbytes = stage_bytes(E, R, P, H, F)
    step_flops = sum(flops.values())                     # = 18 R H F
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = sum(stages[k] for k in flops)
    gemm_tflops = step_flops / (gemm_ms * 1e-3) / 1e12

    def roof(k):
        """Bound of stage k: whichever of MFMA time and HBM time at peak is larger."""
        t = stages[k] * 1e-3
        fl = flops.get(k, 0.0)
        if fl / (PEAK_FP8_TFLOPS * 1e12) >= nbytes[k] / (PEAK_HBM_GBPS * 1e9):
            ach = fl / t / 1e12
            return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_FP8_TFLOPS, 4)}
        ach = nbytes[k] / t / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBPS, 4)}

    dom = max(stages, key=lambda k: stages[k])
    roofline = dict(roof(dom), traffic=traffic_from_profiles(wl.name, dom), kernel=dom,
                    algorithmic_flop_per_launch=flops.get(dom, 0.0),
                    algorithmic_bytes_per_launch=round(nbytes[dom]), avg_launch_ms=round(stages[dom], 4))
    per_stage = {k: dict(ms=round(stages[k], 4), **roof(k),
                         tflops=round(flops.get(k, 0.0) / (stages[k] * 1e-3) / 1e12, 1),
                         gbps=round(nbytes[k] / (stages[k] * 1e-3) / 1e9, 1)) for k in stages}
    log(f"step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; GEMM-only {gemm_tflops:.1f} TFLOP/s")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp8_e4m3",
        "data": "synthetic (seeded; shapes of the Mixtral-8x7B-shaped MoE MLP)",
        "config": {"workload": wl.name, "tokens": wl.tokens, "topk": wl.topk, "experts": E,
                   "rows": R, "hidden": H, "ffn": F, "split_sizes": split,
                   "step": "grouped_mlp_fwd(training) + grouped_mlp_bwd(fp32 wgrad accumulate)"},
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(float(np.median(per_step)), 4),
                    "min": round(float(np.min(per_step)), 4), "max": round(float(np.max(per_step)), 4),
                    "timing": "HIP events on the launch stream: one pair around the timed steps (mean) and "
                              "one event between consecutive steps (median, min, max)"},
        "serial_ms_per_step": round(serial_ms, 4),
        "gemm_only": {"tflops": round(gemm_tflops, 1),
                      "frac_mfma_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "ms": round(gemm_ms, 4)},
        "stages": per_stage,
        "roofline": roofline,
    }

    clk = measure_clock(step, torch) if not args.no_clock else {"sclk_mhz": None, "source": "not sampled"}
    if clk.get("sclk_mhz"):
        scale = NOMINAL_SCLK_MHZ / clk["sclk_mhz"]
        out["clock"] = dict(clk, gemm_only_frac_mfma_peak_at_clock=round(out["gemm_only"]["frac_mfma_peak"] * scale, 4))
        for k, v in out["stages"].items():
            if v["bound"] == "mfma":
                v["frac_at_measured_clock"] = round(v["frac"] * scale, 4)
        log(f"sclk {clk['sclk_mhz']:.0f} MHz under the step loop")
    else:
        out["clock"] = clk

    # qinit-style variant: the weights are cast into the MXFP8 weight cache
    # once, outside the timed region (as after an optimizer update), and the
    # step runs grouped_mlp_fwd_cached + grouped_mlp_bwd_cached
    if not args.no_qinit:
        measure_qinit(args, runner, x, probs, w1, w2, dy, dw1, dw2, start, end, step_flops, out, torch)

    # the same step with every GEMM on MXFP4 copies (the MLP of an FP4 layer)
    if not args.no_fp4_step:
        out["mxfp4_step"] = measure_fp4_step(mx, torch, args, x, probs, w1, w2, dy, dw1, dw2, split, step_flops,
                                             ms_per_step)
        f4s = out["mxfp4_step"]
        log(f"MXFP4 step {f4s['ms']:.3f} ms -> {f4s['tflops']:.1f} TFLOP/s "
            f"({f4s['speedup_vs_mxfp8']:.2f}x the MXFP8 step); cached weights "
            f"{f4s['cached_weights']['ms']:.3f} ms -> {f4s['cached_weights']['tflops']:.1f} TFLOP/s")

    samples, c2_rows = {}, None
    if not args.no_quantize:
        out["quantize"], c2_rows = measure_quantize(mx, torch, np, wlmod, dev)
        f4 = out["quantize"]["fp4_rowwise"]
        log(f"device copy {out['quantize']['copy_reference']['gbps']:.0f} GB/s")
        log(f"quantize {out['quantize']['gbps']:.0f} GB/s; MXFP4 rowwise {f4['gbps']:.0f} GB/s, "
            f"both layouts {f4['both_layouts_gbps']:.0f} GB/s")

    if not args.no_gemm_fp4:
        out["gemm_fp4"] = measure_gemm_fp4(mx, torch, dev, split)
        g4 = out["gemm_fp4"]
        log(f"MXFP4 GEMM {g4['workload']}: {g4['ms']:.3f} ms -> {g4['tflops']:.0f} TFLOP/s "
            f"({g4['roofline']['frac']:.3f} of the FP4 peak); grouped over the step's split_sizes "
            f"{g4['grouped']['ms']:.3f} ms -> {g4['grouped']['tflops']:.0f} TFLOP/s; weight gradient "
            f"{g4['wgrad']['ms']:.3f} ms -> {g4['wgrad']['tflops']:.0f} TFLOP/s")
        nv = g4["nvfp4"]
        log(f"NVFP4 cast {nv['cast']['gbps']:.0f} GB/s; GEMM {nv['gemm']['ms']:.3f} ms -> "
            f"{nv['gemm']['tflops']:.0f} TFLOP/s ({nv['gemm']['frac_bf16_peak']:.3f} of the bf16 peak); grouped "
            f"{nv['grouped']['ms']:.3f} ms -> {nv['grouped']['tflops']:.0f} TFLOP/s")

    if not args.no_moe:
        out["dispatch_combine"] = measure_moe(mx, torch, np, wlmod, dev)
        dc = out["dispatch_combine"]
        log(f"dispatch {dc['dispatch_gbps']:.0f} GB/s (routing only {dc['routing_only_ms'] * 1e3:.0f} us), "
            f"combine {dc['combine_gbps']:.0f} GB/s; MoE block fwd {dc['moe_block_fwd']['ms']:.3f} ms "
            f"-> {dc['moe_block_fwd']['tflops']:.0f} TFLOP/s; MoE layer train step "
            f"{dc['moe_layer_train_step']['ms']:.3f} ms -> {dc['moe_layer_train_step']['tflops']:.0f} TFLOP/s")
        log(f"MoE layer train step with this step's counts: host copy "
            f"{dc['moe_layer_train_step_host_counts']['ms']:.3f} ms, device-resident "
            f"{dc['moe_layer_train_step_device_counts']['ms']:.3f} ms")

    # free device memory before the forward-only workloads and the CPU leg
    del runner, dw1, dw2, x, w1, w2, dy
    torch.cuda.empty_cache()
    if not args.no_forward:
        out["forward_only"] = {}
        for name in ("tiny_moe_fwd", "llama8b_dense_fwd", "mixtral_moe_fwd"):
            r = measure_forward(mx, torch, np, wlmod, dev, wlmod.WORKLOADS[name], args.steps, args.warmup,
                                samples if not args.no_cpu_baseline else None)
            out["forward_only"][name] = r
            log(f"{name}: forward {r['ms']:.3f} ms -> {r['tflops']:.1f} TFLOP/s; "
                f"cached weights {r['qinit_style_ms']:.3f} ms -> {r['qinit_style_tflops']:.1f} TFLOP/s")
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on bounded samples")
        samples[wl.name] = oracle_sample(inp, wl)
        for name in ("llama8b_dense_fwd", "mixtral_moe_fwd"):
            if name not in samples:
                samples[name] = oracle_sample(wlmod.make_mlp_inputs(wlmod.WORKLOADS[name]), wlmod.WORKLOADS[name])
        if c2_rows is None:
            c2_rows = wlmod.quantize_tensor_c2()[:1024].copy()
        tiny = wlmod.make_mlp_inputs(wlmod.WORKLOADS["tiny_moe_fwd"])
        out["cpu_baseline"] = cpu_baseline(samples, tiny, c2_rows)
        log(f"oracle {out['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s on {out['cpu_baseline']['cores']} threads")
    print(json.dumps(out), flush=True)


def measure_fp4_step(mx, torch, args, x, probs, w1, w2, dy, dw1, dw2, split, step_flops, ms_mxfp8):
    """grouped_mlp_fwd_fp4 (training) + grouped_mlp_bwd_fp4 (accumulating into
    the fp32 gradients) on the step's inputs: the same work as the MXFP8 step
    (18 R H F flops) with every GEMM on MXFP4 copies; workspaces allocated
    once, outside the timed region."""
    R, H = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    fws, _, bws = mx.mlp_fp4_sizes(E, R, H, F, split)
    wsf = torch.empty(fws, dtype=torch.uint8, device=x.device)
    wsb = torch.empty(bws, dtype=torch.uint8, device=x.device)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=x.device)

    def step():
        _, st = mx.grouped_mlp_fwd_fp4(x, probs, w1, w2, split, training=True, workspace=wsf, out=y)
        mx.grouped_mlp_bwd_fp4(dy, probs, st, dw1=dw1, dw2=dw2, accumulate=True, workspace=wsb)

    # cached weights: cast once into the MXFP4 weight cache outside the timed
    # region (as after an optimizer update); the step reads the cache
    cache = mx.grouped_mlp_fp4_quantize_weights(w1, w2)

    def step_cached():
        _, st = mx.grouped_mlp_fwd_fp4_cached(x, probs, cache, split, training=True, workspace=wsf, out=y)
        mx.grouped_mlp_bwd_fp4_cached(dy, probs, st, cache, dw1=dw1, dw2=dw2, accumulate=True, workspace=wsb)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = timed(step)
    ms_c = timed(step_cached)
    tf = lambda t: round(step_flops / (t * 1e-3) / 1e12, 1)
    return {"workload": "mixtral_moe_fwd_bwd at MXFP4", "ms": round(ms, 4),
            "tflops": tf(ms), "frac_fp4_peak": round(step_flops / (ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4),
            "speedup_vs_mxfp8": round(ms_mxfp8 / ms, 3),
            "cached_weights": {"ms": round(ms_c, 4), "tflops": tf(ms_c),
                               "step": "grouped_mlp_fwd_fp4_cached + grouped_mlp_bwd_fp4_cached; weights cast "
                                       "once (grouped_mlp_fp4_quantize_weights) outside the timed region"}}


def measure_clock(step, torch, seconds=2.0, samples=3):
    """Shader clock while the step runs: `rocm-smi --showclocks --json` sampled
    from a helper thread during about `seconds` of untimed steps. The MXFP8
    peak (5.0 PFLOP/s) is quoted at 2.4 GHz; the fractions at the measured
    clock rescale by 2.4 GHz / sclk."""
    import re
    import subprocess
    import threading
    vals = []

    def sample():
        time.sleep(seconds / (samples + 1))
        for _ in range(samples):
            try:
                r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                                   timeout=10)
                m = re.search(r'"sclk clock speed:":\s*"\((\d+)Mhz\)"', r.stdout)
                if m:
                    vals.append(int(m.group(1)))
            except Exception:
                pass
            time.sleep(seconds / (samples + 1))

    th = threading.Thread(target=sample)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < 4 * seconds:
        step()
        torch.cuda.synchronize()
    th.join()
    if not vals:
        return {"sclk_mhz": None, "source": "rocm-smi --showclocks (not available)"}
    return {"sclk_mhz": round(sum(vals) / len(vals), 1), "samples_mhz": vals, "nominal_mhz": NOMINAL_SCLK_MHZ,
            "source": "rocm-smi --showclocks during untimed steps"}


def measure_qinit(args, runner, x, probs, w1, w2, dy, dw1, dw2, start, end, step_flops, out, torch):
    """The training step on weights cast once into the weight cache before the
    timed region (grouped_mlp_quantize_weights), as after an optimizer update."""
    runner.quantize_weights(w1, w2)
    for _ in range(args.warmup):
        runner.forward_cached(x, probs, training=True)
        runner.backward_cached(dy, probs, dw1, dw2, accumulate=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        runner.forward_cached(x, probs, training=True)
        runner.backward_cached(dy, probs, dw1, dw2, accumulate=True)
    end.record()
    torch.cuda.synchronize()
    q_ms = start.elapsed_time(end) / args.steps
    out["qinit_style"] = {"ms_per_step": round(q_ms, 4),
                          "tflops": round(step_flops / (q_ms * 1e-3) / 1e12, 2),
                          "step": "grouped_mlp_fwd_cached + grouped_mlp_bwd_cached; weights cast "
                                  "once by grouped_mlp_quantize_weights before the timed region"}
    log(f"qinit-style step {q_ms:.3f} ms -> {out['qinit_style']['tflops']:.1f} TFLOP/s")


def measure_moe(mx, torch, np, wlmod, dev, iters=20, T=8192, E=8, H=4096, ffn=14336):
    """Token dispatch and combine for 8192 tokens, top-2 of 8 experts, hidden
    4096 (the Mixtral-shaped forward workload's routing shape). Algorithmic
    bytes: dispatch reads x once and writes the 2T routed rows; combine reads
    the 2T routed rows and writes y (index arrays are negligible)."""
    c = wlmod.make_dispatch_inputs(T, E, H, seed=60)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, y_perm = bits(c["x"]), bits(c["y_perm"])
    idx = torch.from_numpy(c["topk_idx"]).to(dev)
    w = torch.from_numpy(c["topk_w"]).to(dev)
    _, _, perm, _, _ = mx.mx_moe_dispatch(x, idx, w, E)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    d_ms = timed(lambda: mx.mx_moe_dispatch(x, idx, w, E))
    r_ms = timed(lambda: mx.mx_moe_dispatch(x, idx, w, E, gather=False))
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    c_ms = timed(lambda: mx.mx_moe_combine(y_perm, perm, out=y))
    d_bytes = (T + 2 * T) * H * 2
    c_bytes = (2 * T + T) * H * 2
    out = {"tokens": T, "topk": 2, "experts": E, "hidden": H,
           "dispatch_ms": round(d_ms, 4), "dispatch_gbps": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
           "routing_only_ms": round(r_ms, 4),
           "combine_ms": round(c_ms, 4), "combine_gbps": round(c_bytes / (c_ms * 1e-3) / 1e9, 1),
           "note": "dispatch time includes the binding's output allocation per call (torch caching allocator)"}
    # the whole MoE MLP block forward (inference) on these tokens: routing-only
    # dispatch, the fused forward gathering X through row_token, combine;
    # weights are seeded N(0, 0.02) draws made on the device
    F = ffn
    g = torch.Generator(device=dev)
    g.manual_seed(61)
    w1 = (torch.randn((E, 2 * F, H), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((E, H, F), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    _, probs, perm, row_token, counts = mx.mx_moe_dispatch(x, idx, w, E, gather=False)
    split = counts.cpu().tolist()
    R = sum(split)
    runner_ws = mx._byte_buffer(mx.mlp_sizes(E, R, H, F, split)[0], dev)
    y_r = torch.empty((R, H), dtype=torch.bfloat16, device=dev)

    def block():
        _, p_, pm, rt, _ = mx.mx_moe_dispatch(x, idx, w, E, gather=False)
        mx.grouped_mlp_fwd_gather(x, rt, p_, w1, w2, split, training=False, workspace=runner_ws, out=y_r)
        mx.mx_moe_combine(y_r, pm, out=y)

    b_ms = timed(block)
    out["moe_block_fwd"] = {"ms": round(b_ms, 4), "rows": R, "ffn": F,
                            "tflops": round(6.0 * R * H * F / (b_ms * 1e-3) / 1e12, 1),
                            "step": "mx_moe_dispatch (routing only) + grouped_mlp_fwd_gather (inference, "
                                    "weights cast in the call) + mx_moe_combine; split_sizes taken from "
                                    "the routing before the timed region"}
    # the MoE layer training step (no router): routing-only dispatch, the
    # fused forward (training), combine, the fused backward with dY gathered
    # from the tokens' output gradient, combine of dX; fp32 main grads
    dy_tok = (torch.randn((T, H), generator=g, device=dev) * 1e-3).to(torch.bfloat16)
    dw1 = torch.zeros((E, 2 * F, H), dtype=torch.float32, device=dev)
    dw2 = torch.zeros((E, H, F), dtype=torch.float32, device=dev)
    _, _, bws = mx.mlp_sizes(E, R, H, F, split)
    bwd_ws = mx._byte_buffer(bws, dev)
    dx_t = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def layer_step():
        _, p_, pm, rt, _ = mx.mx_moe_dispatch(x, idx, w, E, gather=False)
        yr, st = mx.grouped_mlp_fwd_gather(x, rt, p_, w1, w2, split, training=True, workspace=runner_ws, out=y_r)
        mx.mx_moe_combine(yr, pm, out=y)
        dxr, _, _, _ = mx.grouped_mlp_bwd_gather(dy_tok, rt, p_, st, dw1=dw1, dw2=dw2, accumulate=True,
                                                 workspace=bwd_ws)
        mx.mx_moe_combine(dxr, pm, out=dx_t)

    t_ms = timed(layer_step)
    out["moe_layer_train_step"] = {"ms": round(t_ms, 4), "rows": R,
                                   "tflops": round(18.0 * R * H * F / (t_ms * 1e-3) / 1e12, 1),
                                   "step": "routing-only dispatch + grouped_mlp_fwd_gather (training) + combine + "
                                           "grouped_mlp_bwd_gather (fp32 wgrad accumulate) + combine of dX"}
    # the same step as a real layer runs it, where the counts come from this
    # step's routing: (a) copied to the host before the MLP calls (a host
    # round trip and a wait each step), (b) left on the device and read by the
    # device-split calls (no copy, no wait)
    def layer_step_host_counts():
        _, p_, pm, rt, cnt = mx.mx_moe_dispatch(x, idx, w, E, gather=False)
        sp = cnt.cpu().tolist()
        yr, st = mx.grouped_mlp_fwd_gather(x, rt, p_, w1, w2, sp, training=True, workspace=runner_ws, out=y_r)
        mx.mx_moe_combine(yr, pm, out=y)
        dxr, _, _, _ = mx.grouped_mlp_bwd_gather(dy_tok, rt, p_, st, dw1=dw1, dw2=dw2, accumulate=True,
                                                 workspace=bwd_ws)
        mx.mx_moe_combine(dxr, pm, out=dx_t)

    h_ms = timed(layer_step_host_counts)
    dev_run = mx.DeviceSplitMLPRunner(E, R, H, F, device=dev)

    def layer_step_device_counts():
        _, p_, pm, rt, cnt = mx.mx_moe_dispatch(x, idx, w, E, gather=False)
        yr = dev_run.forward(cnt, x, p_, w1, w2, row_token=rt)
        mx.mx_moe_combine(yr, pm, out=y)
        dxr, _ = dev_run.backward(cnt, dy_tok, p_, dw1, dw2, accumulate=True, row_token=rt)
        mx.mx_moe_combine(dxr, pm, out=dx_t)

    v_ms = timed(layer_step_device_counts)
    flop = 18.0 * R * H * F
    out["moe_layer_train_step_host_counts"] = {
        "ms": round(h_ms, 4), "tflops": round(flop / (h_ms * 1e-3) / 1e12, 1),
        "step": "as moe_layer_train_step, with this step's counts copied to the host (counts.cpu()) before "
                "the MLP calls"}
    out["moe_layer_train_step_device_counts"] = {
        "ms": round(v_ms, 4), "tflops": round(flop / (v_ms * 1e-3) / 1e12, 1),
        "step": "as moe_layer_train_step, with this step's counts read on the device by "
                "grouped_mlp_fwd_device_split / grouped_mlp_bwd_device_split (no host copy, no wait)"}
    del w1, w2, runner_ws, dw1, dw2, bwd_ws, dev_run
    return out


def measure_forward(mx, torch, np, wlmod, dev, wl, steps, warmup, samples=None):
    """Inference forward (grouped_mlp_fwd without a saved buffer: quantize X
    and the weights rowwise, GEMM1 + SwiGLU epilogue, GEMM2) on a forward-only
    workload, then the same with the weights cast once into the weight cache
    before the timed region (grouped_mlp_fwd_cached). Algorithmic GEMM FLOP:
    6 R H F."""
    log(f"generating inputs for {wl.name} (seed {wl.seed})")
    inp = wlmod.make_mlp_inputs(wl)
    if samples is not None and wl.name != "tiny_moe_fwd":
        samples[wl.name] = oracle_sample(inp, wl)

    def to_dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w1, w2 = (to_dev_bf16(inp[k]) for k in ("x", "w1", "w2"))
    probs = torch.from_numpy(inp["probs"]).to(dev)
    E, R, H, F = wl.experts, wl.rows, wl.hidden, wl.ffn
    split = inp["split_sizes"].tolist()
    runner = mx.MLPRunner(E, R, H, F, split, device=dev)
    flops = 6.0 * R * H * F
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    ms = timed(lambda: runner.forward(x, probs, w1, w2, training=False))
    runner.quantize_weights(w1, w2)
    q_ms = timed(lambda: runner.forward_cached(x, probs, training=False))
    del runner, x, w1, w2, probs
    return {"rows": R, "experts": E, "hidden": H, "ffn": F, "split_sizes": split,
            "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "qinit_style_ms": round(q_ms, 4), "qinit_style_tflops": round(flops / (q_ms * 1e-3) / 1e12, 1),
            "step": "grouped_mlp_fwd (inference; weights cast in the call) / grouped_mlp_fwd_cached"}


def copy_calibration(mx, torch, dev, nbytes=1 << 30, reps=3):
    """The library's plain device copy (mx_device_copy) of nbytes (read
    nbytes, write nbytes), reps times: the HBM counters (FETCH_SIZE,
    WRITE_SIZE) of these dispatches give the factor between counter units and
    bytes on this machine."""
    L = mx.load()
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        mx._check(L.mx_device_copy(mx._ptr(dst), mx._ptr(src), nbytes, mx._stream()))
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}}),
          flush=True)


def measure_gemm_fp4(mx, torch, dev, split, iters=10, m=16384, n=28672, k=4096):
    """mx_gemm_fp4 (C = A . B^T, bf16 out) on random MXFP4 operands of the
    Mixtral MLP's first GEMM taken as one group: 16384 rows, 28672 columns,
    k = 4096; and mx_grouped_gemm_fp4 on the step's routed rows over its
    split_sizes (one 28672 x 4096 weight per expert); and
    mx_grouped_gemm_fp4_wgrad for the same experts' first weight gradient
    (28672 x 4096 per expert, summed over its routed rows). 2 m n k flops per
    call (k = routed rows for the weight gradient), priced at the FP4 MFMA
    peak."""
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    aq = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device=dev, generator=g)
    bq = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=g)
    as_ = torch.randint(122, 133, (m, k // 32), dtype=torch.uint8, device=dev, generator=g)
    bs = torch.randint(122, 133, (n, k // 32), dtype=torch.uint8, device=dev, generator=g)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        mx.mx_gemm_fp4(aq, as_, bq, bs, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        mx.mx_gemm_fp4(aq, as_, bq, bs, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    # grouped: the step's routed rows (sum of split) over its experts
    G, mg = len(split), int(sum(split))
    ag, ags = aq[:mg], as_[:mg]
    bgq = torch.randint(0, 256, (G, n, k // 2), dtype=torch.uint8, device=dev, generator=g)
    bgs = torch.randint(122, 133, (G, n, k // 32), dtype=torch.uint8, device=dev, generator=g)
    cg = torch.empty((mg, n), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        mx.mx_grouped_gemm_fp4(ag, ags, bgq, bgs, split, out=cg)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        mx.mx_grouped_gemm_fp4(ag, ags, bgq, bgs, split, out=cg)
    e1.record()
    torch.cuda.synchronize()
    msg = e0.elapsed_time(e1) / iters
    tfg = 2.0 * mg * n * k / (msg * 1e-3) / 1e12
    grouped = {"workload": f"grouped_gemm_fp4_{mg}x{n}x{k}_{G}experts", "split_sizes": [int(v) for v in split],
               "ms": round(msg, 4), "tflops": round(tfg, 1), "frac_fp4_peak": round(tfg / PEAK_FP4_TFLOPS, 4)}
    del bgq, bgs, cg
    # weight gradient: dW1[e] = dH[e]^T X[e] (m = n_ffn rows of dH's columnwise
    # copy, n = k = hidden), summed over each expert's routed rows padded to 32
    kw = sum(-(-int(v) // 32) * 32 for v in split)
    wq = torch.randint(0, 256, (n, kw // 2), dtype=torch.uint8, device=dev, generator=g)
    ws = torch.randint(122, 133, (n, kw // 32), dtype=torch.uint8, device=dev, generator=g)
    xq = torch.randint(0, 256, (k, kw // 2), dtype=torch.uint8, device=dev, generator=g)
    xs = torch.randint(122, 133, (k, kw // 32), dtype=torch.uint8, device=dev, generator=g)
    cw = torch.empty((G, n, k), dtype=torch.float32, device=dev)
    for _ in range(3):
        mx.mx_grouped_gemm_fp4_wgrad(wq, ws, xq, xs, split, out=cw)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        mx.mx_grouped_gemm_fp4_wgrad(wq, ws, xq, xs, split, out=cw)
    e1.record()
    torch.cuda.synchronize()
    msw = e0.elapsed_time(e1) / iters
    tfw = 2.0 * mg * n * k / (msw * 1e-3) / 1e12
    wgrad = {"workload": f"grouped_gemm_fp4_wgrad_{n}x{k}x{mg}_{G}experts", "ms": round(msw, 4),
             "tflops": round(tfw, 1), "frac_fp4_peak": round(tfw / PEAK_FP4_TFLOPS, 4)}
    del wq, ws, xq, xs, cw
    nv = measure_nvfp4(mx, torch, dev, split, g, iters, m, n, k)
    return {"workload": f"gemm_fp4_{m}x{n}x{k}", "ms": round(ms, 4), "tflops": round(tflops, 1),
            "grouped": grouped, "wgrad": wgrad, "nvfp4": nv,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_FP4_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP4_TFLOPS, 4)}}


def measure_nvfp4(mx, torch, dev, split, g, iters, m, n, k):
    """NVFP4 on the same shapes: the cast of a 16384 x 4096 bf16 tensor (amax
    reduction + both layouts; bytes = 2 read + 2 x (0.5 + 1/16) written per
    value, plus the amax pass's 2 read), mx_gemm_nvfp4 (16384 x 28672 x 4096)
    and mx_grouped_gemm_nvfp4 over the step's split_sizes. The GEMMs run on
    the fp16 MFMA (gfx950 has no scaled MFMA for E4M3 block scales), so they
    are priced at the 16-bit (bf16 / fp16) peak."""
    x = (torch.randn((m, k), generator=g, device=dev, dtype=torch.float32) * 3).to(torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms_cast = timed(lambda: mx.mx_quantize_nvfp4(x, colwise=True))
    cast_bytes = m * k * (2 + 2 + 2 * (0.5 + 1.0 / 16))
    aq, as_, aa = mx.mx_quantize_nvfp4(x)
    bq = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=g)
    bs = torch.randint(0x28, 0x48, (n, k // 16), dtype=torch.uint8, device=dev, generator=g)
    ba = torch.tensor([1.5], dtype=torch.float32, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: mx.mx_gemm_nvfp4(aq, as_, aa, bq, bs, ba, out=c))
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    G, mg = len(split), int(sum(split))
    bgq = bq.unsqueeze(0).expand(G, n, k // 2).contiguous()
    bgs = bs.unsqueeze(0).expand(G, n, k // 16).contiguous()
    bga = torch.full((G,), 1.5, dtype=torch.float32, device=dev)
    cg = torch.empty((mg, n), dtype=torch.bfloat16, device=dev)
    msg = timed(lambda: mx.mx_grouped_gemm_nvfp4(aq[:mg], as_[:mg], aa, bgq, bgs, bga, split, out=cg))
    tfg = 2.0 * mg * n * k / (msg * 1e-3) / 1e12
    return {"cast": {"workload": f"nvfp4_cast_{m}x{k}_both_layouts", "ms": round(ms_cast, 4),
                     "gbps": round(cast_bytes / (ms_cast * 1e-3) / 1e9, 1)},
            "gemm": {"workload": f"gemm_nvfp4_{m}x{n}x{k}", "ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)},
            "grouped": {"workload": f"grouped_gemm_nvfp4_{mg}x{n}x{k}_{G}experts", "ms": round(msg, 4),
                        "tflops": round(tfg, 1), "frac_bf16_peak": round(tfg / PEAK_BF16_TFLOPS, 4)}}


def measure_quantize(mx, torch, np, wlmod, dev, iters=50, copies=4):
    """mx_quantize on the 16384 x 4096 Student-t tensor (rowwise + columnwise),
    rotating over 4 distinct 128 MiB inputs so re-reads cannot hit the 256 MB
    Infinity Cache. Algorithmic bytes: 2 read + 2 * (1 + 1/32) written per element."""
    bits = wlmod.quantize_tensor_c2()
    first_rows = bits[:1024].copy()
    rows, cols = bits.shape
    base = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [base.clone() for _ in range(copies)]
    del base
    L = mx.load()
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s_row = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    s_col = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    stream = mx._stream()

    def call(t):
        mx._check(L.mx_quantize(mx._ptr(t), mx.MX_BF16, rows, cols, None, 0, mx._ptr(q_row), mx._ptr(s_row),
                                mx._ptr(q_col), mx._ptr(s_col), stream))

    for i in range(8):
        call(xs[i % copies])
    torch.cuda.synchronize()
    # batches of back-to-back launches between one pair of events (an event
    # between every launch would add its own gap to each ~60 us kernel)
    batches = 5
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    evs[0].record()
    for b in range(batches):
        for i in range(iters):
            call(xs[i % copies])
        evs[b + 1].record()
    torch.cuda.synchronize()
    times = [evs[b].elapsed_time(evs[b + 1]) / iters for b in range(batches)]
    # the hand-written device copy of the same inputs (read 128 MiB, write
    # 128 MiB), timed the same way: the practical HBM rate of a cast-shaped
    # read-then-write stream on this device
    dst = torch.empty_like(xs[0])
    nb = xs[0].numel() * 2

    def copy(t):
        mx._check(L.mx_device_copy(mx._ptr(dst), mx._ptr(t), nb, stream))

    for i in range(8):
        copy(xs[i % copies])
    torch.cuda.synchronize()
    evs[0].record()
    for b in range(batches):
        for i in range(iters):
            copy(xs[i % copies])
        evs[b + 1].record()
    torch.cuda.synchronize()
    ctimes = [evs[b].elapsed_time(evs[b + 1]) / iters for b in range(batches)]
    cms = float(np.median(ctimes))
    copy_ref = {"kernel": "mx_device_copy", "bytes": 2 * nb, "median_ms": round(cms, 4),
                "gbps": round(2 * nb / (cms * 1e-3) / 1e9, 1)}
    del dst
    # rowwise MXFP4 of the same tensor: 2 bytes read, 0.5 + 1/32 written per element
    q4 = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    s4 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)

    def call4(t):
        mx._check(L.mx_quantize_fp4(mx._ptr(t), rows, cols, mx._ptr(q4), mx._ptr(s4), None, None, stream))

    for i in range(8):
        call4(xs[i % copies])
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(iters):
        call4(xs[i % copies])
    evs[1].record()
    torch.cuda.synchronize()
    ms4 = evs[0].elapsed_time(evs[1]) / iters
    algo4 = rows * cols * 2 + rows * cols // 2 + rows * cols // 32
    fp4 = {"layouts": "rowwise MXFP4 (E2M1 + E8M0)", "bytes": algo4, "ms": round(ms4, 4),
           "gbps": round(algo4 / (ms4 * 1e-3) / 1e9, 1), "frac_hbm_peak": round(algo4 / (ms4 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    # both layouts (two kernels, each reading x)
    q4c = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
    s4c = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    for i in range(8):
        mx._check(L.mx_quantize_fp4(mx._ptr(xs[i % copies]), rows, cols, mx._ptr(q4), mx._ptr(s4), mx._ptr(q4c),
                                    mx._ptr(s4c), stream))
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(iters):
        mx._check(L.mx_quantize_fp4(mx._ptr(xs[i % copies]), rows, cols, mx._ptr(q4), mx._ptr(s4), mx._ptr(q4c),
                                    mx._ptr(s4c), stream))
    evs[1].record()
    torch.cuda.synchronize()
    ms4b = evs[0].elapsed_time(evs[1]) / iters
    algo4b = rows * cols * 2 + 2 * (rows * cols // 2 + rows * cols // 32)
    fp4["both_layouts_ms"] = round(ms4b, 4)
    fp4["both_layouts_gbps"] = round(algo4b / (ms4b * 1e-3) / 1e9, 1)
    algo = rows * cols * 2 + 2 * (rows * cols + rows * cols // 32)
    med = float(np.median(times))
    gbps = algo / (med * 1e-3) / 1e9
    return {"workload": "quantize_16384x4096", "layouts": "rowwise+columnwise", "bytes": algo,
            "median_ms": round(med, 4), "min_ms": round(float(np.min(times)), 4),
            "timing": f"median over {batches} batches of the mean of {iters} back-to-back launches",
            "copy_reference": dict(copy_ref, quantize_frac_of_copy_rate=round(
                algo / (med * 1e-3) / 1e9 / copy_ref["gbps"], 4)),
            "fp4_rowwise": fp4,
            "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4)}}, first_rows


if __name__ == "__main__":
    main()
