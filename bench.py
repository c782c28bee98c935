#!/usr/bin/env python3
"""Benchmark of the fused FP8 FFN chain on one MI355X.

A step is one replay of the captured HIP graph of the whole chain (every
layer's norm+quantise, gate/up GEMM with fused activation and re-quantise,
down GEMM, then the final residual add) over one batch already resident in
HBM.  The headline workload is the dense-LLM decode step (M=1, H=5120,
I=17408, SwiGLU, 64 layers: ~17 GB of FP8 weights streamed per step); the
VLM-prefix chain (M=788, H=2048, I=16384, GeGLU, 18 layers) is measured in the
same run for the MFMA side of the metric.

Printed: one JSON line with the chain latency per layer (the metric), the
roofline of the dominant kernel (HIP events around each kernel on the plan's
stream during a profiled eager forward of the same kernels), and the CPU
oracle timed on this host on a bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA
FP4_PEAK_TFLOPS = 10100.0  # dense FP4 (MXFP4) MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def recorded_traffic(kernel_file_record):
    """HBM bytes per launch from the committed rocprofv3 counter record, or None
    if the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", kernel_file_record)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    for rel, digest in rec.get("sources_sha256", {}).items():
        f = os.path.join(ROOT, rel)
        if not os.path.exists(f) or hashlib.sha256(open(f, "rb").read()).hexdigest() != digest:
            return None
    return rec.get("bytes_per_launch")


def setup(cfg, calibrate=True, keep_layers=(), flags=0):
    """Plan with every layer quantised, calibrated, inputs set, graph captured."""
    from realtime_transformer_amd import datagen
    from realtime_transformer_amd.plan import FFNPlan
    from realtime_transformer_amd import _abi as abi
    t0 = time.time()
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps, flags=flags)
    kept = {}
    for l in range(cfg.L):
        w = datagen.layer_weights(cfg, l)
        plan.load_layer(l, *w)
        if flags & abi.FRT_FLAG_ADA_NORM:
            plan.set_modulation(l, *datagen.modulation(cfg, l))
        if l in keep_layers:
            kept[l] = w
        if l % 8 == 7 or l == cfg.L - 1:
            log("[bench %s] quantised layers 0..%d (%.1fs)" % (cfg.name, l, time.time() - t0))
    r0, y0 = datagen.eval_inputs(cfg)
    if calibrate:
        plan.calibrate(datagen.calib_batches(cfg))
        log("[bench %s] calibrated (%.1fs)" % (cfg.name, time.time() - t0))
    plan.set_inputs(r0, y0)
    plan.capture()
    return plan, kept, (r0, y0)


def time_replays(plan, steps, warmup):
    """Mean ms per replay over `steps` back-to-back replays between two HIP
    events on the plan's stream, and the wall time of that region."""
    import torch
    for _ in range(warmup):
        plan.replay()
    plan.sync()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(plan.stream)
    for _ in range(steps):
        plan.replay()
    e1.record(plan.stream)
    e1.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def replay_percentiles(plan, n):
    """Each of n replays timed on its own (an event pair around it, a wait
    after it): median, p10 and p90 in ms.  Isolated replays include the
    graph launch latency that back-to-back replays overlap."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(plan.stream)
        plan.replay()
        b.record(plan.stream)
        b.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median": round(float(np.median(t)), 4), "p10": round(float(np.percentile(t, 10)), 4),
            "p90": round(float(np.percentile(t, 90)), 4), "n": n}


def per_kernel_ms(plan, reps=3):
    """Average duration (ms) of each kernel kind [norm, gate/up, down]: every
    layer's launch of that kind back to back between two HIP events on the
    plan's stream, reps times."""
    return [plan.time_kernel(k, reps) / 1000.0 for k in range(3)]


def measure_mxfp4(steps, warmup):
    """The MXFP4 variant (FRT_FLAG_MXFP4, AWQ pre-scale set) of the decode and
    action-expert chains: graph replay per layer, per-kernel times, and the
    HBM rate against the 4-bit algorithmic bytes (E2M1 codes + one E8M0 byte
    per 32 values = 17/32 byte per value)."""
    import torch
    from realtime_transformer_amd import _abi, datagen
    from realtime_transformer_amd.configs import BY_NAME
    res = {"format": "OCP MXFP4 (E2M1, E8M0 per 32 along K), AWQ pre-scale, bf16 residual"}
    for name in ("llm_decode_m1", "action_expert_m50", "vlm_prefix_m788"):
        c = BY_NAME[name]
        p, _, _ = setup_mx(c)
        ms, _ = time_replays(p, steps, warmup)
        k = [float(v) for v in per_kernel_ms(p)]
        p.close()
        f = 17.0 / 32
        gu_b = 2 * c.I * c.H * f + c.M * c.H * f + c.M * c.I * f
        dn_b = c.I * c.H * f + c.M * c.I * f + 2 * c.M * c.H
        layer_b = gu_b + dn_b + 7 * c.M * c.H + 2 * c.H
        us = float(ms) * 1000.0 / c.L
        rec = {"us_per_layer": round(us, 3), "layer_bytes": int(layer_b),
               "chain_hbm_gbs": round(layer_b / (us * 1e-6) / 1e9, 1),
               "kernels_us": {"norm_quant": round(k[0] * 1000, 3), "gateup": round(k[1] * 1000, 3),
                              "down": round(k[2] * 1000, 3)}}
        if c.M <= 64:
            gbs = gu_b / (k[1] * 1e-3) / 1e9
            rec["roofline"] = {"bound": "hbm", "kernel": "gemv_gateup_mx", "achieved": round(gbs, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "bytes_per_launch": int(gu_b)}
        else:
            tf_gu = c.gateup_flops() / (k[1] * 1e-3) / 1e12
            tf_chain = c.layer_flops() / (us * 1e-6) / 1e12
            rec["chain_tflops"] = round(tf_chain, 1)
            rec["roofline"] = {"bound": "mfma", "kernel": "mxmm_gateup", "achieved": round(tf_gu, 1),
                               "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf_gu / FP4_PEAK_TFLOPS, 4),
                               "flops_per_launch": c.gateup_flops()}
        res[name] = rec
        log("[bench %s mxfp4] %.2f us/layer (norm %.2f gate/up %.2f down %.2f us)" % (
            name, us, k[0] * 1000, k[1] * 1000, k[2] * 1000))
    return res


def setup_mx(cfg):
    """MXFP4 plan with the AWQ pre-scale and weights of every layer, inputs set, graph captured."""
    from realtime_transformer_amd import _abi, datagen
    from realtime_transformer_amd.plan import FFNPlan
    plan = FFNPlan(cfg.M, cfg.H, cfg.I, cfg.L, cfg.act, cfg.eps, flags=_abi.FRT_FLAG_MXFP4)
    for l in range(cfg.L):
        plan.set_awq(l, datagen.awq_scales(cfg, l))
        plan.load_layer(l, *datagen.layer_weights(cfg, l))
    r0, y0 = datagen.eval_inputs(cfg)
    plan.set_inputs(r0, y0)
    plan.capture()
    return plan, None, (r0, y0)


def measure_qkv(steps, warmup, calibrate=True):
    """Attention-input workloads: graph replay of K1 + fused QKV GEMM with the
    split + rotary epilogue, per-kernel times, and the GEMM's roofline (HBM
    bytes for the GEMV shapes, matrix-core flops for the prefill shape)."""
    import torch
    from realtime_transformer_amd import datagen
    from realtime_transformer_amd.configs import QKV_CONFIGS
    from realtime_transformer_amd.plan import QkvPlan
    res = {}
    for name, c in QKV_CONFIGS.items():
        p = QkvPlan(c.M, c.H, c.nq, c.nkv, c.hd, c.max_pos, c.eps, c.rope_base)
        p.load(*datagen.qkv_weights(c))
        if calibrate:
            p.calibrate(datagen.calib_batches(c))
        else:
            p.set_act_scale(0.01)
        r0, y0 = datagen.eval_inputs(c)
        p.set_inputs(r0, y0, datagen.positions(c))
        p.capture()
        for _ in range(warmup):
            p.replay()
        p.sync()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(p.stream)
        for _ in range(steps):
            p.replay()
        e1.record(p.stream)
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / steps
        k = [p.time_kernel(i, 20) for i in range(2)]
        p.close()
        rec = {"M": c.M, "H": c.H, "heads": [c.nq, c.nkv, c.hd], "us_per_block": round(us, 3),
               "kernels_us": {"norm_quant": round(k[0], 3), "qkv": round(k[1], 3)}}
        if c.M <= 64:
            gbs = c.qkv_bytes() / (k[1] * 1e-6) / 1e9
            rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": c.qkv_bytes()}
        else:
            tf = c.qkv_flops() / (k[1] * 1e-6) / 1e12
            rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(tf / F16_PEAK_TFLOPS, 4), "flops_per_launch": c.qkv_flops(),
                               "note": "f16 matrix cores on exactly converted E4M3 operands; of the FP8 peak: %.4f"
                                       % (tf / FP8_PEAK_TFLOPS)}
        res[name] = rec
        log("[bench %s] %.2f us per block (norm %.2f, qkv %.2f)" % (name, us, k[0], k[1]))
    return res


def cpu_baseline(cfg, kept, inputs, budget_s):
    """Time the CPU oracle's block on the kept layers until budget_s has passed."""
    import oracle
    lws = [oracle.LayerWeights.quantize(*kept[l]) for l in sorted(kept)]
    from realtime_transformer_amd import datagen
    r, y = inputs
    nthreads = oracle.default_threads()
    # static scales from the oracle's own measurement pass over one
    # calibration batch (not timed)
    cal = datagen.calib_batches(cfg, 1)
    pre = oracle.calibrate_and_run([(lambda lw=lw: lw) for lw in lws], cfg.act, cfg.eps, r, y, cal,
                                   nthreads=nthreads)
    scales = list(zip(pre.s_x, pre.s_h))
    done = 0
    t0 = time.perf_counter()
    while True:
        for lw, (s_x, s_h) in zip(lws, scales):
            r, _, _, y = oracle.block(r, y, lw, cfg.act, cfg.eps, s_x, s_h, nthreads)
            done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(el / done * 1e6, 1), "unit": "us/layer", "cores": nthreads, "kind": "oracle",
            "sample": "%d block forwards of the %s workload (M=%d, H=%d, I=%d), exact int64 "
                      "FP8 GEMMs and fp64 norm/activations, weights quantised beforehand"
                      % (done, cfg.name, cfg.M, cfg.H, cfg.I)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llm_decode_m1")
    ap.add_argument("--secondary", default="vlm_prefix_m788", help="second workload or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-fp8-modes", action="store_true",
                    help="skip timing the opt-in FP8 matrix-core modes of the second workload")
    ap.add_argument("--no-norm-variants", action="store_true",
                    help="skip timing the action-expert chain with the norm variants")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip timing the MXFP4 variant of the decode and action-expert chains")
    ap.add_argument("--no-qkv", action="store_true",
                    help="skip timing the attention-input (K1 + fused QKV + rotary) workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first copy this many MiB device-to-device once (a plain copy kernel of known "
                         "size against which HBM byte counters are scaled)")
    ap.add_argument("--no-calibrate", action="store_true",
                    help="skip the calibration pass (scales fixed to 1/448-ish); for profiling runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(token rows would shard across GPUs with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from realtime_transformer_amd.configs import BY_NAME
    from realtime_transformer_amd import _abi
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    _abi.load(build_if_missing=False)

    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    cfg = BY_NAME[args.workload]
    plan, kept, inputs = setup(cfg, calibrate=not args.no_calibrate, keep_layers=(0, 1))
    if args.no_calibrate:
        plan.set_act_scales([0.01] * cfg.L, [0.01] * cfg.L)
        plan.capture()
    ms, wall = time_replays(plan, args.steps, args.warmup)
    pct = replay_percentiles(plan, max(10, min(100, args.steps)))
    kms = [float(v) for v in per_kernel_ms(plan)]
    ms = float(ms)
    plan.close()
    log("[bench %s] %.3f ms/step, kernels (norm, gate/up, down) %s ms" % (cfg.name, ms, np.round(kms, 4)))

    us_layer = ms * 1000.0 / cfg.L
    chain_gbs = cfg.layer_bytes() * cfg.L / (ms * 1e-3) / 1e9
    gu_bytes = cfg.gateup_bytes()
    gu_gbs = gu_bytes / (kms[1] * 1e-3) / 1e9
    out = {
        "metric": "FFN-chain latency (us/layer) + achieved HBM GB/s (M=1) / FP8 MFMA % (M=788)",
        "value": round(us_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 weights/activations, bf16 residual, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) residual, N(0,0.02) weights, calibrated static scales)",
        "config": {"workload": cfg.name, "M": cfg.M, "H": cfg.H, "I": cfg.I, "layers": cfg.L,
                   "activation": {0: "geglu_tanh", 1: "swiglu", 2: "gelu_tanh"}[cfg.act],
                   "tokens_per_s": round(cfg.M / (ms * 1e-3), 2),
                   "chain_hbm_gbs": round(chain_gbs, 1),
                   "chain_hbm_frac": round(chain_gbs / HBM_PEAK_GBS, 4),
                   "wall_s_timed": round(wall, 4),
                   "isolated_replay_ms": pct},
        "roofline": {"bound": "hbm", "kernel": "gemv_gateup", "achieved": round(gu_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("traffic_gemv_gateup_llm_decode_m1.json")
                     if cfg.name == "llm_decode_m1" else None,
                     "bytes_per_launch": gu_bytes,
                     "avg_launch_us": round(float(kms[1]) * 1000, 3),
                     "kernel_us": {"norm_quant": round(float(kms[0]) * 1000, 3),
                                   "gateup": round(float(kms[1]) * 1000, 3),
                                   "down": round(float(kms[2]) * 1000, 3)}},
    }

    if args.secondary and args.secondary != "none":
        from realtime_transformer_amd import _abi as abi
        c2 = BY_NAME[args.secondary]

        def measure(flags):
            p2, _, _ = setup(c2, calibrate=not args.no_calibrate, flags=flags)
            if args.no_calibrate:
                p2.set_act_scales([0.01] * c2.L, [0.01] * c2.L)
                p2.capture()
            ms2, _ = time_replays(p2, args.steps, args.warmup)
            pct2 = replay_percentiles(p2, max(10, min(50, args.steps)))
            k2 = [float(v) for v in per_kernel_ms(p2)]
            p2.close()
            ms2 = float(ms2)
            chain_tf = c2.layer_flops() * c2.L / (ms2 * 1e-3) / 1e12
            gu_tf = c2.gateup_flops() / (k2[1] * 1e-3) / 1e12
            dn_tf = c2.down_flops() / (k2[2] * 1e-3) / 1e12
            return {"us_per_layer": round(ms2 * 1000.0 / c2.L, 3), "ms_per_step": round(ms2, 4),
                    "tokens_per_s": round(c2.M / (ms2 * 1e-3), 1), "chain_tflops": round(chain_tf, 1),
                    "fp8_mfma_frac": round(chain_tf / FP8_PEAK_TFLOPS, 4),
                    "isolated_replay_ms": pct2,
                    "kernels_us": {"norm_quant": round(k2[0] * 1000, 3), "gateup": round(k2[1] * 1000, 3),
                                   "down": round(k2[2] * 1000, 3)},
                    "gateup_tflops": round(gu_tf, 1), "down_tflops": round(dn_tf, 1)}

        base = measure(0)
        out["secondary"] = dict({"workload": c2.name, "M": c2.M, "H": c2.H, "I": c2.I, "layers": c2.L,
                                 "mfma": "f16 matrix cores on exactly converted E4M3 operands (fp32-accurate "
                                         "accumulation; default)",
                                 "gateup_frac_of_f16_peak": round(base["gateup_tflops"] / F16_PEAK_TFLOPS, 4),
                                 "down_frac_of_f16_peak": round(base["down_tflops"] / F16_PEAK_TFLOPS, 4)}, **base)
        log("[bench %s] default: %.2f us/layer, %.1f TFLOP/s chain" % (c2.name, base["us_per_layer"],
                                                                      base["chain_tflops"]))
        if not args.no_fp8_modes:
            # the opt-in FP8 matrix-core modes: same chain, products on the FP8
            # cores (their per-instruction alignment loses low bits: the down
            # GEMM still meets the per-block bf16 tolerance, the gate/up GEMM's
            # re-quantised HQ codes flip ~1e-3 of the time, above the byte
            # tolerance)
            modes = {}
            for name, fl in (("fp8_down", abi.FRT_FLAG_FP8_MFMA_DOWN),
                             ("fp8_both", abi.FRT_FLAG_FP8_MFMA_DOWN | abi.FRT_FLAG_FP8_MFMA_GATEUP)):
                modes[name] = measure(fl)
                log("[bench %s] %s: %.2f us/layer, %.1f TFLOP/s chain" % (c2.name, name, modes[name]["us_per_layer"],
                                                                         modes[name]["chain_tflops"]))
            modes["fp8_down"]["accuracy"] = "per-block bf16 Y within tolerance; chain drifts further than exact sums"
            modes["fp8_both"]["accuracy"] = "HQ code mismatch ~1.4e-3 (above the 1e-4 byte tolerance)"
            out["secondary"]["fp8_matrix_core_modes"] = modes

    if not args.no_norm_variants:
        # the action-expert chain (where the pages place AdaRMSNorm) with the
        # plain norm, the norm weight folded into gate/up, and AdaRMSNorm
        from realtime_transformer_amd import _abi as abi
        c3 = BY_NAME["action_expert_m50"]
        nv = {"workload": c3.name, "M": c3.M, "H": c3.H, "I": c3.I, "layers": c3.L}
        for name, fl in (("plain", 0), ("norm_fuse", abi.FRT_FLAG_NORM_FUSE), ("ada_norm", abi.FRT_FLAG_ADA_NORM)):
            p3, _, _ = setup(c3, calibrate=not args.no_calibrate, flags=fl)
            if args.no_calibrate:
                p3.set_act_scales([0.01] * c3.L, [0.01] * c3.L)
                p3.capture()
            ms3, _ = time_replays(p3, args.steps, args.warmup)
            k3 = [float(v) for v in per_kernel_ms(p3)]
            p3.close()
            nv[name] = {"us_per_layer": round(float(ms3) * 1000.0 / c3.L, 3),
                        "kernels_us": {"norm_quant": round(k3[0] * 1000, 3), "gateup": round(k3[1] * 1000, 3),
                                       "down": round(k3[2] * 1000, 3)}}
            log("[bench %s] %s: %.2f us/layer" % (c3.name, name, nv[name]["us_per_layer"]))
        out["norm_variants"] = nv

    if not args.no_mxfp4:
        out["mxfp4"] = measure_mxfp4(args.steps, args.warmup)

    if not args.no_qkv:
        out["qkv"] = measure_qkv(args.steps, args.warmup, calibrate=not args.no_calibrate)

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle for ~%.0fs" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(cfg, kept, inputs, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
