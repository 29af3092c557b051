"""Benchmark: one MoE expert layer, forward + backward, on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: permutation, gate/up grouped GEMM + SwiGLU, down
grouped GEMM + routing-weight scale, combine, then dH GEMM + SwiGLU backward
+ routing-weight-gradient partials, dX GEMM, dx / d_topk_w reduce, dW13 and
dW2 grouped GEMMs. Workload: the Qwen3-30B-A3B-shaped layer (T=16384, H=2048,
I=768, E=128, top-8, uniform random routing, bf16).

Prints one JSON line. `value` is TFLOP/s of algorithmic work
(18 * T * k * H * I flops per step: 6 forward, 12 backward).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd ms and TFLOP/s (frac of MFMA peak), Qwen3-30B-A3B shape, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
COPY_CALIB_BYTES = 1 << 30   # bytes read (and written) by the calibration copy

# algorithmic flops per launch of each GEMM, as a multiple of M*H*I
GEMM_FLOP_FACTOR = {
    "gemm1_swiglu": 4, "gemm2": 2, "gemm_dh_dswiglu": 2, "gemm_dx": 4, "gemm_dw13": 4, "gemm_dw2": 2,
}
# timer name -> kernel function name in rocprofv3 output
KERNEL_FN = {
    "gemm1_swiglu": "gemm1_swiglu_kernel", "gemm2": "gemm2_kernel", "gemm_dh_dswiglu": "gemm_dh_kernel",
    "gemm_dx": "gemm_dx_kernel", "gemm_dw13": "gemm_dw13_kernel", "gemm_dw2": "gemm_dw2_kernel",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_qwen3_30b_bf16.json")


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none or the kernels changed since it was taken."""
    from grouped_gemm_02_amd import profile_summary
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("source_sha256") != profile_summary.source_hash():
        return None
    k = d.get("kernels", {}).get(KERNEL_FN.get(kernel, kernel))
    if not k or "fetch_size_bytes" not in k or "write_size_bytes" not in k:
        return None
    return k["fetch_size_bytes"] + k["write_size_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_30b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    return ap.parse_args()


def cpu_baseline(cfg, d, n_tok):
    """The CPU oracle, as it stands, on the first n_tok tokens of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as orc
    n_tok = min(n_tok, cfg.T)
    sub = {k: d[k][:n_tok].cpu() for k in ("x", "topk_idx", "topk_w", "dy")}
    W13 = d["W13"].cpu()
    W2 = d["W2"].cpu()
    t0 = time.perf_counter()
    orc.forward(sub["x"], sub["topk_idx"], sub["topk_w"], W13, W2)
    orc.backward(sub["dy"], sub["x"], sub["topk_idx"], sub["topk_w"], W13, W2)
    dt = time.perf_counter() - t0
    flops = 18.0 * n_tok * cfg.k * cfg.H * cfg.I
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(threads) if threads else 1),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"first {n_tok} tokens of the workload (all {cfg.E} experts, full weights), "
                      f"forward + backward in float64 numpy; flops counted as 18*tokens*k*H*I"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer is one GPU's share; see DESIGN.md on sharding)", file=sys.stderr)
        sys.exit(2)
    import torch

    from grouped_gemm_02_amd import binding as B
    from grouped_gemm_02_amd import inputs

    cfg = inputs.CONFIGS[args.config]
    if cfg.precision != "bf16":
        cfg = cfg.scaled(precision="bf16")
    torch.cuda.set_device(0)
    d = inputs.make_layer_inputs(cfg, "cuda")
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.precision)
    buf = B.LayerBuffers.allocate(shape)
    grads = (torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda"),
             torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda"),
             torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device="cuda"),
             torch.empty((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device="cuda"))
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def step(evs=None):
        if evs:
            evs[0].record()
        B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], y=y)
        if evs:
            evs[1].record()
        B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], grads=grads)
        if evs:
            evs[2].record()

    # A plain device-to-device copy of known size: rocprofv3 counter runs
    # (FETCH_SIZE / WRITE_SIZE) use it to calibrate the layer kernels' HBM
    # traffic. Outside the timed region.
    calib = torch.empty(COPY_CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    calib.zero_()
    torch.cuda.synchronize()
    calib_out = calib.clone()
    torch.cuda.synchronize()
    del calib, calib_out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if B.moe_read_status(buf.fwd_ws) != 0:
        raise RuntimeError("routing status word set")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    B.moe_kernel_timing_collect()          # drop anything recorded before
    B.moe_set_kernel_timing(True)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    B.moe_set_kernel_timing(False)
    kt = B.moe_kernel_timing_collect()

    ms_step = start.elapsed_time(stop) / args.steps
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    flops = cfg.flops_fwd() + cfg.flops_bwd()
    tflops = flops / (ms_step * 1e-3) / 1e12
    MHI = float(cfg.M) * cfg.H * cfg.I

    kernels = {}
    for name, (n, tot) in sorted(kt.items(), key=lambda kv: -kv[1][1]):
        avg = tot / max(n, 1)
        ent = {"launches": n, "avg_ms": round(avg, 5), "ms_per_step": round(tot / args.steps, 5)}
        if name in GEMM_FLOP_FACTOR:
            ent["tflops"] = round(GEMM_FLOP_FACTOR[name] * MHI / (avg * 1e-3) / 1e12, 1)
        kernels[name] = ent
    gemm_names = [n for n in kernels if n in GEMM_FLOP_FACTOR]
    dom = max(gemm_names, key=lambda n: kernels[n]["ms_per_step"])
    dom_avg = kernels[dom]["avg_ms"]
    achieved = GEMM_FLOP_FACTOR[dom] * MHI / (dom_avg * 1e-3) / 1e12
    gemm_ms = sum(kernels[n]["ms_per_step"] for n in gemm_names)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Qwen3-30B-A3B-shaped MoE layer fwd+bwd", "T": cfg.T, "H": cfg.H,
                   "I": cfg.I, "E": cfg.E, "k": cfg.k, "routing": cfg.routing, "precision": cfg.precision},
        "fwd_ms": round(sum(fwd_ms) / len(fwd_ms), 4),
        "bwd_ms": round(sum(bwd_ms) / len(bwd_ms), 4),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_tflops": round((flops) / (gemm_ms * 1e-3) / 1e12, 1),
        "wall_s": round(wall, 3),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
