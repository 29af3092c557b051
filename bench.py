"""Benchmark: one MoE expert layer, forward + backward, on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: permutation, gate/up grouped GEMM + SwiGLU, down
grouped GEMM + routing-weight scale, combine, then dH GEMM + SwiGLU backward
+ routing-weight-gradient partials, dX GEMM, dx / d_topk_w reduce, dW13 and
dW2 grouped GEMMs. FP8 precisions add the weight quantization (once per
step, as after an optimizer update) and the activation quantizations.
Default workload: the Qwen3-30B-A3B-shaped layer (T=16384, H=2048, I=768,
E=128, top-8, uniform random routing, bf16); --config picks another layer
shape (ep8_share: blockwise FP8 with fp32 block scales, qwen3_235b: bf16
forward with that FP8 backward, zipf: MXFP8).

Prints one JSON line. `value` is TFLOP/s of algorithmic work
(18 * T * k * H * I flops per step: 6 forward, 12 backward).

    python bench.py [--gpus 1] [--steps 15] [--warmup 5] [--config NAME] [--precision P]
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
COPY_CALIB_BYTES = 1 << 30   # bytes read (and written) by the calibration copy

# algorithmic flops per launch of each GEMM, as a multiple of M*H*I
GEMM_FLOP_FACTOR = {
    "gemm1_swiglu": 4, "gemm2": 2, "gemm_dh_dswiglu": 2, "gemm_dx": 4, "gemm_dw13": 4, "gemm_dw2": 2,
}
GEMM_FLOP_FACTOR.update({k + "_fp8": v for k, v in list(GEMM_FLOP_FACTOR.items())})
# fp32 block scales (fp8_block_f32, fp8_bwd_f32)
GEMM_FLOP_FACTOR.update({k + "f32": v for k, v in list(GEMM_FLOP_FACTOR.items()) if k.endswith("_fp8")})
GEMM_FLOP_FACTOR.update({"gemm1_swiglu_fp8_fp4": 4, "gemm2_fp8_fp4": 2})  # FP8 activations x FP4 weights


def hbm_bytes(name: str, cfg) -> float | None:
    """Algorithmic HBM bytes of one launch of an HBM-bound kernel (each input
    read once, each output written once), or None."""
    T, H, I, k, M = cfg.T, cfg.H, cfg.I, cfg.k, cfg.M
    nparts = 2 * -(-I // 256)
    if name == "permute":  # histogram + scan + scatter: ids and weights in; counts, offsets, maps, row weights out
        return 4.0 * T * k + 4.0 * T * k + 8.0 * cfg.E + 4.0 * (3 * T * k)
    if name == "combine_y" and k > 1:
        return 2.0 * M * H + 4.0 * T * k + 2.0 * T * H
    if name == "combine_dx_dw" and k > 1:
        return 2.0 * M * H + 4.0 * T * k + 2.0 * T * H + 4.0 * M * nparts + 4.0 * T * k

    def quant(rows, K, outs=1):  # bf16 in, E4M3 codes + one E8M0 byte per 32 out (per output layout)
        return rows * K * (2.0 + outs * (1.0 + 1.0 / 32))
    return {"quant_x": lambda: quant(T, H), "quant_dy": lambda: quant(T, H),
            "quant_act": lambda: quant(M, I), "quant_dh13": lambda: quant(M, 2 * I),
            # along tokens: every routed row read once (gathered for x, dY)
            # [dg | du] (and dY under top-1) also get their row codes in the same pass
            "quant_wg_x": lambda: quant(M, H), "quant_wg_dy": lambda: quant(M, H, 2 if k == 1 else 1),
            "quant_wg_dh13": lambda: quant(M, 2 * I, 2), "quant_wg_act": lambda: quant(M, I)}.get(name, lambda: None)()
WORKLOADS = {
    "tiny": "tiny MoE layer",
    "qwen3_30b": "Qwen3-30B-A3B-shaped MoE layer fwd+bwd",
    "ep8_share": "one EP=8 GPU's share of the Qwen3-30B-A3B layer (16 local experts) fwd+bwd",
    "qwen3_235b": "Qwen3-235B-A22B-shaped MoE layer fwd+bwd",
    "zipf": "Qwen3-30B-A3B-shaped MoE layer, Zipf(1.2) routing, fwd+bwd",
}
# timer name -> kernel function name in rocprofv3 output
KERNEL_FN = {
    "gemm1_swiglu": "gemm1_swiglu_kernel<false, false>", "gemm2": "gemm2_kernel<false, false>",
    "gemm_dh_dswiglu": "gemm_dh_kernel<false>", "gemm_dx": "gemm_dx_kernel<false>",
    "gemm1_swiglu_fp8": "gemm1_swiglu_kernel<true, false>", "gemm2_fp8": "gemm2_kernel<true, false>",
    "gemm1_swiglu_fp8_fp4": "gemm1_swiglu_kernel<true, true>", "gemm2_fp8_fp4": "gemm2_kernel<true, true>",
    "gemm_dh_dswiglu_fp8": "gemm_dh_kernel<true>", "gemm_dx_fp8": "gemm_dx_kernel<true>",
    "gemm_dw13": "gemm_dw13_kernel", "gemm_dw2": "gemm_dw2_kernel",
    "gemm1_swiglu_fp8f32": "gemm1_swiglu_kernel<true, false, true>", "gemm2_fp8f32": "gemm2_kernel<true, false, true>",
    "gemm_dh_dswiglu_fp8f32": "gemm_dh_kernel<true, true>", "gemm_dx_fp8f32": "gemm_dx_kernel<true, true>",
}


def kernel_peak(name: str) -> float:
    # an FP8 x FP4 product runs at the FP8 rate (the wider operand's)
    return PEAK_FP8_TFLOPS if name.endswith(("_fp8", "_fp8_fp4", "_fp8f32")) else PEAK_BF16_TFLOPS
WORKLOAD_KEY = ["qwen3_30b/bf16"]   # <config>/<precision>[/...] of this run


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    this workload (profiles/gemm_traffic_<config>_<precision>.json), or None
    when there is none or the kernels changed since it was taken."""
    from grouped_gemm_02_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "gemm_traffic_" + "_".join(WORKLOAD_KEY[0].split("/")[:2]) + ".json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha256") != profile_summary.source_hash():
        return None
    if d.get("workload", "qwen3_30b/bf16") != WORKLOAD_KEY[0]:
        return None
    k = d.get("kernels", {}).get(KERNEL_FN.get(kernel, kernel))
    if not k or "fetch_size_bytes" not in k or "write_size_bytes" not in k:
        return None
    return k["fetch_size_bytes"] + k["write_size_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_30b", choices=sorted(WORKLOADS))
    ap.add_argument("--precision", default=None, choices=["bf16", "fp8_block", "mxfp8", "fp8_bwd", "fp8_fp4",
                                                          "fp8_block_f32", "fp8_bwd_f32"],
                    help="override the configuration's precision")
    ap.add_argument("--wgrad", default="bf16", choices=["bf16", "fp8"],
                    help="weight-gradient GEMMs on bf16 operands, or (FP8 precisions) on operands "
                         "quantized along each expert's rows")
    ap.add_argument("--router", default="none", choices=["none", "uniform", "skewed"],
                    help="include the router step (moe_fwd_logits: the router fused with the permutation's "
                         "first pass; moe_route_bwd after the backward) on synthetic logits: N(0,1), or N(0,1) "
                         "with a Zipf-like per-expert bias")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    return ap.parse_args()


def host_info() -> dict:
    """The host the CPU baseline ran on: logical CPUs, CPUs this process may
    use, the CPU model and the thread settings."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": usable, "logical_cpus": os.cpu_count(), "cpu_model": model,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def _blas_threads() -> int:
    from threadpoolctl import threadpool_info
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return int(max(threads) if threads else 1)


def cpu_baseline(cfg, d, n_tok, n_tok_1core=1024):
    """The CPU oracle, as it stands, on the first n_tok tokens of the workload
    with every BLAS thread, and on the first n_tok_1core tokens with one."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as orc
    W13 = d["W13"].cpu()
    W2 = d["W2"].cpu()

    def run(n):
        sub = {k: d[k][:n].cpu() for k in ("x", "topk_idx", "topk_w", "dy")}
        t0 = time.perf_counter()
        orc.forward(sub["x"], sub["topk_idx"], sub["topk_w"], W13, W2)
        orc.backward(sub["dy"], sub["x"], sub["topk_idx"], sub["topk_w"], W13, W2)
        return time.perf_counter() - t0
    n_tok = min(n_tok, cfg.T)
    dt = run(n_tok)
    threads = _blas_threads()
    n1 = min(n_tok_1core, cfg.T)
    with threadpool_limits(limits=1, user_api="blas"):
        dt1 = run(n1)
    per_tok = 18.0 * cfg.k * cfg.H * cfg.I
    return {"value": per_tok * n_tok / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "one_core": {"value": per_tok * n1 / dt1 / 1e12, "unit": "TFLOP/s", "seconds": round(dt1, 3),
                         "sample": f"first {n1} tokens, BLAS limited to 1 thread"},
            "host": host_info(),
            "sample": f"first {n_tok} tokens of the workload (all {cfg.E} experts, full weights), "
                      f"forward + backward in float64 numpy with {threads} BLAS threads; "
                      f"flops counted as 18*tokens*k*H*I"}


def cpu_baseline_fp8(cfg, d, n_experts, wgrad="bf16"):
    """The CPU oracle's FP8 emulation, as it stands, on the routed pairs of
    the first n_experts experts (other pairs dropped), weight quantization of
    those experts included."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_fp8 as f8
    n_experts = min(n_experts, cfg.E)
    idx = d["topk_idx"].cpu().numpy()
    keep = idx < n_experts
    toks = np.nonzero(keep.any(axis=1))[0]
    sub_idx = np.where(keep[toks], idx[toks], -1)
    pairs = int(keep.sum())
    x = d["x"][toks].cpu()
    dy = d["dy"][toks].cpu()
    w = d["topk_w"][toks].cpu()
    W13 = d["W13"][:n_experts].cpu()
    W2 = d["W2"][:n_experts].cpu()
    t0 = time.perf_counter()
    f8.forward(x, sub_idx, w, W13, W2, cfg.precision)
    f8.backward(dy, x, sub_idx, w, W13, W2, cfg.precision, wgrad=wgrad)
    dt = time.perf_counter() - t0
    flops = 18.0 * pairs * cfg.H * cfg.I
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(threads) if threads else 1),
            "kind": "oracle", "seconds": round(dt, 3),
            "host": host_info(),
            "sample": f"the {pairs} routed pairs of experts 0..{n_experts - 1} ({len(toks)} tokens), "
                      f"{cfg.precision} emulation (weight quantization of those experts included), "
                      f"forward + backward in float64 numpy; flops counted as 18*pairs*H*I"}


def cpu_baseline_fp4(cfg, d, n_experts):
    """The CPU oracle's FP8 x FP4 forward, as it stands, on the routed pairs
    of the first n_experts experts (other pairs dropped), weight
    quantization of those experts included."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_fp4 as f4
    n_experts = min(n_experts, cfg.E)
    idx = d["topk_idx"].cpu().numpy()
    keep = idx < n_experts
    toks = np.nonzero(keep.any(axis=1))[0]
    sub_idx = np.where(keep[toks], idx[toks], -1)
    pairs = int(keep.sum())
    t0 = time.perf_counter()
    f4.forward(d["x"][toks].cpu(), sub_idx, d["topk_w"][toks].cpu(), d["W13"][:n_experts].cpu(),
               d["W2"][:n_experts].cpu())
    dt = time.perf_counter() - t0
    flops = 6.0 * pairs * cfg.H * cfg.I
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(threads) if threads else 1),
            "kind": "oracle", "seconds": round(dt, 3),
            "host": host_info(),
            "sample": f"the {pairs} routed pairs of experts 0..{n_experts - 1} ({len(toks)} tokens), "
                      f"FP8 x FP4 forward emulation (weight quantization of those experts included) "
                      f"in float64 numpy; flops counted as 6*pairs*H*I"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer is one GPU's share: a sharded step adds an all-to-all of the token rows "
              f"before and after it)", file=sys.stderr)
        sys.exit(2)
    import torch

    from grouped_gemm_02_amd import binding as B
    from grouped_gemm_02_amd import inputs

    cfg = inputs.CONFIGS[args.config]
    if args.precision:
        cfg = cfg.scaled(precision=args.precision)
    WORKLOAD_KEY[0] = f"{cfg.name}/{cfg.precision}"
    fp8 = cfg.precision != "bf16"
    fwd_only = cfg.precision == "fp8_fp4"  # an inference forward: no backward
    if args.wgrad == "fp8" and (not fp8 or fwd_only):
        print("--wgrad fp8 needs an FP8 precision with a backward", file=sys.stderr)
        sys.exit(2)
    if args.wgrad == "fp8":
        WORKLOAD_KEY[0] += "/fp8_wgrad"
    if args.router != "none":
        WORKLOAD_KEY[0] += f"/router_{args.router}"
    torch.cuda.set_device(0)
    d = inputs.make_layer_inputs(cfg, "cuda")
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.precision, wgrad=args.wgrad)
    buf = B.LayerBuffers.allocate(shape)
    grads = (torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda"),
             torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda"),
             torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device="cuda"),
             torch.empty((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device="cuda"))
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    if args.router != "none":
        # the router decides the routing each step (renormalised top-k)
        logits = inputs.make_router_logits(cfg.T, cfg.E, cfg.seed + 100, "cuda",
                                           skew=1.2 if args.router == "skewed" else 0.0)
        d["topk_idx"] = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
        d["topk_w"] = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
        d_logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")

    def step(evs=None):
        if evs:
            evs[0].record()
        if fp8:
            B.quantize_weights(buf, d["W13"], d["W2"])
        if evs:
            evs[3].record()
        if args.router != "none":  # the router fused with the permutation's first pass
            B.forward_logits(buf, d["x"], logits, True, d["topk_idx"], d["topk_w"], d["W13"], d["W2"], y=y)
        else:
            B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], y=y)
        if evs:
            evs[1].record()
        if not fwd_only:
            B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], grads=grads)
            if args.router != "none":
                B.moe_route_bwd(shape, logits, d["topk_idx"], d["topk_w"], grads[1], True, d_logits)
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
    # the same copy timed (the measured HBM ceiling of a plain stream)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        calib_out.copy_(calib)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 3 * 2.0 * COPY_CALIB_BYTES / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del calib, calib_out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if B.moe_read_status(buf.fwd_ws) != 0:
        raise RuntimeError("routing status word set")

    # The timed steps: events only around each step and its forward and
    # backward halves. Events around every kernel put gaps between the
    # kernels (~2-3 % of the step), so the kernels' own durations are taken
    # over the next `steps` steps, the same work with per-kernel events.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / args.steps

    B.moe_kernel_timing_collect()          # drop anything recorded before
    B.moe_set_kernel_timing(True)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(args.steps):
        step()
    k1.record()
    torch.cuda.synchronize()
    B.moe_set_kernel_timing(False)
    kt = B.moe_kernel_timing_collect()
    ms_step_kernel_events = k0.elapsed_time(k1) / args.steps
    fwd_ms = [e[3].elapsed_time(e[1]) for e in evs]
    wq_ms = [e[0].elapsed_time(e[3]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
    med = lambda v: (sorted(v)[(len(v) - 1) // 2] + sorted(v)[len(v) // 2]) / 2  # noqa: E731
    flops = cfg.flops_fwd() + (0 if fwd_only else cfg.flops_bwd())
    tflops = flops / (ms_step * 1e-3) / 1e12
    MHI = float(cfg.M) * cfg.H * cfg.I

    kernels = {}
    for name, (n, tot) in sorted(kt.items(), key=lambda kv: -kv[1][1]):
        avg = tot / max(n, 1)
        ent = {"launches": n, "avg_ms": round(avg, 5), "ms_per_step": round(tot / args.steps, 5)}
        if name in GEMM_FLOP_FACTOR:
            ent["tflops"] = round(GEMM_FLOP_FACTOR[name] * MHI / (avg * 1e-3) / 1e12, 1)
            ent["frac_of_peak"] = round(ent["tflops"] / kernel_peak(name), 4)
        nb = hbm_bytes(name, cfg)
        if nb is not None:
            ent["gbps"] = round(nb / (avg * 1e-3) / 1e9, 1)
            ent["frac_of_hbm_peak"] = round(ent["gbps"] / PEAK_HBM_GBS, 4)
        kernels[name] = ent
    perm = [kt[n] for n in ("permute_hist", "permute_scan", "permute_scatter") if n in kt]
    if perm:
        n_launch = perm[0][0]
        tot = sum(t for _, t in perm)
        avg = tot / max(n_launch, 1)
        nb = hbm_bytes("permute", cfg)
        kernels["permute"] = {"launches": n_launch, "avg_ms": round(avg, 5), "ms_per_step": round(tot / args.steps, 5),
                              "avg_us": round(avg * 1e3, 1), "gbps": round(nb / (avg * 1e-3) / 1e9, 1),
                              "frac_of_hbm_peak": round(nb / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "note": "histogram + scan + scatter together (latency-bound)"}
    gemm_names = [n for n in kernels if n in GEMM_FLOP_FACTOR]
    dom = max(gemm_names, key=lambda n: kernels[n]["ms_per_step"])
    dom_avg = kernels[dom]["avg_ms"]
    achieved = GEMM_FLOP_FACTOR[dom] * MHI / (dom_avg * 1e-3) / 1e12
    gemm_ms = sum(kernels[n]["ms_per_step"] for n in gemm_names)
    dtype = {"bf16": "bf16", "fp8_block": "fp8_e4m3+bf16", "mxfp8": "fp8_e4m3+bf16",
             "fp8_bwd": "bf16+fp8_e4m3", "fp8_fp4": "fp8_e4m3+fp4_e2m1", "fp8_block_f32": "fp8_e4m3+bf16",
             "fp8_bwd_f32": "bf16+fp8_e4m3"}[cfg.precision]
    workload = WORKLOADS[cfg.name]
    if fwd_only:
        workload = workload.replace("fwd+bwd", "forward only (inference)")

    out = {
        "metric": METRIC if not fwd_only else METRIC.replace("fwd+bwd", "forward"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {workload}", "T": cfg.T, "H": cfg.H,
                   "I": cfg.I, "E": cfg.E, "k": cfg.k, "routing": cfg.routing, "precision": cfg.precision,
                   "wgrad": args.wgrad, "router": args.router},
        # per-step event times over the timed steps (after the warm-up: with
        # the default 5 + 15 these are the mean, median and min of steps 6-20)
        "step_ms": {"mean": round(sum(step_ms) / len(step_ms), 4), "median": round(med(step_ms), 4),
                    "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4)},
        "fwd_ms": round(sum(fwd_ms) / len(fwd_ms), 4),
        "fwd_ms_median": round(med(fwd_ms), 4),
        "fwd_ms_min": round(min(fwd_ms), 4),
        "bwd_ms": round(sum(bwd_ms) / len(bwd_ms), 4),
        "bwd_ms_median": round(med(bwd_ms), 4),
        "bwd_ms_min": round(min(bwd_ms), 4),
        # a training step with activation checkpointing runs the forward twice
        "two_fwd_plus_bwd_ms": None if fwd_only else round(2 * sum(fwd_ms) / len(fwd_ms) + sum(bwd_ms) / len(bwd_ms), 4),
        "weight_quant_ms": round(sum(wq_ms) / len(wq_ms), 4),
        # the weights are quantized once per optimizer step; a step that reuses
        # them (e.g. gradient accumulation) costs this much
        "ms_per_step_excl_weight_quant": round(ms_step - sum(wq_ms) / len(wq_ms), 4),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_tflops": round((flops) / (gemm_ms * 1e-3) / 1e12, 1),
        "hbm_copy_gbps": round(copy_gbs, 1),
        "wall_s": round(wall, 3),
        # per-kernel durations (kernels, roofline) come from a second run of
        # the same number of steps with an event pair around every kernel;
        # its step time, gaps for the events included:
        "ms_per_step_with_kernel_events": round(ms_step_kernel_events, 4),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": kernel_peak(dom),
                     "unit": "TFLOP/s", "frac": round(achieved / kernel_peak(dom), 4),
                     "traffic": measured_traffic(dom)},
    }
    if not args.no_cpu_baseline:
        if fwd_only:
            n_exp = min(8, max(1, -(-cfg.E * 24576 // cfg.M)))
            out["cpu_baseline"] = cpu_baseline_fp4(cfg, d, n_exp)
        elif fp8:
            # about 24k routed pairs, at most 8 experts (the emulation also
            # quantizes the sampled experts' weights)
            n_exp = min(8, max(1, -(-cfg.E * 24576 // cfg.M)))
            out["cpu_baseline"] = cpu_baseline_fp8(cfg, d, n_exp, args.wgrad)
        else:
            out["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
