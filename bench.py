"""Benchmark of the MoE layer on one MI355X.

One step = one layer call over one batch of seeded synthetic inputs already
resident in HBM: moe_forward (moe_forward_hash for hash-routed workloads,
moe_forward_fp8 for FP8-expert workloads), i.e. router, capacity when
configured, permute, (FP8: activation quantisation,) gate/up+SwiGLU GEMM,
down GEMM, combine.  Default workload: the DeepSeek-V3-shaped prefill layer
(16384 tokens, hidden 7168, 256 routed + 1 shared experts, top-8 of 8 groups
/ 4 kept, intermediate 2048, bf16).

Prints one JSON line: tokens/s of the whole job, the roofline of the dominant
kernel (gate/up + SwiGLU grouped GEMM on the bf16 or fp8 matrix cores) timed
live with HIP events on the launch stream, and the CPU oracle timed on a
bounded token sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at DeepSeek-V3 shape; % bf16 MFMA peak / % HBM BW"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "routing_expert_ffn_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_sha(dtype):
    """sha256[:16] of the source of the gate/up kernel of this dtype."""
    name = "gemm_fp8.hip" if dtype == "fp8" else "gemm.hip"
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, dtype):
    """HBM bytes per gate/up launch from the committed counter summary of
    this workload, or None when it is missing or was taken on another kernel
    source."""
    path = os.path.join(ROOT, "profiles", "gateup_swiglu_%s_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"gemm_source_sha:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != gemm_source_sha(dtype):
        return None
    return float(val.group(1))


def cpu_baseline(shape, inp, target_s):
    """The fp64 oracle on a bounded sample of the same workload's tokens."""
    import numpy as np
    import torch

    import oracle
    from tests.hostdata import to_oracle

    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    log("cpu baseline: copying inputs to the host")
    x = to_oracle(inp["x"])
    wr = to_oracle(inp["w_router"])
    sb = to_oracle(inp["sel_bias"])
    lb = to_oracle(inp["logit_bias"])
    wg, wu, wd = to_oracle(inp["w_gate"]), to_oracle(inp["w_up"]), to_oracle(inp["w_down"])
    ids, tab = to_oracle(inp["token_ids"]), to_oracle(inp["tid2eid"])
    sg, su, sd = (to_oracle(inp.get(n)) for n in ("s_gate", "s_up", "s_down"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    order = rng.permutation(shape.T)

    def run(tokens):
        t0 = time.perf_counter()
        logits = oracle.router_logits(shape, x[tokens], wr, lb)
        if tab is not None:
            idx, w, _ = oracle.hash_select(shape, logits, ids[tokens], tab)
        else:
            idx, w, _, _ = oracle.select(shape, logits, sb)
        if shape.dtype == "fp8":
            oracle.forward_tokens_fp8(shape, np.arange(len(tokens)), x[tokens], idx, w,
                                      lambda e: (wg[e], sg[e], wu[e], su[e], wd[e], sd[e]))
        else:
            oracle.forward_tokens(shape, np.arange(len(tokens)), x[tokens], idx, w, lambda e: (wg[e], wu[e], wd[e]))
        return time.perf_counter() - t0

    n1 = max(cores, 4)
    t1 = run(order[:n1])
    per_tok = t1 / n1
    n2 = int(max(0, (target_s - t1) / per_tok))
    n2 = min(n2, shape.T - n1)
    t2 = run(order[n1:n1 + n2]) if n2 > 0 else 0.0
    n = n1 + n2
    secs = t1 + t2
    log("cpu baseline: %d tokens in %.1f s on %d threads" % (n, secs, cores))
    return {"value": n / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d random tokens of the %d-token %s batch: router logits, selection, %d routed + %d shared "
                      "SwiGLU experts each and the combine, fp64, %.1f s" % (n, shape.T, shape.name, shape.k,
                                                                          shape.S, secs)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v3_prefill")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="override the workload's capacity factor (<= 0: unlimited)")
    ap.add_argument("--drop-tokens", action="store_true", help="with a capacity: drop the overflow")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="copy 1 GiB device-to-device 3 times first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import routing_expert_ffn_amd as moe
    from workloads import CONFIGS, make_inputs

    shape = CONFIGS[args.workload]
    if args.capacity_factor is not None or args.drop_tokens:
        cf = shape.capacity_factor if args.capacity_factor is None else args.capacity_factor
        shape = shape.with_(capacity_factor=cf, drop_tokens=args.drop_tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs for", shape.name)
    inp = make_inputs(shape, device=dev)
    cfg = moe.make_config(shape, out_dtype="bf16")
    T = shape.T
    ws = moe.workspace(cfg, T, dev)
    out = torch.empty((T, shape.H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, shape.k), dtype=torch.int32, device=dev)
    counts = torch.empty((shape.E,), dtype=torch.int32, device=dev)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration: 3 device copies of 1 GiB")

    def step():
        if shape.dtype == "fp8":
            moe.forward_fp8(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"],
                            inp["w_down"], inp["s_down"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"],
                            out=out, topk_idx=idx, expert_counts=counts, ws=ws)
        elif inp["tid2eid"] is not None:
            moe.forward_hash(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                             inp["token_ids"], inp["tid2eid"], logit_bias=inp["logit_bias"], out=out, topk_idx=idx,
                             expert_counts=counts, ws=ws)
        else:
            moe.forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                        logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], out=out, topk_idx=idx,
                        expert_counts=counts, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    moe.timing_enable(args.steps * 16)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    kern = moe.timing_read()
    moe.timing_enable(0)
    log("timed %d steps: %.3f ms/step" % (args.steps, total_ms / args.steps))

    assigned = int((idx >= 0).sum().item())
    rows = assigned + shape.S * T
    gateup_flops = 4.0 * shape.H * shape.I * rows
    down_flops = 2.0 * shape.H * shape.I * rows
    layer_flops = shape.flops(assigned)
    ms_step = total_ms / args.steps
    kernels = {name: ms / n for name, (ms, n) in kern.items()}
    gu_ms = kernels.get("gateup_swiglu")
    achieved = gateup_flops / (gu_ms * 1e-3) / 1e12
    touched = int((counts > 0).sum().item())
    wsz = {"fp8": 1, "bf16": 2, "f32": 4}[shape.dtype]
    weight_bytes = (touched + shape.S) * 3 * shape.H * shape.I * wsz
    if shape.dtype == "fp8":  # plus the UE8M0 block scales
        weight_bytes += (touched + shape.S) * 3 * (shape.H // 128) * (shape.I // 128)
    peak = PEAK_FP8_TFLOPS if shape.dtype == "fp8" else PEAK_BF16_TFLOPS
    res = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic",
        "config": {"workload": shape.name, "tokens": T, "hidden": shape.H, "routed_experts": shape.E,
                   "shared_experts": shape.S, "top_k": shape.k, "groups": shape.G, "groups_kept": shape.topk_group,
                   "intermediate": shape.I, "scoring": shape.scoring, "capacity_factor": shape.capacity_factor,
                   "drop_tokens": shape.drop_tokens, "routing": "hash" if shape.hash_vocab else "learned",
                   "out_dtype": "bf16"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic(shape.name, shape.dtype),
                     "kernel": "gateup_swiglu", "flops_per_launch": gateup_flops, "ms_per_launch": gu_ms},
        "layer_tflops": layer_flops / (ms_step * 1e-3) / 1e12,
        "layer_mfma_frac": layer_flops / (ms_step * 1e-3) / 1e12 / peak,
        "layer_weight_gbs": weight_bytes / (ms_step * 1e-3) / 1e9,
        "layer_hbm_frac": weight_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels_ms": kernels,
        "assigned_slots": assigned,
        "touched_experts": touched,
    }
    if shape.T <= 1024:
        # decode-sized: the weight stream is the bound
        res["roofline"] = {"bound": "hbm", "achieved": res["layer_weight_gbs"], "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": res["layer_hbm_frac"], "traffic": None,
                           "kernel": "whole layer (weights of touched experts)"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(shape, inp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
