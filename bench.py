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
bounded token sample.  The same line carries
 - "decode": the decode-sized layer of the same model (128 tokens, capacity
   factor 1.25, Zipf-skewed load), which is bound by reading the weights of
   the experts it touches: ms per layer, touched experts, weight bytes and the
   fraction of HBM bandwidth, per kernel;
 - "attainable": the sustained bf16 matrix-core rate and the HBM streaming
   read rate of this GPU, measured with the library's own probe kernels, and
   the layer's rates as fractions of them next to the nominal peaks.

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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
    return {"value": n / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d random tokens of the %d-token %s batch: router logits, selection, %d routed + %d shared "
                      "SwiGLU experts each and the combine, fp64, %.1f s" % (n, shape.T, shape.name, shape.k,
                                                                          shape.S, secs)}


def run_workload(shape, steps, warmup, dev):
    """Time `steps` layer calls (after `warmup`) of one workload; per-kernel
    launch times from the library's HIP events on the launch stream."""
    import torch

    import routing_expert_ffn_amd as moe
    from workloads import make_inputs

    log("generating inputs for", shape.name)
    inp = make_inputs(shape, device=dev)
    cfg = moe.make_config(shape, out_dtype="bf16")
    T = shape.T
    ws = moe.workspace(cfg, T, dev)
    out = torch.empty((T, shape.H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, shape.k), dtype=torch.int32, device=dev)
    counts = torch.empty((shape.E,), dtype=torch.int32, device=dev)

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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("%s: warmup done" % shape.name)

    # timed region: events around the layer and around the launches of the
    # roofline kernel (gate/up) only -- events around every launch would add
    # tens of microseconds per layer to what is measured
    moe.timing_only("gateup_swiglu")
    moe.timing_enable(steps * 2)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    gu = moe.timing_read().get("gateup_swiglu")
    log("%s: timed %d steps: %.3f ms/step" % (shape.name, steps, total_ms / steps))
    # per-kernel breakdown: a second pass of the same steps, every launch
    # bracketed (not part of the timed region)
    moe.timing_only(None)
    moe.timing_enable(steps * 16)
    for _ in range(steps):
        step()
    kern = moe.timing_read()
    moe.timing_enable(0)
    torch.cuda.synchronize()
    graph_ms, graph_same = graph_replay_ms(step, steps, out)
    log("%s: %d replays of the layer captured in a HIP graph: %.3f ms/step (output %s)"
        % (shape.name, steps, graph_ms, "bit-identical" if graph_same else "DIFFERENT"))

    assigned = int((idx >= 0).sum().item())
    touched = int((counts > 0).sum().item())
    wsz = {"fp8": 1, "bf16": 2, "f32": 4}[shape.dtype]
    per_expert = 3 * shape.H * shape.I * wsz
    if shape.dtype == "fp8":  # plus the UE8M0 block scales
        per_expert += 3 * (shape.H // 128) * (shape.I // 128)
    return {"inp": inp, "ms_step": total_ms / steps, "kernels": {name: ms / n for name, (ms, n) in kern.items()},
            "ms_step_graph": graph_ms, "graph_output_identical": graph_same,
            "gateup_ms": gu[0] / gu[1] if gu else None,
            "assigned": assigned, "touched": touched, "weight_bytes": (touched + shape.S) * per_expert,
            "gateup_weight_bytes": (touched + shape.S) * per_expert * 2 // 3,
            "down_weight_bytes": (touched + shape.S) * per_expert // 3}


def graph_replay_ms(step, steps, out):
    """The same layer call captured once in a HIP graph (torch.cuda.CUDAGraph
    on the library's launches) and replayed `steps` times: ms per replay, and
    whether the replayed output equals the eager one bit for bit (the layer is
    deterministic).  Not the headline figure: the graph removes the host's
    launch overhead that a caller without one pays."""
    import torch

    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref))
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    same = same and bool(torch.equal(out, ref))
    del g
    return a.elapsed_time(b) / steps, same


def decode_record(shape, r):
    """The decode-sized layer: weight-read bound."""
    ms = r["ms_step"]
    k = r["kernels"]
    gbs = r["weight_bytes"] / (ms * 1e-3) / 1e9
    rec = {"workload": shape.name, "tokens": shape.T, "capacity_factor": shape.capacity_factor,
           "ms_per_layer": ms, "tokens_per_s": shape.T / (ms * 1e-3), "touched_experts": r["touched"],
           "assigned_slots": r["assigned"], "weight_bytes": r["weight_bytes"], "weight_gbs": gbs,
           "hbm_frac": gbs / PEAK_HBM_GBS, "kernels_ms": k,
           "ms_per_layer_graph": r["ms_step_graph"], "graph_output_identical": r["graph_output_identical"]}
    for name, key in (("gateup_swiglu", "gateup_weight_bytes"), ("down", "down_weight_bytes")):
        if k.get(name):
            rec[name + "_weight_gbs"] = r[key] / (k[name] * 1e-3) / 1e9
    # HBM bytes of one gate/up launch from the committed counter summary (null
    # when it was taken on another kernel source)
    rec["gateup_traffic"] = measured_traffic(shape.name, shape.dtype)
    return rec


def attainable_rates(dev, mfma_seconds=1.2):
    """Sustained bf16 MFMA rate (about mfma_seconds of back-to-back launches;
    operands that change between instructions, as in a GEMM, and for
    comparison one fixed operand pair), the same for the FP8 experts' scaled
    E4M3 instruction (varying operands), and HBM streaming read rate of this
    GPU, from the library's probe kernels."""
    import torch

    import routing_expert_ffn_amd as moe

    stream = torch.cuda.current_stream()
    blocks = 1024
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()                                     # warm-up launch
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    out = {}
    for probe, vary, key in ((moe.probe_mfma_bf16, True, "mfma_bf16_tflops"),
                             (moe.probe_mfma_bf16, False, "mfma_bf16_tflops_fixed_operands"),
                             (moe.probe_mfma_fp8, True, "mfma_fp8_tflops")):
        # size one launch to about a quarter of the target, then time four
        iters = 20000
        ms = timed(lambda: probe(blocks, iters, sink, vary=vary), 1)
        iters = max(1, int(iters * (mfma_seconds * 250.0) / ms))
        flops = probe(blocks, iters, sink, vary=vary)
        ms = timed(lambda: probe(blocks, iters, sink, vary=vary), 4)
        out[key] = flops / (ms * 1e-3) / 1e12
        log("probe: %s MFMA %.0f TFLOP/s sustained, %s operands (4 launches of %.0f ms)"
            % ("fp8" if probe is moe.probe_mfma_fp8 else "bf16", out[key], "varying" if vary else "fixed", ms))
    out["mfma_seconds"] = 5 * ms * 1e-3
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    read = {}
    rblocks = 256 * 8
    rsink = torch.empty(rblocks * 256, dtype=torch.float32, device=dev)
    for mode, name in ((0, "plain"), (1, "nontemporal"), (2, "to_lds"), (3, "to_lds_nontemporal")):
        rms = timed(lambda: moe.probe_read(buf, mode, rblocks, rsink), 10)
        read[name] = nbytes / (rms * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    log("probe: HBM read %s GB/s" % ", ".join("%s %.0f" % kv for kv in read.items()))
    out.update({"hbm_read_gbs": max(read.values()), "hbm_read_gbs_by_mode": read, "hbm_read_bytes": nbytes})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v3_prefill")
    ap.add_argument("--decode-workload", default="deepseek_v3_decode",
                    help="decode-sized workload measured after the main one ('' to skip)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the attainable-rate probes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="override the workload's capacity factor (<= 0: unlimited)")
    ap.add_argument("--drop-tokens", action="store_true", help="with a capacity: drop the overflow")
    ap.add_argument("--sweep-tokens", default="",
                    help="comma-separated batch sizes: the main workload's layer at each, as a 'sweep' record")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="copy 1 GiB device-to-device 3 times first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import CONFIGS

    shape = CONFIGS[args.workload]
    if args.capacity_factor is not None or args.drop_tokens:
        cf = shape.capacity_factor if args.capacity_factor is None else args.capacity_factor
        shape = shape.with_(capacity_factor=cf, drop_tokens=args.drop_tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration: 3 device copies of 1 GiB")

    r = run_workload(shape, args.steps, args.warmup, dev)
    T = shape.T
    rows = r["assigned"] + shape.S * T
    gateup_flops = 4.0 * shape.H * shape.I * rows
    layer_flops = shape.flops(r["assigned"])
    ms_step = r["ms_step"]
    kernels = r["kernels"]
    gu_ms = r["gateup_ms"]  # launches inside the timed region
    achieved = gateup_flops / (gu_ms * 1e-3) / 1e12
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
        "layer_weight_gbs": r["weight_bytes"] / (ms_step * 1e-3) / 1e9,
        "layer_hbm_frac": r["weight_bytes"] / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels_ms": kernels,  # a separate pass with every launch bracketed
        "ms_per_step_graph": r["ms_step_graph"],  # the same call replayed from a HIP graph
        "graph_output_identical": r["graph_output_identical"],
        "assigned_slots": r["assigned"],
        "touched_experts": r["touched"],
    }
    if shape.T <= 1024:
        # decode-sized: the weight stream is the bound
        res["roofline"] = {"bound": "hbm", "achieved": res["layer_weight_gbs"], "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": res["layer_hbm_frac"], "traffic": None,
                           "kernel": "whole layer (weights of touched experts)"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(shape, r["inp"], args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    del r
    torch.cuda.empty_cache()

    if args.sweep_tokens:
        res["sweep"] = []
        for t in [int(v) for v in args.sweep_tokens.split(",") if v]:
            sshape = shape.with_(name="%s_T%d" % (shape.name, t), T=t)
            d = run_workload(sshape, args.steps, args.warmup, dev)
            ms = d["ms_step"]
            fl = sshape.flops(d["assigned"])
            res["sweep"].append({
                "tokens": t, "ms_per_layer": ms, "tokens_per_s": t / (ms * 1e-3),
                "layer_tflops": fl / (ms * 1e-3) / 1e12, "layer_mfma_frac": fl / (ms * 1e-3) / 1e12 / peak,
                "weight_gbs": d["weight_bytes"] / (ms * 1e-3) / 1e9,
                "hbm_frac": d["weight_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "touched_experts": d["touched"], "assigned_slots": d["assigned"],
                "gateup_ms": d["kernels"].get("gateup_swiglu"), "down_ms": d["kernels"].get("down")})
            log("sweep T=%d: %.3f ms, %.0f tokens/s" % (t, ms, t / (ms * 1e-3)))
            del d
            torch.cuda.empty_cache()

    if args.decode_workload and args.decode_workload != shape.name:
        dshape = CONFIGS[args.decode_workload]
        d = run_workload(dshape, args.steps, args.warmup, dev)
        res["decode"] = decode_record(dshape, d)
        del d
        torch.cuda.empty_cache()

    if not args.no_peaks:
        att = attainable_rates(dev)
        if shape.dtype in ("bf16", "fp8"):
            rate = att["mfma_fp8_tflops" if shape.dtype == "fp8" else "mfma_bf16_tflops"]
            att["layer_frac_of_attainable_mfma"] = res["layer_tflops"] / rate
            att["gateup_frac_of_attainable_mfma"] = achieved / rate
        if "decode" in res:
            att["decode_frac_of_attainable_hbm"] = res["decode"]["weight_gbs"] / att["hbm_read_gbs"]
        res["attainable"] = att
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
