"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Bars (FP8 experts: see check_layer):
 - routing indices, expert counts and the permutation: bit-exact given the
   same fp32 logits;
 - router logits: within 2e-4 absolute of the oracle's fp32-rounded exact dot
   products (fp32 accumulation of bf16 products over H <= 7168);
 - gates: within 1e-5 relative (fp32 gate arithmetic vs fp64);
 - end to end: tokens whose oracle selection margin is below 1e-5 are left out
   of the index comparison (their outputs are checked against the oracle run
   with the GPU's selection); layer outputs within max-abs 2e-2 x RMS(output)
   for bf16 layers and 1e-4 x RMS for fp32 layers, on the fp32-valued output;
   a bf16-stored output additionally gets half a bf16 ulp of the reference.
Capacity layers couple tokens through the expert counts, so their indices are
compared in identical-logits mode (GPU logits fed to the oracle).
"""
import ctypes
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_amd as moe
from tests.hostdata import to_oracle
from workloads import CONFIGS, TEST_SHAPES, make_inputs, zipf_logit_offsets

pytestmark = pytest.mark.gpu

MARGIN = 1e-5
LOGIT_ATOL = 2e-4


def gpu_available():
    return torch.cuda.is_available()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def run_layer(shape, inp, out_dtype):
    cfg = moe.make_config(shape, out_dtype=out_dtype)
    T = inp["x"].shape[0]
    dev = inp["x"].device
    g = dict(
        idx=torch.empty((T, shape.k), dtype=torch.int32, device=dev),
        w=torch.empty((T, shape.k), dtype=torch.float32, device=dev),
        counts=torch.empty((shape.E,), dtype=torch.int32, device=dev),
        logits=torch.empty((T, shape.E), dtype=torch.float32, device=dev),
    )
    if shape.dtype == "fp8":
        g["out"] = moe.forward_fp8(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["s_gate"], inp["w_up"],
                                   inp["s_up"], inp["w_down"], inp["s_down"], logit_bias=inp["logit_bias"],
                                   sel_bias=inp["sel_bias"], topk_idx=g["idx"], topk_w=g["w"],
                                   expert_counts=g["counts"], logits_out=g["logits"])
    elif inp.get("tid2eid") is not None:
        g["out"] = moe.forward_hash(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                                    inp["token_ids"], inp["tid2eid"], logit_bias=inp["logit_bias"],
                                    topk_idx=g["idx"], topk_w=g["w"], expert_counts=g["counts"],
                                    logits_out=g["logits"])
    else:
        g["out"] = moe.forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                               logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], topk_idx=g["idx"],
                               topk_w=g["w"], expert_counts=g["counts"], logits_out=g["logits"])
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in g.items()}


def bf16_half_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return 0.5 * 2.0 ** (e - 7)


def check_layer(shape, inp, g, tokens, out_dtype):
    """Compare one GPU layer call with the oracle on `tokens`."""
    x_h = to_oracle(inp["x"])
    wr_h = to_oracle(inp["w_router"])
    sb = to_oracle(inp["sel_bias"])
    lb = to_oracle(inp["logit_bias"])
    L = g["logits"].numpy()
    idx = g["idx"].numpy()
    hashed = inp.get("tid2eid") is not None
    if hashed:
        ids, tab = to_oracle(inp["token_ids"]), to_oracle(inp["tid2eid"])

        def select(logits, rows):
            i, w, c = oracle.hash_select(shape, logits, ids[rows], tab)
            return i, w, np.full(len(rows), np.inf), c
    else:
        def select(logits, rows):
            return oracle.select(shape, logits, sb)
    # routing from identical logits: bit-exact for every token
    oidx, ow, _, ocounts = select(L, np.arange(L.shape[0]))
    assert np.array_equal(idx, oidx), "routing differs from the oracle on identical logits"
    assert np.array_equal(g["counts"].numpy(), ocounts)
    np.testing.assert_allclose(g["w"].numpy(), ow, rtol=1e-5, atol=1e-6)
    # logits against the oracle's own dot products
    ol = oracle.router_logits(shape, x_h[tokens], wr_h, lb)
    assert np.max(np.abs(L[tokens] - ol)) <= LOGIT_ATOL
    if shape.capacity_factor > 0:
        ref_idx, ref_w = oidx[tokens], ow[tokens]
        keep = np.ones(len(tokens), bool)
    else:
        ref_idx, ref_w, ref_margin, _ = select(ol, tokens)
        keep = ref_margin >= MARGIN
        assert np.array_equal(idx[tokens][keep], ref_idx[keep]), "indices differ from the oracle"
        ref_idx = np.where(keep[:, None], ref_idx, oidx[tokens])
        ref_w = np.where(keep[:, None], ref_w, ow[tokens])

    if shape.dtype == "fp8":
        def get_expert(e):
            return tuple(to_oracle(inp[n][e]) for n in ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"))

        ref = oracle.forward_tokens_fp8(shape, np.arange(len(tokens)), x_h[tokens], ref_idx, ref_w, get_expert)
    else:
        def get_expert(e):
            return to_oracle(inp["w_gate"][e]), to_oracle(inp["w_up"][e]), to_oracle(inp["w_down"][e])

        ref = oracle.forward_tokens(shape, np.arange(len(tokens)), x_h[tokens], ref_idx, ref_w, get_expert)
    out = g["out"].float().numpy().astype(np.float64)[tokens]
    rms = np.sqrt(np.mean(ref ** 2))
    # FP8 experts: h codes that the GPU and the oracle round to neighbouring
    # E4M3 values (the FP8 matrix cores accumulate more loosely than fp32)
    # set the max; the mean catches anything systematic
    rel = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}[shape.dtype]
    tol = rel * rms
    if out_dtype == "bf16":
        tol = tol + bf16_half_ulp(ref)
    err = np.abs(out - ref)
    assert np.all(err <= tol), "max err %.4g x RMS (limit %.1e)" % (np.max(err) / rms, rel)
    if shape.dtype == "fp8":
        assert np.mean(err) <= 2e-3 * rms, "mean err %.4g x RMS" % (np.mean(err) / rms)
    return float(np.max(err) / rms), int((~keep).sum())


# ---- whole layer, reduced shapes, every token -----------------------------------

@pytest.mark.parametrize("name", sorted(TEST_SHAPES))
def test_layer_reduced_shapes_all_tokens(name):
    shape = TEST_SHAPES[name]
    inp = make_inputs(shape, device="cuda")
    for out_dtype in ("f32", "bf16") if shape.dtype != "f32" else ("f32",):
        g = run_layer(shape, inp, out_dtype)
        err, excluded = check_layer(shape, inp, g, np.arange(shape.T), out_dtype)
        print("%s out=%s: max err %.3g x RMS, %d tokens below the margin" % (name, out_dtype, err, excluded))


# ---- whole layer at the workloads' full sizes, sampled tokens --------------------

@pytest.mark.parametrize("name", ["deepseek_v3_decode", "deepseek_v3_prefill", "deepseek_v2", "mixtral_8x7b",
                                  "tiny_mixtral_fp32", "deepseek_v4_flash", "deepseek_v4_flash_hash",
                                  "deepseek_v3_prefill_fp8", "deepseek_v3_decode_fp8"])
def test_layer_full_size_sampled_tokens(name):
    shape = CONFIGS[name]
    inp = make_inputs(shape, device="cuda")
    rng = np.random.default_rng(1234)
    n = min(shape.T, 10)
    tokens = np.unique(np.concatenate([[0, shape.T - 1], rng.choice(shape.T, n, replace=False)]))
    outs = ("bf16", "f32") if shape.dtype != "f32" else ("f32",)
    for out_dtype in outs:
        g = run_layer(shape, inp, out_dtype)
        err, _ = check_layer(shape, inp, g, tokens, out_dtype)
        print("%s out=%s: max err %.3g x RMS on %d tokens" % (name, out_dtype, err, len(tokens)))
        # permutation invariants over all tokens
        counts = g["counts"].numpy()
        idx = g["idx"].numpy()
        assert counts.sum() == (idx >= 0).sum()
    del inp
    torch.cuda.empty_cache()


# ---- stages ----------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,S,drop", [(1, 8, 2, 0, 0.0), (333, 160, 6, 2, 0.0), (2048, 256, 8, 1, 0.05),
                                          (64, 8, 8, 0, 0.3), (4097, 16, 4, 3, 0.0)])
def test_permute_bit_exact(T, E, k, S, drop):
    from workloads import LayerShape
    shape = LayerShape("p", T=T, H=256, E=E, S=S, k=k, I=128)
    rng = np.random.default_rng(T * 7 + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, k)) < drop] = -1
    cfg = moe.make_config(shape)
    counts, offsets, row_token, slot_row = moe.permute(cfg, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    oc, oo, ort, osr = oracle.permute(shape, idx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(row_token.cpu().numpy(), ort)
    assert np.array_equal(slot_row.cpu().numpy(), osr)


def test_expert_ffn_stage_rows():
    shape = TEST_SHAPES["v2_small"]
    inp = make_inputs(shape, device="cuda")
    cfg = moe.make_config(shape)
    T = shape.T
    idx, _ = moe.route(cfg, T, inp["x"], inp["w_router"])
    counts, offsets, row_token, slot_row = moe.permute(cfg, idx)
    y = moe.expert_ffn(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], offsets, row_token)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    rt = row_token.cpu().numpy()
    x_h = to_oracle(inp["x"])
    yh = y.float().cpu().numpy()
    rng = np.random.default_rng(3)
    for e in list(rng.choice(shape.E, 12, replace=False)) + [shape.E, shape.E + 1]:
        if e < shape.E:
            rows = np.arange(off[e], off[e + 1])
        else:
            rows = T * shape.k + (e - shape.E) * T + np.arange(T)
        if rows.size == 0:
            continue
        ref = oracle.expert_rows(shape, x_h[rt[rows]], to_oracle(inp["w_gate"][e]), to_oracle(inp["w_up"][e]),
                                 to_oracle(inp["w_down"][e]))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.max(np.abs(yh[rows] - ref))
        assert err <= 2e-2 * rms + np.max(bf16_half_ulp(ref)), (e, err / rms)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("T0", [256, 4096])
def test_weight_stream_policy_is_bit_identical(fp8, T0):
    """The expert GEMMs copy the weights of an expert whose rows fit one row
    tile with the non-temporal cache policy (gate/up: per item; down: per
    launch, when every expert fits one row tile -- at most 256 tokens -- or,
    bf16, when the routed experts average at most 128 rows) and the others
    with the default one.  A cache hint only: the rows of T0 tokens come out
    bit-identical when one more token is appended (its rows go to the end of
    every expert segment, the earlier rows keep their row tiles and their K
    order).  At 256 -> 257 the shared expert moves to two row tiles (and the
    FP8 down GEMM to the default policy); at 4096 -> 4097 (256 experts,
    top-8: T*k passes 128*E) the bf16 down GEMM does, and expert segments of
    128 rows move to the next tile height."""
    base = TEST_SHAPES["v3_fp8_small" if fp8 else "v3_small"]
    shape = base.with_(T=T0 + 1)
    inp = make_inputs(shape, device="cuda")
    rng = np.random.default_rng(11)
    idx_all = np.stack([rng.permutation(shape.E)[:shape.k] for _ in range(T0 + 1)]).astype(np.int32)
    ys, srs = [], []
    for T in (T0, T0 + 1):
        cfg = moe.make_config(shape.with_(T=T))
        x = inp["x"][:T].contiguous()
        _, offsets, row_token, slot_row = moe.permute(cfg, torch.from_numpy(idx_all[:T]).cuda())
        if fp8:
            y = moe.expert_ffn_fp8(cfg, x, inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"], inp["w_down"],
                                   inp["s_down"], offsets, row_token)
        else:
            y = moe.expert_ffn(cfg, x, inp["w_gate"], inp["w_up"], inp["w_down"], offsets, row_token)
        torch.cuda.synchronize()
        ys.append(y.float().cpu().numpy())
        srs.append(slot_row.cpu().numpy())
    k = shape.k
    a = ys[0][srs[0][:T0].ravel()]
    b = ys[1][srs[1][:T0].ravel()]
    assert np.array_equal(a, b)
    assert np.array_equal(ys[0][T0 * k:T0 * k + T0], ys[1][(T0 + 1) * k:(T0 + 1) * k + T0])   # shared expert rows


def test_expert_ffn_gathers_x_up_to_2gib():
    """The gate/up GEMM gathers token rows through one 32-bit buffer resource
    over x: with x just under 2 GiB (149796 tokens of H = 7168), the rows of
    the last tokens, whose byte offsets approach 2^31, and a random sample of
    others match the oracle.  (One token more is rejected before any launch:
    test_abi.)"""
    from workloads import LayerShape
    H, I = 7168, 128
    T = (2 ** 31 - 1) // (H * 2)
    assert T * H * 2 < 2 ** 31 and (T + 1) * H * 2 >= 2 ** 31
    shape = LayerShape("x_2gib", T=T, H=H, E=2, S=0, k=1, I=I)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    x = (torch.randn(T, H, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    wg = (torch.randn(2, I, H, device="cuda", generator=g) / H ** 0.5).to(torch.bfloat16)
    wu = (torch.randn(2, I, H, device="cuda", generator=g) / H ** 0.5).to(torch.bfloat16)
    wd = (torch.randn(2, H, I, device="cuda", generator=g) / I ** 0.5).to(torch.bfloat16)
    idx = (torch.arange(T, device="cuda", dtype=torch.int32) % 2).view(T, 1)
    cfg = moe.make_config(shape)
    counts, offsets, row_token, slot_row = moe.permute(cfg, idx)
    y = moe.expert_ffn(cfg, x, wg, wu, wd, offsets, row_token)
    torch.cuda.synchronize()
    off, rt = offsets.cpu().numpy(), row_token.cpu().numpy()
    rng = np.random.default_rng(5)
    for e in (0, 1):
        seg = np.arange(off[e], off[e + 1])
        rows = np.concatenate([seg[-48:], rng.choice(seg[:-48], 16, replace=False)])
        toks = rt[rows]
        assert toks.max() >= T - 2
        yr = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
        ref = oracle.expert_rows(shape, to_oracle(x[torch.from_numpy(toks.astype(np.int64)).cuda()]),
                                 to_oracle(wg[e]), to_oracle(wu[e]), to_oracle(wd[e]))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.max(np.abs(yr - ref))
        assert err <= 2e-2 * rms, (e, err / rms)
    del x, y


@pytest.mark.parametrize("dtype,k,S", [("bf16", 4, 2), ("f32", 4, 2), ("bf16", 12, 1), ("bf16", 32, 0),
                                       ("f32", 9, 3)])
def test_combine_stage(dtype, k, S):
    """Combine of expert rows: slots in batches of eight (k up to 32, a
    partial last batch), empty slots, zero to three shared experts."""
    from workloads import LayerShape
    H = 256 if dtype == "bf16" else 64
    shape = LayerShape("c", T=300, H=H, E=40, S=S, k=k, I=128, dtype=dtype)
    rng = np.random.default_rng(4 + k)
    T = shape.T
    idx = np.stack([rng.permutation(40)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, k)) < 0.1] = -1
    _, _, _, slot_row = oracle.permute(shape, idx)
    w = rng.random((T, k)).astype(np.float32)
    y = torch.from_numpy(rng.standard_normal((T * k + S * T, H)).astype(np.float32))
    for out_dtype in ("f32", "bf16"):
        cfg = moe.make_config(shape, out_dtype=out_dtype)
        out = moe.combine(cfg, T, y.cuda(), torch.from_numpy(slot_row).cuda(), torch.from_numpy(w).cuda())
        torch.cuda.synchronize()
        ref = oracle.combine(shape, y.numpy().astype(np.float64), slot_row, w.astype(np.float64))
        o = out.float().cpu().numpy()
        tol = 1e-5 + (bf16_half_ulp(ref) if out_dtype == "bf16" else 1e-6 * np.abs(ref))
        assert np.all(np.abs(o - ref) <= tol)


@pytest.mark.parametrize("E,G,tg,k", [(512, 8, 4, 32), (384, 1, 1, 12)])
def test_layer_many_experts_and_slots(E, G, tg, k):
    """Whole layer with more than 256 routed experts (router GEMM over four
    expert blocks per wavefront, eight experts per lane in the selection) and
    up to 32 slots per token (the combine's slot batches), every token
    against the oracle."""
    shape = TEST_SHAPES["v3_small"].with_(T=203, E=E, G=G, topk_group=tg, k=k)
    inp = make_inputs(shape, device="cuda")
    for out_dtype in ("f32", "bf16"):
        g = run_layer(shape, inp, out_dtype)
        err, excluded = check_layer(shape, inp, g, np.arange(shape.T), out_dtype)
        print("E=%d k=%d out=%s: max err %.3g x RMS, %d tokens below the margin" % (E, k, out_dtype, err, excluded))


@pytest.mark.parametrize("T,H,E", [(8200, 7168, 256), (12811, 1024, 96), (16461, 1024, 200), (8200, 256, 64),
                                   (8063, 2048, 256), (16384, 7168, 256), (16320, 1024, 256), (16321, 512, 128),
                                   (20000, 4096, 256)])
def test_router_gemm_large_batches(T, H, E):
    """The router GEMM at large batch sizes (128-token tiles at one workgroup
    per compute unit, K split into slices, ragged last token tile, ragged last
    slice, slices of one step, 128 or 256 expert columns) and just below them
    (64-token tiles): logits of every token of the first and last tiles and
    of a sample in between against the oracle's dot products, and the routing
    of the GPU logits bit-exact."""
    shape = TEST_SHAPES["v3_small"].with_(T=T, H=H, E=E, G=8 if E % 8 == 0 else 1,
                                         topk_group=4 if E % 8 == 0 else 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(T + H + E)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    sb = (torch.rand((E,), generator=g, device="cuda") * 0.1 - 0.05).contiguous()
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    idx, wts = moe.route(moe.make_config(shape), T, x=x, w_router=w, sel_bias=sb, logits_out=lo,
                         expert_counts=counts)
    torch.cuda.synchronize()
    L = lo.cpu().numpy()
    rng = np.random.default_rng(T)
    tokens = np.unique(np.concatenate([np.arange(130), np.arange(T - 130, T), rng.choice(T, 60, replace=False)]))
    ol = oracle.router_logits(shape, to_oracle(x[tokens]), to_oracle(w))
    assert np.max(np.abs(L[tokens] - ol)) <= LOGIT_ATOL
    oidx, ow, _, oc = oracle.select(shape, L, sb.cpu().numpy())
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_allclose(wts.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("cf", [0.0, 1.25])
def test_large_batch_router_without_logits_output(cf):
    """At a prefill-sized batch the selection is the same with and without a
    logits output (without one the logits live in the workspace) and
    bit-exact with the oracle run on the GPU's logits, with and without a
    capacity limit (Zipf-skewed logits, so experts fill)."""
    T, H, E = 16400, 1024, 256
    shape = TEST_SHAPES["v3_small"].with_(T=T, H=H, E=E, capacity_factor=cf)
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    sb = (torch.rand((E,), generator=g, device="cuda") * 0.1 - 0.05).contiguous()
    lb = torch.from_numpy(zipf_logit_offsets(E, 1.1, 5)).cuda() if cf > 0 else None
    cfg = moe.make_config(shape)
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    c1 = torch.empty(E, dtype=torch.int32, device="cuda")
    c2 = torch.empty(E, dtype=torch.int32, device="cuda")
    i1, w1 = moe.route(cfg, T, x=x, w_router=w, logit_bias=lb, sel_bias=sb, logits_out=lo, expert_counts=c1)
    i2, w2 = moe.route(cfg, T, x=x, w_router=w, logit_bias=lb, sel_bias=sb, expert_counts=c2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(c1, c2)
    oidx, ow, _, oc = oracle.select(shape, lo.cpu().numpy(), sb.cpu().numpy())
    assert np.array_equal(i1.cpu().numpy(), oidx)
    assert np.array_equal(c1.cpu().numpy(), oc)
    np.testing.assert_allclose(w1.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)
    if cf > 0:
        assert oc.max() == oracle.capacity(shape, T)


# ---- routing edge cases ------------------------------------------------------------

def test_route_ties_and_sigmoid_near_ties_from_given_logits():
    shape = TEST_SHAPES["v3_small"]
    T, E = 256, shape.E
    rng = np.random.default_rng(5)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:32] = 0.25                                     # exact ties everywhere
    # logits on consecutive fp32 values: sigmoid scores tie or differ by one ulp
    base = np.float32(0.3)
    L[32:128] = base + np.spacing(base) * rng.integers(0, 6, (96, E)).astype(np.float32)
    L[128:160] = np.float32(90.0) * np.sign(rng.standard_normal((32, E))).astype(np.float32)  # clamp region
    sb = np.zeros(E, np.float32)
    sb[::3] = np.float32(2.0 ** -24)                  # biases at the resolution of the scores
    cfg = moe.make_config(shape)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    Lg = torch.from_numpy(L).cuda()
    idx, w = moe.route(cfg, T, logits_in=Lg, sel_bias=torch.from_numpy(sb).cuda(), expert_counts=counts)
    torch.cuda.synchronize()
    oidx, ow, _, oc = oracle.select(shape, L, sb)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)
    # softmax variant on the same logits
    sm = TEST_SHAPES["v2_small"].with_(E=E, G=1, topk_group=1)
    idx2, w2 = moe.route(moe.make_config(sm), T, logits_in=Lg)
    torch.cuda.synchronize()
    oidx2, ow2, _, _ = oracle.select(sm, L, None)
    assert np.array_equal(idx2.cpu().numpy(), oidx2)
    np.testing.assert_allclose(w2.cpu().numpy(), ow2, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("E,G,tg,k", [(64, 32, 4, 6), (128, 32, 8, 8), (256, 32, 4, 8), (256, 16, 3, 8),
                                      (256, 8, 4, 8), (256, 4, 2, 8), (512, 8, 3, 8), (192, 3, 2, 6),
                                      (160, 8, 3, 6), (96, 4, 2, 4)])
def test_group_limit_every_group_size(E, G, tg, k):
    """Group-limited sigmoid selection for groups of 2, 4, 8, 16, 32 and 64
    experts (kept in place inside a register) and of 20 and 24 (the general
    walk), bit-exact with the oracle on logits with exact ties and scores one
    ulp apart."""
    shape = TEST_SHAPES["v3_small"].with_(E=E, G=G, topk_group=tg, k=k)
    T = 192
    rng = np.random.default_rng(E * 100 + G)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:24] = 0.5                                       # every score ties
    base = np.float32(-0.2)
    L[24:96] = base + np.spacing(base) * rng.integers(0, 4, (72, E)).astype(np.float32)
    sb = (rng.uniform(-0.05, 0.05, E)).astype(np.float32)
    sb[::4] = 0.0
    cfg = moe.make_config(shape)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    idx, w = moe.route(cfg, T, logits_in=torch.from_numpy(L).cuda(), sel_bias=torch.from_numpy(sb).cuda(),
                       expert_counts=counts)
    torch.cuda.synchronize()
    oidx, ow, _, oc = oracle.select(shape, L, sb)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)


def test_sqrtsoftplus_near_ties_from_given_logits():
    """sqrt(softplus) selection is bit-exact: logits one ulp apart, exact
    ties, biases at the resolution of the scores, the clamp region and large
    logits, with and without a group limit."""
    base = TEST_SHAPES["v4_small"]
    T, E = 320, base.E
    rng = np.random.default_rng(6)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:32] = -0.75
    for r0, v in ((32, 0.3), (96, 2.5), (160, -1.7)):
        b = np.float32(v)
        L[r0:r0 + 64] = b + np.spacing(b) * rng.integers(0, 8, (64, E)).astype(np.float32)
    L[224:256] = np.float32(95.0) * np.sign(rng.standard_normal((32, E))).astype(np.float32)
    L[256:288] = rng.uniform(-200, 200, (32, E)).astype(np.float32)
    sb = np.zeros(E, np.float32)
    sb[::5] = np.float32(2.0 ** -23)
    Lg = torch.from_numpy(L).cuda()
    for shape in (base, base.with_(G=8, topk_group=4)):
        cfg = moe.make_config(shape)
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        idx, w = moe.route(cfg, T, logits_in=Lg, sel_bias=torch.from_numpy(sb).cuda(), expert_counts=counts)
        torch.cuda.synchronize()
        oidx, ow, _, oc = oracle.select(shape, L, sb)
        assert np.array_equal(idx.cpu().numpy(), oidx)
        assert np.array_equal(counts.cpu().numpy(), oc)
        np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("scoring,renorm", [("sqrtsoftplus", True), ("sigmoid", True), ("softmax", True),
                                            ("softmax", False)])
def test_hash_routing_table_edge_cases(scoring, renorm):
    """Repeated and out-of-range table entries, ids outside the table, and
    gates of every scoring over the table's experts."""
    shape = TEST_SHAPES["v4_hash_small"].with_(scoring=scoring, renorm=renorm, scale=1.7)
    E, k, V, T = shape.E, shape.k, 97, 700
    rng = np.random.default_rng(12)
    tab = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    tab[3, 2] = tab[3, 0]                 # repeated entries
    tab[4, :] = tab[4, 1]
    tab[5, 1], tab[5, 4] = -1, E          # out of range
    tab[6, :] = 2 ** 30
    ids = rng.integers(-3, V + 3, T).astype(np.int32)   # some outside the table
    ids[:40] = np.arange(40) % 8
    L = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    cfg = moe.make_config(shape)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, w = moe.route_hash(cfg, T, torch.from_numpy(ids).cuda(), torch.from_numpy(tab).cuda(),
                            logits_in=torch.from_numpy(L).cuda(), logits_out=lo, expert_counts=counts)
    torch.cuda.synchronize()
    oidx, ow, oc = oracle.hash_select(shape, L, ids, tab)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(lo.cpu().numpy(), L)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)
    assert (oidx < 0).any() and (oidx >= 0).any()


@pytest.mark.parametrize("cf", [0.3, 1.25])
def test_hash_routing_drop_capacity_and_empty_table(cf):
    shape = TEST_SHAPES["v4_hash_small"].with_(capacity_factor=cf, drop_tokens=True)
    inp = make_inputs(shape, device="cuda")
    g = run_layer(shape, inp, "f32")
    C = oracle.capacity(shape, shape.T)
    assert g["counts"].numpy().max() <= C
    check_layer(shape, inp, g, np.arange(shape.T), "f32")
    # re-routing has no next-best expert under hash routing: rejected
    cfg = moe.make_config(shape.with_(drop_tokens=False))
    with pytest.raises(moe.MoeError):
        moe.route_hash(cfg, shape.T, inp["token_ids"], inp["tid2eid"], x=inp["x"], w_router=inp["w_router"])
    # a table with no rows: every slot empty, the shared expert alone remains
    cfg = moe.make_config(shape.with_(capacity_factor=0.0))
    empty = torch.empty((0, shape.k), dtype=torch.int32, device="cuda")
    idx, w = moe.route_hash(cfg, shape.T, inp["token_ids"], empty, x=inp["x"], w_router=inp["w_router"])
    torch.cuda.synchronize()
    assert bool((idx == -1).all()) and bool((w == 0).all())


@pytest.mark.parametrize("cf,drop", [(0.25, False), (1.0, False), (1.2, False), (1.25, False), (0.25, True),
                                     (1.0, True), (1.2, True), (1.25, True)])
def test_capacity_with_drops_and_overflow(cf, drop):
    """Re-route mode (overflow to the next-best allowed expert) and drop mode
    (overflow assignments dropped, the top-k's gates kept)."""
    shape = TEST_SHAPES["v3_decode_small"].with_(capacity_factor=cf, drop_tokens=drop)
    inp = make_inputs(shape, device="cuda")
    g = run_layer(shape, inp, "f32")
    idx = g["idx"].numpy()
    C = oracle.capacity(shape, shape.T)
    assert g["counts"].numpy().max() <= C
    if cf < 1:
        assert (idx < 0).any()
    check_layer(shape, inp, g, np.arange(shape.T), "f32")


@pytest.mark.parametrize("T,cf,G", [(2048, 1.0, 8), (5000, 1.25, 8), (16384, 1.25, 8), (16384, 0.5, 1),
                                    (9000, 2.0, 8)])
def test_capacity_rounds_match_oracle(T, cf, G):
    """Large batches take the block-round capacity pass: bit-exact with the
    oracle's serial first-come-first-served walk, on skewed logits where
    experts fill inside blocks."""
    E = 256
    shape = TEST_SHAPES["v3_small"].with_(T=T, G=G, topk_group=4 if G > 1 else 1, capacity_factor=cf)
    rng = np.random.default_rng(T + int(cf * 10))
    skew = zipf_logit_offsets(E, 1.2, 7) * 2.0
    L = (rng.standard_normal((T, E)) + skew).astype(np.float32)
    sb = (rng.uniform(-0.05, 0.05, E)).astype(np.float32)
    cfg = moe.make_config(shape)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    idx, w = moe.route(cfg, T, logits_in=torch.from_numpy(L).cuda(), sel_bias=torch.from_numpy(sb).cuda(),
                       expert_counts=counts)
    torch.cuda.synchronize()
    oidx, ow, _, oc = oracle.select(shape, L, sb)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)
    assert oc.max() == oracle.capacity(shape, T) or cf >= 2.0


@pytest.mark.parametrize("cf,T,k,E", [(1.2, 160, 8, 256), (1.1, 320, 8, 256), (0.3, 320, 8, 256), (1.2, 40, 2, 8)])
@pytest.mark.parametrize("drop", [False, True])
@pytest.mark.parametrize("ranking", ["shared", "skewed"])
def test_capacity_value_for_decimal_factors(cf, T, k, E, drop, ranking):
    """Capacity factors that fp32 cannot represent (1.2 is the GPT-4 page's
    configured value) give the same C on the library and the oracle: C =
    ceil(((cf*T)*k)/E) in IEEE double.  At these sizes cf*T*k/E is an
    integer in decimal, where an fp32 factor would make C one larger.  With
    every token ranking the experts alike the first experts fill to exactly
    C, which pins C; indices and counts are bit-exact with the oracle in
    re-route and drop mode."""
    if E == 8:
        shape = TEST_SHAPES["mixtral_small"].with_(T=T, E=E, k=k)
    else:
        shape = TEST_SHAPES["v3_small"].with_(T=T, E=E, k=k)
    shape = shape.with_(capacity_factor=cf, drop_tokens=drop)
    C = math.ceil(cf * T * k / E)
    assert C == math.ceil(Fraction(repr(cf)) * T * k / E)   # the decimal value
    assert oracle.capacity(shape, T) == C
    rng = np.random.default_rng(T + E + int(drop))
    if ranking == "shared":
        L = np.tile(np.linspace(1.0, -1.0, E, dtype=np.float32), (T, 1))
        L += rng.standard_normal((T, E)).astype(np.float32) * 1e-3
    else:
        L = (rng.standard_normal((T, E)) + zipf_logit_offsets(E, 1.2, 3) * 2.0).astype(np.float32)
    sb = rng.uniform(-0.05, 0.05, E).astype(np.float32) if shape.scoring == "sigmoid" else None
    cfg = moe.make_config(shape)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    idx, w = moe.route(cfg, T, logits_in=torch.from_numpy(L).cuda(),
                       sel_bias=None if sb is None else torch.from_numpy(sb).cuda(), expert_counts=counts)
    torch.cuda.synchronize()
    oidx, ow, _, oc = oracle.select(shape, L, sb)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.array_equal(counts.cpu().numpy(), oc)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-6)
    assert oc.max() <= C
    if ranking == "shared":
        assert oc.max() == C


def test_all_tokens_to_one_expert():
    shape = TEST_SHAPES["mixtral_small"].with_(T=700)
    inp = make_inputs(shape, device="cuda")
    lb = torch.zeros(shape.E, dtype=torch.float32, device="cuda")
    lb[3] = 100.0
    inp["logit_bias"] = lb
    g = run_layer(shape, inp, "f32")
    assert np.all(g["idx"].numpy()[:, 0] == 3)
    assert g["counts"].numpy()[3] == shape.T
    check_layer(shape, inp, g, np.arange(0, shape.T, 7), "f32")


@pytest.mark.parametrize("T", [1, 2, 63, 65])
def test_small_batches(T):
    shape = TEST_SHAPES["v3_small"].with_(T=T)
    inp = make_inputs(shape, device="cuda")
    g = run_layer(shape, inp, "f32")
    check_layer(shape, inp, g, np.arange(T), "f32")


def test_top1_single_group():
    shape = TEST_SHAPES["mixtral_small"].with_(name="top1", k=1, T=130)
    inp = make_inputs(shape, device="cuda")
    g = run_layer(shape, inp, "f32")
    check_layer(shape, inp, g, np.arange(shape.T), "f32")


def test_empty_batch_leaves_output_untouched():
    """T == 0 is a successful no-op: every output buffer passed in (here
    non-empty and pre-filled) keeps its contents, for the layer and the
    router; the permutation reports zero rows for every expert."""
    shape = TEST_SHAPES["v3_small"]
    inp = make_inputs(shape, device="cuda", T=1)
    cfg = moe.make_config(shape, out_dtype="f32")
    x0 = inp["x"][:0]
    E, k = shape.E, shape.k
    out = torch.full((4, shape.H), 7.0, device="cuda")
    idx = torch.full((4, k), 7, dtype=torch.int32, device="cuda")
    w = torch.full((4, k), 7.0, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), 7, dtype=torch.int32, device="cuda")
    logits = torch.full((4, E), 7.0, dtype=torch.float32, device="cuda")
    L = moe.lib()
    st = L.moe_forward(ctypes.byref(cfg), 0, moe._p(x0), moe._p(inp["w_router"]), None, moe._p(inp["sel_bias"]),
                       moe._p(inp["w_gate"]), moe._p(inp["w_up"]), moe._p(inp["w_down"]), moe._p(out), moe._p(idx),
                       moe._p(w), moe._p(counts), moe._p(logits), None, 0, moe._stream(None))
    assert st == 0
    st = L.moe_route(ctypes.byref(cfg), 0, moe._p(x0), moe._p(inp["w_router"]), None, moe._p(inp["sel_bias"]),
                     None, moe._p(logits), moe._p(idx), moe._p(w), moe._p(counts), None, 0, moe._stream(None))
    assert st == 0
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((idx == 7).all()) and bool((w == 7.0).all())
    assert bool((counts == 7).all()) and bool((logits == 7.0).all())
    c, off, _, _ = moe.permute(cfg, torch.empty((0, k), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((c == 0).all()) and bool((off == 0).all())


def test_deterministic_bitwise():
    shape = TEST_SHAPES["v3_small"]
    inp = make_inputs(shape, device="cuda")
    a = run_layer(shape, inp, "bf16")
    b = run_layer(shape, inp, "bf16")
    for key in ("out", "idx", "w", "logits", "counts"):
        assert torch.equal(a[key], b[key]), key


def test_timing_records_every_kernel():
    shape = TEST_SHAPES["v3_small"]
    inp = make_inputs(shape, device="cuda")
    moe.timing_enable(64)
    run_layer(shape, inp, "bf16")
    t = moe.timing_read()
    moe.timing_enable(0)
    for name in ("router", "permute_count", "permute_scan", "permute_scatter", "schedule", "gateup_swiglu", "down",
                 "combine"):
        assert name in t and t[name][1] == 1 and t[name][0] > 0.0, name
    # only the selected kernel's launches are bracketed
    moe.timing_only("gateup_swiglu")
    moe.timing_enable(64)
    run_layer(shape, inp, "bf16")
    run_layer(shape, inp, "bf16")
    t = moe.timing_read()
    moe.timing_enable(0)
    moe.timing_only(None)
    assert list(t) == ["gateup_swiglu"] and t["gateup_swiglu"][1] == 2 and t["gateup_swiglu"][0] > 0.0


def test_native_library_is_the_one_loaded():
    moe.lib()
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(moe.LIB_PATH) in maps
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


def test_expert_ffn_row_tile_boundaries():
    """Experts whose row counts sit on and around the row-tile sizes (full
    256-row tiles, last tiles of 129-192 rows that run three 32-row blocks per
    wavefront, and the short last tiles of at most 128 rows that run at half
    height in pairs of column tiles)."""
    from workloads import LayerShape
    counts = [128, 256, 129, 1, 0, 127, 255, 257, 384, 385, 513, 540, 577, 1050, 160, 192, 193, 448, 449]
    E = len(counts)
    T = max(counts)
    shape = LayerShape("tb", T=T, H=256, E=E, S=1, k=E, I=256)
    # token t is routed to every expert e with t < counts[e] (slots in expert order)
    idx = np.full((T, E), -1, np.int32)
    for t in range(T):
        es = [e for e in range(E) if t < counts[e]]
        idx[t, :len(es)] = es
    inp = make_inputs(shape, device="cuda")
    cfg = moe.make_config(shape)
    c, off, rt, sr = moe.permute(cfg, torch.from_numpy(idx).cuda())
    y = moe.expert_ffn(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], off, rt)
    torch.cuda.synchronize()
    assert c.cpu().numpy().tolist() == counts
    offh, rth, yh = off.cpu().numpy(), rt.cpu().numpy(), y.cpu().numpy()
    x_h = to_oracle(inp["x"])
    for e in list(range(E)) + [E]:
        rows = np.arange(offh[e], offh[e + 1]) if e < E else T * E + np.arange(T)
        if rows.size == 0:
            continue
        ref = oracle.expert_rows(shape, x_h[rth[rows]], to_oracle(inp["w_gate"][e]), to_oracle(inp["w_up"][e]),
                                 to_oracle(inp["w_down"][e]))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.max(np.abs(yh[rows] - ref))
        assert err <= 2e-2 * rms, (e, counts[e] if e < E else T, err / rms)


# ---- auxiliary-loss-free balancing step -------------------------------------------

@pytest.mark.parametrize("case", ["forward_counts", "random", "at_mean", "empty"])
def test_balance_update_matches_oracle(case):
    shape = TEST_SHAPES["v3_small"]
    cfg = moe.make_config(shape)
    E = shape.E
    rng = np.random.default_rng(17)
    if case == "forward_counts":
        inp = make_inputs(shape, device="cuda")
        g = run_layer(shape, inp, "f32")
        counts = g["counts"].numpy().astype(np.int32)
    elif case == "random":
        counts = rng.poisson(40, E).astype(np.int32)
        counts[:7] = 0
    elif case == "at_mean":
        counts = np.full(E, 9, np.int32)
        counts[0], counts[1] = 12, 6          # the mean stays 9
    else:
        counts = np.zeros(E, np.int32)
    b0 = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    bias = torch.from_numpy(b0.copy()).cuda()
    share, stats = moe.balance_update(cfg, torch.from_numpy(counts).cuda(), bias, 0.001)
    torch.cuda.synchronize()
    ob, oshare, ost = oracle.balance_update(counts, b0, 0.001)
    assert np.array_equal(bias.cpu().numpy(), ob)                     # the fp32 step is exact
    np.testing.assert_allclose(share.cpu().numpy(), oshare, rtol=1e-7, atol=0)
    st = stats.cpu().numpy()
    np.testing.assert_allclose(st[0], ost["entropy"], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(st[1], ost["max_share"], rtol=1e-7)
    assert int(st[2]) == ost["over"] and int(st[3]) == ost["under"]
