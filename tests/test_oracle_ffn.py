"""Pins of the oracle's expert FFN and combine.

Expert = SwiGLU FFN with gate, up and down matrices ("MoE on KnightLi的博客",
activation-function section; "15. DeepSeek：MLA、MoE 与 MTP", section
"671B 和 37B 的参数账": gate, up, down = three H x I matrices).  Layer output =
gate-weighted sum of the chosen experts plus the shared experts (same page,
section "V3 的 MoE：256 个专家怎样选 8 个", last line of the router sketch).

The pages print no worked numeric example, so values are pinned by closed
forms (selection matrices + sigmoid(ln 3) = 3/4), a dense special case checked
against a library matmul, and structural identities.
"""
import math

import numpy as np

import oracle
from workloads import LayerShape

LN3 = math.log(3.0)


def f32shape(**kw):
    base = dict(name="f", T=1, H=4, E=1, S=0, k=1, I=6, dtype="f32")
    base.update(kw)
    return LayerShape(**base)


def selection_matrix(rows, cols, pick):
    m = np.zeros((rows, cols), np.float32)
    m[np.arange(rows), pick] = 1.0
    return m


def silu_closed(v):
    """silu at the closed-form points used here: 0, +-ln3."""
    if v == 0.0:
        return 0.0
    if abs(v - LN3) < 1e-6:
        return 0.75 * v
    if abs(v + LN3) < 1e-6:
        return 0.25 * v
    raise AssertionError(v)


def test_swiglu_closed_form_with_selection_matrices():
    H, I = 4, 6
    cfg = f32shape(H=H, I=I)
    x = np.array([[0.0, LN3, -LN3, LN3]], np.float32)
    a = np.array([1, 2, 3, 0, 1, 2])   # gate row i reads x[a[i]]
    b = np.array([3, 3, 0, 1, 2, 1])   # up row i reads x[b[i]]
    c = np.array([4, 0, 5, 2])         # output n reads h[c[n]]
    wg = selection_matrix(I, H, a)
    wu = selection_matrix(I, H, b)
    wd = selection_matrix(H, I, c)
    y = oracle.expert_rows(cfg, x, wg, wu, wd)[0]
    xv = x[0].astype(np.float64)
    want = [silu_closed(float(x[0, a[c[n]]])) * xv[b[c[n]]] for n in range(H)]
    np.testing.assert_allclose(y, want, rtol=2e-7, atol=1e-12)


def test_single_expert_layer_is_a_dense_swiglu_ffn():
    # E = 1, k = 1, renormalised softmax: gate = 1, so the layer is the dense FFN
    rng = np.random.default_rng(3)
    H, I, T = 32, 48, 7
    cfg = f32shape(T=T, H=H, I=I)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((1, H)).astype(np.float32)
    wg = (rng.standard_normal((1, I, H)) / np.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((1, I, H)) / np.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((1, H, I)) / np.sqrt(I)).astype(np.float32)
    res = oracle.forward(cfg, x, wr, wg, wu, wd)
    assert np.all(res["idx"] == 0) and np.all(res["w"] == 1.0)
    xd = x.astype(np.float64)
    g = xd @ wg[0].astype(np.float64).T
    u = xd @ wu[0].astype(np.float64).T
    ref = (g * (1.0 / (1.0 + np.exp(-g))) * u) @ wd[0].astype(np.float64).T
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_factor_out():
    # every routed expert equal -> out = (sum of gates) * FFN(x) + shared(x)
    rng = np.random.default_rng(4)
    H, I, T, E, S, k = 16, 24, 9, 6, 2, 3
    for scoring, scale in (("softmax", 1.0), ("sigmoid", 2.5)):
        cfg = f32shape(T=T, H=H, I=I, E=E, S=S, k=k, scoring=scoring, scale=scale, renorm=False)
        x = rng.standard_normal((T, H)).astype(np.float32)
        wr = rng.standard_normal((E, H)).astype(np.float32)
        g1 = rng.standard_normal((I, H)).astype(np.float32)
        u1 = rng.standard_normal((I, H)).astype(np.float32)
        d1 = rng.standard_normal((H, I)).astype(np.float32)
        gs = rng.standard_normal((S, I, H)).astype(np.float32)
        us = rng.standard_normal((S, I, H)).astype(np.float32)
        ds = rng.standard_normal((S, H, I)).astype(np.float32)
        wg = np.concatenate([np.broadcast_to(g1, (E, I, H)), gs])
        wu = np.concatenate([np.broadcast_to(u1, (E, I, H)), us])
        wd = np.concatenate([np.broadcast_to(d1, (E, H, I)), ds])
        res = oracle.forward(cfg, x, wr, wg, wu, wd)
        ffn = oracle.expert_rows(cfg, x, g1, u1, d1)
        shared = sum(oracle.expert_rows(cfg, x, gs[s], us[s], ds[s]) for s in range(S))
        ref = res["w"].sum(1, keepdims=True) * ffn + shared
        np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(5)
    cfg = f32shape(T=3, H=8, I=8, E=4, S=1, k=2)
    z = np.zeros((3, 8), np.float32)
    w = lambda *s: rng.standard_normal(s).astype(np.float32)
    res = oracle.forward(cfg, z, w(4, 8), w(5, 8, 8), w(5, 8, 8), w(5, 8, 8))
    assert np.all(res["out"] == 0.0)


def test_linear_in_down_and_up_projections():
    rng = np.random.default_rng(6)
    cfg = f32shape(T=5, H=8, I=12, E=4, S=1, k=2, scoring="sigmoid", scale=2.5)
    x = rng.standard_normal((5, 8)).astype(np.float32)
    wr = rng.standard_normal((4, 8)).astype(np.float32)
    wg = rng.standard_normal((5, 12, 8)).astype(np.float32)
    wu = rng.standard_normal((5, 12, 8)).astype(np.float32)
    wd = rng.standard_normal((5, 8, 12)).astype(np.float32)
    base = oracle.forward(cfg, x, wr, wg, wu, wd)["out"]
    np.testing.assert_allclose(oracle.forward(cfg, x, wr, wg, wu, 2 * wd)["out"], 2 * base, rtol=1e-13)
    np.testing.assert_allclose(oracle.forward(cfg, x, wr, wg, -wu, wd)["out"], -base, rtol=1e-13)


def test_empty_slots_are_skipped_and_bf16_inputs_are_exact():
    rng = np.random.default_rng(7)
    cfg = LayerShape("b", T=4, H=8, E=4, S=0, k=2, I=8, dtype="bf16")
    from tests.hostdata import f32_to_bf16_bits, bf16_bits_to_f64
    x = f32_to_bf16_bits(rng.standard_normal((4, 8)))
    wg = f32_to_bf16_bits(rng.standard_normal((4, 8, 8)))
    wu = f32_to_bf16_bits(rng.standard_normal((4, 8, 8)))
    wd = f32_to_bf16_bits(rng.standard_normal((4, 8, 8)))
    idx = np.array([[1, -1], [2, 0], [-1, -1], [3, 1]], np.int32)
    w = np.array([[0.5, 0.0], [0.25, 0.75], [0.0, 0.0], [1.0, 2.0]])
    out = oracle.forward_tokens(cfg, np.arange(4), x, idx, w, lambda e: (wg[e], wu[e], wd[e]))
    xd = bf16_bits_to_f64(x)
    def ffn(e, t):
        g = bf16_bits_to_f64(wg[e]) @ xd[t]
        u = bf16_bits_to_f64(wu[e]) @ xd[t]
        return bf16_bits_to_f64(wd[e]) @ (g / (1 + np.exp(-g)) * u)
    ref = np.stack([0.5 * ffn(1, 0), 0.25 * ffn(2, 1) + 0.75 * ffn(0, 1), np.zeros(8), ffn(3, 3) + 2 * ffn(1, 3)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_combine_over_permuted_rows_equals_token_forward():
    # permute -> per-row experts -> combine must equal the per-token forward
    rng = np.random.default_rng(8)
    cfg = f32shape(T=11, H=8, I=16, E=5, S=2, k=2, scoring="sigmoid", scale=2.5, capacity_factor=0.8)
    x = rng.standard_normal((11, 8)).astype(np.float32)
    wr = rng.standard_normal((5, 8)).astype(np.float32)
    wg = rng.standard_normal((7, 16, 8)).astype(np.float32)
    wu = rng.standard_normal((7, 16, 8)).astype(np.float32)
    wd = rng.standard_normal((7, 8, 16)).astype(np.float32)
    res = oracle.forward(cfg, x, wr, wg, wu, wd)
    assert np.any(res["idx"] < 0)  # capacity dropped something
    counts, offsets, row_token, slot_row = oracle.permute(cfg, res["idx"])
    T = 11
    y = np.zeros((T * cfg.k + cfg.S * T, 8))
    for e in range(cfg.E):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size:
            y[rows] = oracle.expert_rows(cfg, x[row_token[rows]], wg[e], wu[e], wd[e])
    for s in range(cfg.S):
        base = T * cfg.k + s * T
        y[base:base + T] = oracle.expert_rows(cfg, x, wg[cfg.E + s], wu[cfg.E + s], wd[cfg.E + s])
    out = oracle.combine(cfg, y, slot_row, res["w"])
    np.testing.assert_allclose(out, res["out"], rtol=1e-12, atol=1e-12)
