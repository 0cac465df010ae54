"""Pins of the oracle's routing: scoring, group-limited top-k, gates, capacity.

Sources: "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个"
(sigmoid scores, selection-only bias, group score = sum of the two best biased
scores in a group, best groups kept, top-k among them, gates = unbiased scores
renormalised x routed_scaling_factor); "MoE架构揭秘", section 3.1 (softmax then
top-k); "GPT-4 Has 1.8 Trillion Parameters. It Uses 2% of Them Per Token",
section 2.2 (capacity, overflow to the next-best expert) and its MoEBlock
sketch (softmax over the top-k logits).

Nothing here re-types the oracle: selection is checked by hand-built vectors
with hand-derived answers, by exhaustive subset enumeration with exact
rational sums (a different characterisation of "top-k with lower-index
tie-break"), and by reductions to library sorts / softmax.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from workloads import LayerShape

LN3 = math.log(3.0)


def shape(**kw):
    base = dict(name="t", T=1, H=8, E=16, S=0, k=2, I=8)
    base.update(kw)
    return LayerShape(**base)


# ---- hand-built vectors ------------------------------------------------------

def test_group_whose_best_expert_is_global_max_but_pair_sum_loses_is_dropped():
    # 16 experts, 4 groups of 4, keep 2 groups, pick 2 experts, sigmoid scores.
    cfg = shape(E=16, G=4, topk_group=2, k=2, scoring="sigmoid", renorm=True, scale=2.5)
    logits = np.array([[5, -5, -5, -5,      # group 0: global max, pair sum ~1.0
                        2, 2, -3, -3,       # group 1: pair sum ~1.76
                        1.5, 1.5, -3, -3,   # group 2: pair sum ~1.64
                        -1, -1, -1, -1]],   # group 3: pair sum ~0.54
                      dtype=np.float32)
    idx, w, margin, counts = oracle.select(cfg, logits, np.zeros(16, np.float32))
    assert idx.tolist() == [[4, 5]]          # equal scores -> lower index first
    np.testing.assert_allclose(w, [[1.25, 1.25]], rtol=1e-15)
    # without the group limit the global maximum wins
    cfg1 = cfg.with_(G=1, topk_group=1)
    idx1, _, _, _ = oracle.select(cfg1, logits, np.zeros(16, np.float32))
    assert idx1.tolist() == [[0, 4]]


def test_bias_changes_selection_but_not_gates():
    # all logits 0 -> every sigmoid score is exactly 1/2; the bias alone ranks
    cfg = shape(E=8, k=3, scoring="sigmoid", renorm=True, scale=2.5)
    bias = np.array([0, 0.2, 0, 0.3, 0, 0, 0, 0.3], np.float32)
    idx, w, _, _ = oracle.select(cfg, np.zeros((1, 8), np.float32), bias)
    assert idx.tolist() == [[3, 7, 1]]
    np.testing.assert_allclose(w, [[2.5 / 3] * 3], rtol=1e-15)


def test_sigmoid_gates_closed_form():
    # chosen logits ln3, 0, -ln3 -> scores 3/4, 1/2, 1/4 (sum 3/2)
    cfg = shape(E=4, k=3, scoring="sigmoid", renorm=True, scale=2.5)
    logits = np.array([[0.0, -LN3, -9.0, LN3]], np.float32)
    idx, w, _, _ = oracle.select(cfg, logits, None)
    assert idx.tolist() == [[3, 0, 1]]
    np.testing.assert_allclose(w, [[2.5 * 0.5, 2.5 / 3, 2.5 / 6]], rtol=1e-7)
    # without renormalisation the gates are the scaled scores themselves
    _, w2, _, _ = oracle.select(cfg.with_(renorm=False, scale=1.0), logits, None)
    np.testing.assert_allclose(w2, [[0.75, 0.5, 0.25]], rtol=1e-7)


def test_softmax_gates_closed_form():
    # logits ln3, 0 over 4 experts: softmax over all = 3/(3+1+e^-9+e^-9) etc.
    cfg = shape(E=4, k=2, scoring="softmax", renorm=True)
    logits = np.array([[0.0, -9.0, -9.0, LN3]], np.float32)
    idx, w, _, _ = oracle.select(cfg, logits, None)
    assert idx.tolist() == [[3, 0]]
    np.testing.assert_allclose(w, [[0.75, 0.25]], rtol=1e-7)
    _, w2, _, _ = oracle.select(cfg.with_(renorm=False), logits, None)
    z = 3.0 + 1.0 + 2 * math.exp(-9.0)
    np.testing.assert_allclose(w2, [[3.0 / z, 1.0 / z]], rtol=1e-7)


def test_ties_go_to_lower_index():
    cfg = shape(E=6, k=3)
    idx, _, margin, _ = oracle.select(cfg, np.ones((1, 6), np.float32), None)
    assert idx.tolist() == [[0, 1, 2]]
    assert margin[0] == 0.0


def test_zero_input_selects_lowest_indices_softmax_and_bias_order_sigmoid():
    cfg = shape(E=8, k=2)
    idx, w, _, _ = oracle.select(cfg, np.zeros((3, 8), np.float32), None)
    assert idx.tolist() == [[0, 1]] * 3
    np.testing.assert_allclose(w, 0.5)
    cfg2 = shape(E=8, k=2, scoring="sigmoid", scale=2.5)
    bias = np.array([0.01, -0.02, 0.03, 0.0, 0.05, 0.0, 0.0, 0.0], np.float32)
    idx2, w2, _, _ = oracle.select(cfg2, np.zeros((1, 8), np.float32), bias)
    assert idx2.tolist() == [[4, 2]]
    np.testing.assert_allclose(w2, 1.25)


# ---- exhaustive enumeration with exact sums ---------------------------------

def _brute_select(logits_row, bias, E, G, keep, k, scoring):
    """Lexicographically smallest index set maximising the exact sum, first
    over groups (group score = max pair sum, fp32-rounded as the page's
    `topk(2).values.sum` is an fp32 sum), then over experts of kept groups."""
    if scoring == "sigmoid":
        s = oracle.sigmoid32(logits_row)
        c = (s + bias).astype(np.float32)
    else:
        c = logits_row.astype(np.float32)
    allowed = list(range(E))
    if G > 1:
        gsz = E // G
        gs = []
        for g in range(G):
            members = range(g * gsz, (g + 1) * gsz)
            gs.append(max(np.float32(c[a]) + np.float32(c[b]) for a, b in itertools.combinations(members, 2)))
        best = None
        for sub in itertools.combinations(range(G), keep):  # combinations come in lexicographic order
            tot = sum(Fraction(float(gs[g])) for g in sub)
            if best is None or tot > best[0]:
                best = (tot, sub)
        allowed = [e for e in range(E) if e // gsz in best[1]]
    best = None
    for sub in itertools.combinations(allowed, k):
        tot = sum(Fraction(float(c[e])) for e in sub)
        if best is None or tot > best[0]:
            best = (tot, sub)
    return set(best[1])


@pytest.mark.parametrize("E,G,keep,k,scoring", [
    (16, 4, 2, 3, "sigmoid"),
    (12, 3, 2, 4, "sigmoid"),
    (16, 8, 3, 2, "sigmoid"),
    (10, 1, 1, 3, "softmax"),
    (8, 2, 1, 2, "softmax"),
])
def test_selection_matches_exhaustive_enumeration(E, G, keep, k, scoring):
    rng = np.random.default_rng(E * 100 + G * 10 + k)
    cfg = shape(E=E, G=G, topk_group=keep, k=k, scoring=scoring, scale=2.5 if scoring == "sigmoid" else 1.0)
    T = 300
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # force ties: quantise a third of the rows to a few levels
    logits[: T // 3] = np.round(logits[: T // 3] * 2) / 2
    bias = (rng.uniform(-0.05, 0.05, E).astype(np.float32) if scoring == "sigmoid" else None)
    if bias is not None:
        bias[: E // 2] = np.round(bias[: E // 2] * 40) / 40
    idx, w, _, _ = oracle.select(cfg, logits, bias)
    b = bias if bias is not None else np.zeros(E, np.float32)
    for t in range(T):
        assert set(idx[t].tolist()) == _brute_select(logits[t], b, E, G, keep, k, scoring), t
        # rank order: scores non-increasing
        c = (oracle.sigmoid32(logits[t]) + b).astype(np.float32) if scoring == "sigmoid" else logits[t]
        cs = c[idx[t]]
        assert np.all(cs[:-1] >= cs[1:])


# ---- reductions to library routines ----------------------------------------

def test_plain_topk_equals_stable_argsort():
    rng = np.random.default_rng(5)
    cfg = shape(E=64, k=6)
    logits = (rng.integers(-20, 20, size=(500, 64)) / 4).astype(np.float32)  # many ties
    idx, _, _, _ = oracle.select(cfg, logits, None)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert np.array_equal(idx, ref)


def test_sigmoid_without_bias_selects_like_logits():
    rng = np.random.default_rng(6)
    cfg_s = shape(E=32, k=4, scoring="sigmoid")
    cfg_l = shape(E=32, k=4, scoring="softmax")
    logits = rng.uniform(-4, 4, (400, 32)).astype(np.float32)
    a, _, _, _ = oracle.select(cfg_s, logits, None)
    b, _, _, _ = oracle.select(cfg_l, logits, None)
    assert np.array_equal(a, b)


def test_softmax_gates_match_library_softmax():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((200, 8)).astype(np.float32) * 2
    cfg = shape(E=8, k=2, renorm=True)
    idx, w, _, _ = oracle.select(cfg, logits, None)
    sel = np.take_along_axis(logits.astype(np.float64), idx, axis=1)
    np.testing.assert_allclose(w, sp_softmax(sel, axis=1), rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
    cfg2 = shape(E=8, k=2, renorm=False)
    idx2, w2, _, _ = oracle.select(cfg2, logits, None)
    full = sp_softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w2, np.take_along_axis(full, idx2, axis=1), rtol=1e-13)
    assert np.all(w2.sum(1) < 1.0)


def test_v3_gates_sum_to_scaling_factor():
    rng = np.random.default_rng(8)
    cfg = shape(E=256, G=8, topk_group=4, k=8, scoring="sigmoid", scale=2.5)
    logits = rng.standard_normal((100, 256)).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, 256).astype(np.float32)
    idx, w, margin, counts = oracle.select(cfg, logits, bias)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-13)
    # every chosen expert lies in one of at most 4 groups
    assert max(len(set((idx[t] // 32).tolist())) for t in range(100)) <= 4
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=256))
    assert np.all(margin >= 0)


# ---- capacity ---------------------------------------------------------------

def _brute_capacity(logits, bias, cfg):
    """Sequential simulation written from the capacity sentence: tokens in
    order; each takes, among allowed experts that still have room, the
    lexicographically smallest k-set of maximal exact score sum (fewer when
    fewer have room)."""
    T, E = logits.shape
    C = math.ceil(cfg.capacity_factor * T * cfg.k / E)
    load = [0] * E
    out = []
    for t in range(T):
        if cfg.scoring == "sigmoid":
            c = (oracle.sigmoid32(logits[t]) + bias).astype(np.float32)
        else:
            c = logits[t]
        allowed = list(range(E))
        if cfg.G > 1:
            # group choice does not depend on load
            gsz = E // cfg.G
            gs = [max(np.float32(c[a]) + np.float32(c[b])
                      for a, b in itertools.combinations(range(g * gsz, (g + 1) * gsz), 2)) for g in range(cfg.G)]
            best = None
            for sub in itertools.combinations(range(cfg.G), cfg.topk_group):
                tot = sum(Fraction(float(gs[g])) for g in sub)
                if best is None or tot > best[0]:
                    best = (tot, sub)
            allowed = [e for e in range(E) if e // gsz in best[1]]
        room = [e for e in allowed if load[e] < C]
        kk = min(cfg.k, len(room))
        best = None
        for sub in itertools.combinations(room, kk):
            tot = sum(Fraction(float(c[e])) for e in sub)
            if best is None or tot > best[0]:
                best = (tot, sub)
        chosen = set(best[1]) if best else set()
        for e in chosen:
            load[e] += 1
        out.append(chosen)
    return out, C


@pytest.mark.parametrize("E,G,keep,k,cf,scoring", [
    (8, 1, 1, 2, 1.0, "softmax"),
    (12, 3, 2, 3, 1.25, "sigmoid"),
    (16, 4, 2, 3, 0.75, "sigmoid"),
])
def test_capacity_matches_sequential_simulation(E, G, keep, k, cf, scoring):
    rng = np.random.default_rng(E + k)
    T = 40
    cfg = shape(T=T, E=E, G=G, topk_group=keep, k=k, capacity_factor=cf, scoring=scoring,
                scale=2.5 if scoring == "sigmoid" else 1.0)
    # skewed load so that experts fill up
    logits = (rng.standard_normal((T, E)) + np.linspace(2, -2, E)).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if scoring == "sigmoid" else np.zeros(E, np.float32)
    idx, w, _, counts = oracle.select(cfg, logits, bias if scoring == "sigmoid" else None)
    ref, C = _brute_capacity(logits, bias, cfg)
    assert oracle.capacity(cfg, T) == C
    assert counts.max() <= C
    for t in range(T):
        got = set(int(e) for e in idx[t] if e >= 0)
        assert got == ref[t], t
        # empty slots come last and carry zero gate
        n = len(got)
        assert np.all(idx[t, n:] == -1) and np.all(w[t, n:] == 0.0)
        if n:
            tot = 2.5 if scoring == "sigmoid" else 1.0
            np.testing.assert_allclose(w[t, :n].sum(), tot, rtol=1e-13)


@pytest.mark.parametrize("cf", ["1.0", "1.2", "1.25", "0.3", "2.0"])
def test_capacity_value_is_the_decimal_ceiling_for_the_pages_factors(cf):
    """C = ceil(cf * T * k / E) with cf the decimal the configuration states
    (capacity_factor: 1.2 in the GPT-4 page's config block, 1.25 at the
    decode workload), checked with exact rational arithmetic over every T up
    to 3000 at the workloads' (k, E).  The oracle (and the library) evaluate
    ((cf*T)*k)/E in IEEE double on the double nearest the decimal; for these
    factors that never crosses an integer the exact value does not."""
    q = Fraction(cf)
    for k, E in ((2, 8), (6, 160), (8, 256)):
        for T in range(1, 3001):
            want = math.ceil(q * T * k / E)
            assert oracle.capacity(shape(T=T, E=E, k=k, capacity_factor=float(cf)), T) == want, (cf, T, k, E)


def test_capacity_of_a_factor_stored_above_its_decimal():
    """The reading's one visible edge: 1.1 is stored as a double slightly
    above 1.1, so where 1.1 * T * k / E is an integer in decimal the IEEE
    double evaluation lands just above it and C is one more (T = 200, k = 2,
    E = 8: decimal 55, double 56).  Both sides of the build use the double
    value, so they agree with each other."""
    assert math.ceil(Fraction("1.1") * 200 * 2 / 8) == 55
    assert Fraction(1.1) > Fraction("1.1")
    assert oracle.capacity(shape(T=200, E=8, k=2, capacity_factor=1.1), 200) == 56
    assert oracle.capacity(shape(T=320, E=256, k=8, capacity_factor=1.1), 320) == 11


def test_capacity_defining_property_v3_decode_shape():
    """At the decode workload's routing shape: every expert that ranks above a
    chosen one (or above an empty slot) but was not chosen was full when the
    token was served."""
    from workloads import CONFIGS, zipf_logit_offsets
    cfg = CONFIGS["deepseek_v3_decode"]
    rng = np.random.default_rng(9)
    T, E = cfg.T, cfg.E
    logits = (rng.standard_normal((T, E)) + zipf_logit_offsets(E, 1.1, cfg.seed)).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, w, _, counts = oracle.select(cfg, logits, bias)
    C = oracle.capacity(cfg, T)
    assert C == 5
    assert counts.max() <= C
    # unlimited selection gives each token's ranking among its kept groups
    free_cfg = cfg.with_(capacity_factor=0.0, k=E // cfg.G * cfg.topk_group)
    rank, _, _, _ = oracle.select(free_cfg, logits, bias)
    load = np.zeros(E, int)
    for t in range(T):
        chosen = [int(e) for e in idx[t] if e >= 0]
        last = rank[t].tolist().index(chosen[-1]) if len(chosen) == cfg.k else len(rank[t]) - 1
        for e in rank[t][: last + 1]:
            if e not in chosen:
                assert load[e] >= C
        for e in chosen:
            load[e] += 1
    assert np.array_equal(load, counts)


# ---- capacity, drop mode ---------------------------------------------------------
# The serving configuration of "GPT-4 Has 1.8 Trillion Parameters. It Uses 2%
# of Them Per Token" (section 4.2, drop_tokens): an assignment beyond an
# expert's capacity is dropped instead of going to another expert.

def test_drop_mode_hand_example():
    # 4 experts, top-2, softmax; C = ceil(0.5 * 3 * 2 / 4) = 1
    cfg = shape(T=3, E=4, k=2, capacity_factor=0.5, drop_tokens=True)
    assert oracle.capacity(cfg, 3) == 1
    logits = np.array([[3, 2, 0, -1],     # top-2 {0, 1}: both kept
                       [3, -1, 2, 0],     # top-2 {0, 2}: 0 is full -> dropped, 2 kept
                       [-1, 3, 2, 0]],    # top-2 {1, 2}: both full -> both dropped
                      np.float32)
    idx, w, _, counts = oracle.select(cfg, logits, None)
    assert idx.tolist() == [[0, 1], [-1, 2], [-1, -1]]
    assert counts.tolist() == [1, 1, 1, 0]
    # kept gates are those of the full top-2 (renormalised softmax over the pair)
    e2 = math.exp(2.0) / (math.exp(3.0) + math.exp(2.0))
    np.testing.assert_allclose(w, [[1 - e2, e2], [0.0, e2], [0.0, 0.0]], rtol=1e-12)
    # re-route mode on the same logits sends the overflow to the next-best expert
    idx_r, _, _, _ = oracle.select(cfg.with_(drop_tokens=False), logits, None)
    assert idx_r.tolist() == [[0, 1], [2, 3], [-1, -1]]


@pytest.mark.parametrize("E,G,keep,k,cf,scoring", [
    (8, 1, 1, 2, 0.75, "softmax"),
    (16, 4, 2, 3, 1.0, "sigmoid"),
    (256, 8, 4, 8, 1.25, "sigmoid"),
])
def test_drop_mode_is_the_unlimited_top_k_minus_late_assignments(E, G, keep, k, cf, scoring):
    """Defining property, by prefix counts instead of a running counter: an
    assignment (t, e) of the unlimited top-k survives iff fewer than C earlier
    tokens chose e; survivors keep their unlimited gates, the rest are -1/0."""
    rng = np.random.default_rng(E * k)
    T = 128
    cfg = shape(T=T, E=E, G=G, topk_group=keep, k=k, capacity_factor=cf, scoring=scoring, drop_tokens=True,
                scale=2.5 if scoring == "sigmoid" else 1.0)
    logits = (rng.standard_normal((T, E)) + np.linspace(2, -2, E)).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32) if scoring == "sigmoid" else None
    idx, w, _, counts = oracle.select(cfg, logits, bias)
    free_idx, free_w, _, _ = oracle.select(cfg.with_(capacity_factor=0.0, drop_tokens=False), logits, bias)
    C = oracle.capacity(cfg, T)
    onehot = np.zeros((T, E), int)
    for t in range(T):
        onehot[t, free_idx[t]] = 1
    earlier = np.cumsum(onehot, axis=0) - onehot          # selections of e by tokens before t
    for t in range(T):
        for j in range(k):
            e = free_idx[t, j]
            if earlier[t, e] < C:
                assert idx[t, j] == e and w[t, j] == free_w[t, j]
            else:
                assert idx[t, j] == -1 and w[t, j] == 0.0
    assert np.array_equal(counts, np.minimum(onehot.sum(0), C))


def test_drop_mode_with_room_for_everyone_is_unlimited_routing():
    rng = np.random.default_rng(3)
    T, E = 64, 16
    cfg = shape(T=T, E=E, G=4, topk_group=2, k=4, scoring="sigmoid", scale=2.5, capacity_factor=8.0,
                drop_tokens=True)
    assert oracle.capacity(cfg, T) >= T
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    a = oracle.select(cfg, logits, bias)
    b = oracle.select(cfg.with_(capacity_factor=0.0, drop_tokens=False), logits, bias)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_margin_of_hand_built_vector():
    # kept groups 1 and 2; group margin = GS(2) - GS(0), expert margin = s(2) - s(1.5)
    cfg = shape(E=16, G=4, topk_group=2, k=2, scoring="sigmoid", renorm=True, scale=2.5)
    logits = np.array([[5, -5, -5, -5, 2, 2, -3, -3, 1.5, 1.5, -3, -3, -1, -1, -1, -1]], np.float32)
    _, _, margin, _ = oracle.select(cfg, logits, np.zeros(16, np.float32))
    sg = lambda v: 1.0 / (1.0 + math.exp(-v))
    group_margin = 2 * sg(1.5) - (sg(5) + sg(-5))
    expert_margin = sg(2) - sg(1.5)
    np.testing.assert_allclose(margin[0], min(group_margin, expert_margin), atol=1e-6)


def test_router_logits_are_the_fp32_rounded_matmul_plus_bias():
    from tests.hostdata import f32_to_bf16_bits, bf16_bits_to_f64
    rng = np.random.default_rng(10)
    cfg = shape(T=33, H=96, E=12, k=2)
    x = f32_to_bf16_bits(rng.standard_normal((33, 96)))
    w = f32_to_bf16_bits(rng.standard_normal((12, 96)) / np.sqrt(96))
    b = rng.standard_normal(12).astype(np.float32)
    got = oracle.router_logits(cfg.with_(dtype="bf16"), x, w, b)
    ref = bf16_bits_to_f64(x) @ bf16_bits_to_f64(w).T + b.astype(np.float64)
    # one rounding to fp32 of the exact value (double sums of bf16 products of
    # this size are exact to far below fp32 resolution)
    assert np.array_equal(got, ref.astype(np.float32)) or np.max(
        np.abs(got - ref) / np.spacing(np.abs(ref).astype(np.float32))) <= 0.5 + 1e-6
    got_nb = oracle.router_logits(cfg.with_(dtype="bf16"), x, w, None)
    np.testing.assert_allclose(got - got_nb, np.broadcast_to(b, got.shape), atol=1e-5)
