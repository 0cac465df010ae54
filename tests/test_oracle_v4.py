"""Pins of the oracle's V4 routing variants ("15. DeepSeek：MLA、MoE 与 MTP",
section "V4：放弃潜向量，改用压缩注意力", FFN paragraph, and the page's table of
generations): sqrt(softplus) scoring with the selection bias and no group
limit, and hash routing through a fixed token-id -> experts table.

Closed forms come from softplus(log(e^a - 1)) = a, so the scores of such
logits are sqrt(a) and hand-computable gates follow."""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from workloads import LayerShape


def _shape(E, k, scoring="sqrtsoftplus", renorm=True, scale=1.0, G=1, tg=1, cf=0.0, drop=False):
    return LayerShape("t", T=1, H=64, E=E, S=0, k=k, I=64, G=G, topk_group=tg, scoring=scoring,
                      renorm=renorm, scale=scale, capacity_factor=cf, drop_tokens=drop, dtype="f32")


def _logit_of_softplus(a):
    """fp32 logit whose softplus is a (to fp32 rounding of the logit)."""
    return np.float32(math.log(math.expm1(a)))


def _sqsp64(l):
    l = np.asarray(l, dtype=np.float64)
    return np.sqrt(np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l))))


# ---- the fp32 score function ------------------------------------------------------

def test_sqrtsoftplus32_within_2ulp_of_double():
    x = np.concatenate([np.linspace(-80, 80, 400001, dtype=np.float32),
                        np.float32(0.37) * np.arange(-200, 201, dtype=np.float32)])
    x = x[np.abs(x) <= 80]
    v = oracle.sqrtsoftplus32(x).astype(np.float64)
    r = _sqsp64(x)
    ulp = np.spacing(r.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(v - r) / ulp) <= 2.0


def test_sqrtsoftplus32_closed_forms():
    # softplus(0) = ln 2
    assert abs(float(oracle.sqrtsoftplus32(np.zeros(1))[0]) - math.sqrt(math.log(2.0))) <= 1.2e-7
    # softplus(log(e^a - 1)) = a
    for a in (0.25, 1.0, 4.0, 9.0, 30.0):
        l = _logit_of_softplus(a)
        exact = math.sqrt(math.log1p(math.exp(float(l))))
        got = float(oracle.sqrtsoftplus32(np.array([l]))[0])
        assert abs(got - exact) <= 2 * np.spacing(np.float32(exact))
        assert abs(got - math.sqrt(a)) <= 1e-6 * math.sqrt(a)
    # beyond 80 the linear part alone: exactly the fp32 square root of l
    big = np.array([80.0, 81.5, 1e3, 3e7, 1e30], np.float32)
    assert np.array_equal(oracle.sqrtsoftplus32(big), np.sqrt(big))
    # below -80 the value of -80 (the documented clamp), about e^-40
    low = oracle.sqrtsoftplus32(np.array([-80.0, -81.0, -1e4], np.float32))
    assert low[0] == low[1] == low[2]
    assert abs(float(low[0]) - math.exp(-40.0)) <= 1e-6 * math.exp(-40.0)


def test_sqrtsoftplus32_is_monotone_beyond_rounding():
    """Increasing on a grid of steps well above the rounding error; between
    neighbouring fp32 logits a step back of at most one ulp (rounding of the
    sum inside) is all the fp32 evaluation may show."""
    x = np.linspace(-80, 80, 160001, dtype=np.float32)
    v = oracle.sqrtsoftplus32(x)
    assert np.all(np.diff(v[x > -15]) > 0) and np.all(np.diff(v) >= 0)
    x = np.float32(0.5) + np.spacing(np.float32(0.5)) * np.arange(4000, dtype=np.float32)
    v = oracle.sqrtsoftplus32(x)
    assert np.all(np.diff(v) >= -np.spacing(v[1:]))


# ---- learned routing with sqrt(softplus) scores -----------------------------------------

def test_without_bias_selection_is_the_top_k_of_the_logits():
    rng = np.random.default_rng(41)
    shape = _shape(E=256, k=6)
    L = rng.standard_normal((200, 256)).astype(np.float32) * 2
    idx, w, margin, counts = oracle.select(shape, L)
    s = oracle.sqrtsoftplus32(L)
    for t in range(L.shape[0]):
        order = np.argsort(-L[t].astype(np.float64), kind="stable")[:6]
        assert len(np.unique(s[t, order])) == 6  # no fp32 score ties among the chosen
        assert list(idx[t]) == list(order)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=256))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)


def test_gates_closed_form():
    # scores sqrt(9), sqrt(4), sqrt(1) = 3, 2, 1 on experts 5, 2, 7; others lower
    E = 8
    L = np.full((1, E), -3.0, np.float32)
    L[0, 5], L[0, 2], L[0, 7] = _logit_of_softplus(9.0), _logit_of_softplus(4.0), _logit_of_softplus(1.0)
    idx, w, _, _ = oracle.select(_shape(E, 3, scale=1.5), L)
    assert list(idx[0]) == [5, 2, 7]
    np.testing.assert_allclose(w[0], np.array([3.0, 2.0, 1.0]) / 6.0 * 1.5, rtol=1e-6)
    idx, w, _, _ = oracle.select(_shape(E, 3, renorm=False), L)
    np.testing.assert_allclose(w[0], [3.0, 2.0, 1.0], rtol=1e-6)


def test_bias_changes_selection_but_not_gates():
    # unbiased scores 1, 2, 3, 0.5; a bias of 1.6 on expert 0 lifts it above expert 1
    L = np.array([[_logit_of_softplus(1.0), _logit_of_softplus(4.0), _logit_of_softplus(9.0),
                   _logit_of_softplus(0.25)]], np.float32)
    shape = _shape(4, 2)
    idx, w, _, _ = oracle.select(shape, L)
    assert list(idx[0]) == [2, 1]
    np.testing.assert_allclose(w[0], [0.6, 0.4], rtol=1e-6)
    b = np.array([1.6, 0.0, 0.0, 0.0], np.float32)
    idx, w, _, _ = oracle.select(shape, L, b)
    assert list(idx[0]) == [2, 0]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-6)


def test_group_limit_still_applies_when_configured():
    """No group limit is the V4 setting, but the scoring composes with one:
    with two groups and one kept, every choice comes from one group."""
    rng = np.random.default_rng(3)
    L = rng.standard_normal((50, 16)).astype(np.float32)
    idx, _, _, _ = oracle.select(_shape(16, 3, G=2, tg=1), L)
    assert np.all((idx // 8).min(axis=1) == (idx // 8).max(axis=1))


# ---- hash routing -----------------------------------------------------------------

def test_hash_routing_hand_example():
    E, k = 8, 3
    table = np.array([[5, 2, 7],      # id 0
                      [1, 1, 3],      # id 1: repeated entry -> empty slot
                      [9, 0, -4],     # id 2: out-of-range entries -> empty slots
                      [6, 4, 0]], np.int32)
    ids = np.array([0, 1, 2, -1, 4, 3], np.int32)   # -1 and 4 are outside the table
    L = np.full((6, E), -2.0, np.float32)
    L[0, 5], L[0, 2], L[0, 7] = _logit_of_softplus(1.0), _logit_of_softplus(9.0), _logit_of_softplus(4.0)
    L[1, 1], L[1, 3] = _logit_of_softplus(9.0), _logit_of_softplus(1.0)
    L[2, 0] = _logit_of_softplus(0.25)
    L[5, 6], L[5, 4], L[5, 0] = _logit_of_softplus(1.0), _logit_of_softplus(1.0), _logit_of_softplus(4.0)
    shape = _shape(E, k, scale=2.0)
    idx, w, counts = oracle.hash_select(shape, L, ids, table)
    assert idx.tolist() == [[5, 2, 7], [1, -1, 3], [-1, 0, -1], [-1, -1, -1], [-1, -1, -1], [6, 4, 0]]
    # gates keep the table's slot order: sqrt scores renormalised, x 2
    np.testing.assert_allclose(w[0], np.array([1.0, 3.0, 2.0]) / 6.0 * 2.0, rtol=1e-6)
    np.testing.assert_allclose(w[1], np.array([3.0, 0.0, 1.0]) / 4.0 * 2.0, rtol=1e-6)
    np.testing.assert_allclose(w[2], [0.0, 2.0, 0.0], rtol=1e-6)
    assert np.all(w[3:5] == 0.0)
    np.testing.assert_allclose(w[5], np.array([1.0, 1.0, 2.0]) / 4.0 * 2.0, rtol=1e-6)
    assert counts.tolist() == [2, 1, 1, 1, 1, 1, 1, 1]


def test_hash_routing_follows_the_table_whatever_the_logits():
    rng = np.random.default_rng(8)
    E, k, V, T = 64, 6, 1000, 300
    table = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    ids = rng.integers(0, V, T).astype(np.int32)
    shape = _shape(E, k, scale=1.0)
    L1 = rng.standard_normal((T, E)).astype(np.float32)
    L2 = rng.standard_normal((T, E)).astype(np.float32) * 5
    i1, w1, c1 = oracle.hash_select(shape, L1, ids, table)
    i2, w2, c2 = oracle.hash_select(shape, L2, ids, table)
    assert np.array_equal(i1, table[ids]) and np.array_equal(i2, table[ids])
    assert np.array_equal(c1, np.bincount(table[ids].ravel(), minlength=E))
    np.testing.assert_allclose(w1.sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(w1, _sqsp64(np.take_along_axis(L1, table[ids], 1)) /
                               _sqsp64(np.take_along_axis(L1, table[ids], 1)).sum(1, keepdims=True), rtol=1e-6)


def test_hash_routing_softmax_gates_match_library_softmax():
    rng = np.random.default_rng(9)
    E, k, V, T = 32, 4, 50, 40
    table = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    ids = rng.integers(0, V, T).astype(np.int32)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, _ = oracle.hash_select(_shape(E, k, scoring="softmax"), L, ids, table)
    chosen = np.take_along_axis(L.astype(np.float64), table[ids], 1)
    np.testing.assert_allclose(w, softmax(chosen, axis=1), rtol=1e-12)
    idx, w, _ = oracle.hash_select(_shape(E, k, scoring="softmax", renorm=False), L, ids, table)
    full = softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, table[ids], 1), rtol=1e-12)


def test_hash_routing_drop_mode_keeps_the_first_c_assignments():
    rng = np.random.default_rng(10)
    E, k, V, T = 16, 2, 20, 97
    table = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    table[:5] = [3, 7]                              # a hot pair of experts
    ids = rng.integers(0, V, T).astype(np.int32)
    shape = _shape(E, k, cf=0.75, drop=True).with_(T=T)
    C = oracle.capacity(shape, T)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, counts = oracle.hash_select(shape, L, ids, table)
    _, w_free, _ = oracle.hash_select(_shape(E, k), L, ids, table)
    want = table[ids].copy()
    # brute force: walk the (token, slot) pairs in order, count per expert
    seen = {}
    for t in range(T):
        for j in range(k):
            e = int(want[t, j])
            seen[e] = seen.get(e, 0) + 1
            if seen[e] > C:
                want[t, j] = -1
    assert np.array_equal(idx, want)
    assert counts.max() <= C and (idx < 0).any()
    np.testing.assert_allclose(w, np.where(want >= 0, w_free, 0.0), rtol=0, atol=0)


def test_hash_routing_rejects_a_re_route_capacity():
    table = np.zeros((4, 2), np.int32)
    table[:, 1] = 1
    with pytest.raises(ValueError):
        oracle.hash_select(_shape(4, 2, cf=1.0).with_(T=3), np.zeros((3, 4), np.float32),
                           np.zeros(3, np.int32), table)
