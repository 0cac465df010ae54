"""Pins of the oracle's fp32 exp/sigmoid used for bit-reproducible selection.

The fp32 sigmoid is this build's reading of the sigmoid score in the V3 router
("15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个"):
the page fixes sigmoid(x @ W.T) but no precision, so selection uses a sigmoid
made of correctly rounded fp32 operations.  It is pinned here against the
mathematical function evaluated in double by the C library, and by closed-form
points and invariants.
"""
import math

import numpy as np
import pytest

import oracle


def ulp32(v):
    v = np.abs(np.asarray(v, dtype=np.float32))
    return np.spacing(v).astype(np.float64)


def test_exp32_within_2ulp_of_double_exp():
    rng = np.random.default_rng(11)
    z = np.concatenate([
        -np.linspace(0.0, 80.0, 1_000_001, dtype=np.float64),
        -rng.uniform(0.0, 80.0, 1_000_000),
        -rng.uniform(0.0, 1e-3, 100_000),
        np.array([0.0, -0.0, -0.34657359, -0.34657360, -0.6931472, -80.0]),
    ]).astype(np.float32)
    got = oracle.exp32(z).astype(np.float64)
    ref = np.exp(z.astype(np.float64))
    err = np.abs(got - ref) / ulp32(ref.astype(np.float32))
    # degree-7 Taylor remainder on |r| <= ln2/2 is < 0.1 ulp; the Horner
    # roundings and the reduction add well under one more ulp
    assert err.max() <= 1.0, err.max()


def test_sigmoid32_within_2ulp_of_double_sigmoid():
    rng = np.random.default_rng(12)
    l = np.concatenate([
        np.linspace(-80.0, 80.0, 2_000_001, dtype=np.float64),
        rng.standard_normal(2_000_000) * 3.0,
        rng.uniform(-1e-4, 1e-4, 100_000),
    ]).astype(np.float32)
    got = oracle.sigmoid32(l).astype(np.float64)
    ld = l.astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-ld))
    err = np.abs(got - ref) / ulp32(ref.astype(np.float32))
    # exp32 (<= 1 ulp) followed by two correctly rounded operations (1 + e and
    # the division), each <= 1/2 ulp of its own result: <= 2.5 ulp of sigma
    assert err.max() <= 2.5, err.max()


def test_sigmoid32_closed_forms():
    assert oracle.sigmoid32(np.float32([0.0]))[0] == np.float32(0.5)
    assert oracle.sigmoid32(np.float32([-0.0]))[0] == np.float32(0.5)
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 (ln 3 rounded to fp32)
    l3 = np.float32(math.log(3.0))
    v = oracle.sigmoid32(np.float32([l3, -l3])).astype(np.float64)
    d = 1.0 / (3.0 + 1.0) ** 2 * 3.0  # derivative of sigmoid at ln 3
    slack = abs(float(l3) - math.log(3.0)) * d + 1e-7
    assert abs(v[0] - 0.75) <= slack and abs(v[1] - 0.25) <= slack
    # saturation: the clamp makes every logit beyond +-80 equal to the value at +-80
    big = oracle.sigmoid32(np.float32([80.0, 100.0, 1e30, -80.0, -100.0, -1e30]))
    assert big[0] == big[1] == big[2] == np.float32(1.0)
    assert big[3] == big[4] == big[5]
    assert 0.0 < big[3] < 1e-34  # a normal fp32 number near e^-80


def test_sigmoid32_is_monotone_and_symmetric():
    l = np.linspace(-20.0, 20.0, 400_001, dtype=np.float32)
    s = oracle.sigmoid32(l)
    assert np.all(np.diff(s.astype(np.float64)) >= 0.0)
    sp = oracle.sigmoid32(l).astype(np.float64)
    sn = oracle.sigmoid32(-l).astype(np.float64)
    assert np.max(np.abs(sp + sn - 1.0)) <= 2.5 * 2.0 ** -24 * 2


def test_sigmoid32_scalar_matches_array():
    for v in (-3.25, -1e-3, 0.0, 0.7, 12.0):
        a = oracle.sigmoid32(np.float32([v]))[0]
        b = oracle._load().oracle_sigmoid32(np.float32(v))
        assert np.float32(b) == a


@pytest.mark.parametrize("z", [0.0, -1.0, -10.0, -50.0])
def test_exp32_closed_forms(z):
    got = float(oracle.exp32(np.float32([z]))[0])
    assert abs(got - math.exp(z)) <= 2 * float(np.spacing(np.float32(math.exp(z))))
