"""Pins of the oracle's auxiliary-loss-free balancing step and load telemetry.

Source: "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8
个" (per step, an overloaded expert's bias is lowered by gamma and an idle one's
raised; gamma = 0.001; monitor each expert's token share and the bias drift);
"GPT-4稀疏激活原理：2%参数调用背后的MoE工程实践", section 4.4
(the entropy of the expert calls as a health signal).
"""
import math

import numpy as np
from scipy.stats import entropy as sp_entropy

import oracle


def test_uniform_load_changes_nothing_and_has_maximal_entropy():
    E = 256
    b0 = np.linspace(-0.05, 0.05, E, dtype=np.float32)
    b, share, st = oracle.balance_update(np.full(E, 512), b0, 0.001)
    assert np.array_equal(b, b0)
    assert np.all(share == 1.0 / E)
    np.testing.assert_allclose(st["entropy"], math.log(E), rtol=1e-14)
    assert st["max_share"] == 1.0 / E and st["over"] == 0 and st["under"] == 0


def test_single_hot_expert():
    E = 8
    counts = np.zeros(E, int)
    counts[5] = 100
    b0 = np.zeros(E, np.float32)
    b, share, st = oracle.balance_update(counts, b0, 0.001)
    g = np.float32(0.001)
    assert b[5] == -g and np.all(np.delete(b, 5) == g)
    assert st["entropy"] == 0.0 and st["max_share"] == 1.0 and st["over"] == 1 and st["under"] == 7


def test_loads_at_the_mean_keep_their_bias():
    counts = np.array([2, 2, 1, 3])           # mean 2
    b0 = np.array([0.1, -0.1, 0.0, 0.02], np.float32)
    b, _, st = oracle.balance_update(counts, b0, 0.001)
    g = np.float32(0.001)
    assert b[0] == b0[0] and b[1] == b0[1]
    assert b[2] == np.float32(b0[2] + g) and b[3] == np.float32(b0[3] - g)
    assert st["over"] == 1 and st["under"] == 1


def test_random_loads_against_library_entropy_and_float32_steps():
    rng = np.random.default_rng(4)
    E = 160
    counts = rng.poisson(300, E)
    counts[:5] = 0                            # idle experts: 0 * ln 0 = 0
    b0 = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    b, share, st = oracle.balance_update(counts, b0, 0.001)
    N = counts.sum()
    np.testing.assert_allclose(share, counts / N, rtol=1e-15)
    np.testing.assert_allclose(st["entropy"], sp_entropy(counts / N), rtol=1e-12)
    mean = N / E
    g = np.float32(0.001)
    want = np.where(counts > mean, b0 - g, np.where(counts < mean, b0 + g, b0)).astype(np.float32)
    assert np.array_equal(b, want)
    assert st["over"] == int((counts > mean).sum()) and st["under"] == int((counts < mean).sum())


def test_repeated_steps_drift_toward_balance():
    """A fixed skewed load drives the hot expert's bias down and the cold ones'
    up by gamma per step: the drift the monitoring paragraph watches for."""
    E = 4
    counts = np.array([40, 10, 10, 20])       # mean 20: expert 3 sits at it
    b = np.zeros(E, np.float32)
    for _ in range(100):
        b, _, _ = oracle.balance_update(counts, b, 0.001)
    np.testing.assert_allclose(b, [-0.1, 0.1, 0.1, 0.0], atol=1e-5)


def test_empty_step():
    b0 = np.array([0.5, -0.5], np.float32)
    b, share, st = oracle.balance_update(np.zeros(2, int), b0, 0.001)
    assert np.array_equal(b, b0) and np.all(share == 0.0) and st["entropy"] == 0.0
