"""Whole-layer parity on seeded random layer configurations.

The fixed shapes of test_gpu_parity follow the pages' layers; these cases
draw the configuration itself at random (expert count, groups and groups
kept, top-k, shared experts, scoring, renormalisation and scaling, capacity
and drop mode, batch size, widths, input and output precision) from a fixed
seed, so combinations no named layer uses -- softmax with a group limit, a
capacity on a softmax layer, FP8 experts without a shared one, odd batch
sizes against every tile height -- meet the same bars: routing bit-exact on
identical logits, outputs within the per-precision tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import check_layer, run_layer
from workloads import make_inputs
from workloads.configs import LayerShape

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    dtype = rng.choice(["bf16", "bf16", "bf16", "f32", "fp8"])
    if dtype == "f32":
        H, I = 32 * int(rng.integers(4, 13)), 32 * int(rng.integers(2, 11))
    else:
        H, I = 256 * int(rng.integers(1, 3)), 128 * int(rng.integers(1, 4))
    E = int(rng.integers(2, 97))
    divisors = [g for g in range(2, min(E, 32) + 1) if E % g == 0 and E // g >= 2]
    G = int(rng.choice(divisors)) if divisors and rng.random() < 0.5 else 1
    topk_group = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(32, topk_group * (E // G)) + 1))
    scoring = str(rng.choice(["softmax", "sigmoid", "sqrtsoftplus"]))
    cf, drop = 0.0, False
    if rng.random() < 0.4:
        cf = float(rng.choice([0.5, 1.0, 1.25, 2.0]))
        drop = bool(rng.random() < 0.5)
    shape = LayerShape("random_%d" % i, T=int(rng.integers(1, 301)), H=H, E=E, S=int(rng.integers(0, 3)), k=k,
                       I=I, G=G, topk_group=topk_group, scoring=scoring, renorm=bool(rng.random() < 0.7),
                       scale=float(rng.choice([1.0, 2.5])), capacity_factor=cf, drop_tokens=drop, dtype=str(dtype),
                       sel_bias=0.05 if scoring != "softmax" and rng.random() < 0.7 else None,
                       zipf_s=1.1 if rng.random() < 0.3 else None, seed=7000 + i)
    out_dtype = "f32" if dtype == "f32" or rng.random() < 0.3 else "bf16"
    return shape, out_dtype


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_config(i):
    shape, out_dtype = _draw(i)
    print("case %d: %s out=%s" % (i, shape, out_dtype), flush=True)
    inp = make_inputs(shape, device="cuda")
    g = run_layer(shape, inp, out_dtype)
    err, excluded = check_layer(shape, inp, g, np.arange(shape.T), out_dtype)
    print("case %d: max err %.3g x RMS, %d near-tie tokens compared on the GPU's selection" % (i, err, excluded))
    del inp
    torch.cuda.empty_cache()
