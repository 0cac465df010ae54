"""Pins of the parameter arithmetic and of the workload shapes against the
figures the DeepSeek page prints (golden files under tests/golden/ carry the
citations)."""
import json
import os

import oracle
from workloads import CONFIGS

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_v3_per_module_counts():
    g = load("deepseek_param_counts.json")["v3"]
    H, E, S, I, k = g["hidden"], g["routed_experts"], g["shared_experts"], g["moe_intermediate"], g["top_k"]
    layer = oracle.moe_layer_params(H, E, S, I)
    assert layer - oracle.moe_layer_params(H, E, S, 0) == (E + S) * g["per_expert"]
    assert oracle.moe_layer_params(H, E, 0, 0) == g["router"]
    assert oracle.moe_layer_params(H, 0, 1, I) == g["per_expert"]


def test_v3_totals_reproduce_exactly():
    g = load("deepseek_param_counts.json")["v3"]
    H, E, S, I, k = g["hidden"], g["routed_experts"], g["shared_experts"], g["moe_intermediate"], g["top_k"]
    norms = (2 * g["layers"] + 1) * H  # derived reading, see the golden file
    rest = (g["layers"] * g["per_layer_attention"] + g["dense_layers"] * g["dense_ffn"]
            + g["embedding"] + g["output_head"] + norms)
    total = rest + g["moe_layers"] * oracle.moe_layer_params(H, E, S, I)
    active = rest + g["moe_layers"] * oracle.moe_active_params(H, E, S, k, I)
    assert total == g["total"]
    assert active == g["active"]
    routed_share = g["moe_layers"] * E * g["per_expert"] / total
    assert round(100 * routed_share, 1) == g["routed_share_percent_printed"]


def test_workload_shapes_follow_the_spec_table():
    t = load("deepseek_spec_table.json")
    for cfg_name, gen in (("deepseek_v2", "V2"), ("deepseek_v3_prefill", "V3"), ("deepseek_v3_decode", "V3")):
        c, r = CONFIGS[cfg_name], t[gen]
        assert (c.E, c.S, c.k, c.H, c.I, c.scoring) == (r["routed"], r["shared"], r["top_k"], r["hidden"],
                                                          r["moe_intermediate"], r["scoring"])
    v3 = CONFIGS["deepseek_v3_prefill"]
    assert (v3.G, v3.topk_group, v3.scale, v3.renorm) == (8, 4, 2.5, True)
