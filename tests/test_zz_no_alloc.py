"""moe_forward_noalloc: the whole layer on the library's static device scratch
(no workspace argument, nothing allocated), against moe_forward with a
caller workspace on the same inputs.  Both run the same kernels, so every
output -- layer output, indices, gates, counts and logits -- must be
bit-identical.  Two calls in a row, the second with fewer tokens (the scratch
keeps the first call's contents), for the DeepSeek-V3-shaped decode layer
(128 tokens, capacity 1.25, Zipf-skewed logits) and a reduced V3 layer."""
import numpy as np
import pytest
import torch

import routing_expert_ffn_amd as moe
from workloads import CONFIGS, TEST_SHAPES, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _outputs(shape, T, out_dtype):
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    return dict(out=torch.full((T, shape.H), float("nan"), dtype=dt, device="cuda"),
                idx=torch.full((T, shape.k), -7, dtype=torch.int32, device="cuda"),
                w=torch.full((T, shape.k), float("nan"), dtype=torch.float32, device="cuda"),
                counts=torch.full((shape.E,), -7, dtype=torch.int32, device="cuda"),
                logits=torch.full((T, shape.E), float("nan"), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("name,sizes,out_dtype", [("deepseek_v3_decode", (128, 77), "f32"),
                                                  ("v3_small", (517, 200), "bf16")])
def test_noalloc_matches_forward_on_two_calls(name, sizes, out_dtype):
    shape = CONFIGS.get(name) or TEST_SHAPES[name]
    print("case", name, sizes, out_dtype, flush=True)
    inp = make_inputs(shape, device="cuda")
    for T in sizes:
        sub = shape.with_(T=T)
        cfg = moe.make_config(sub, out_dtype=out_dtype)
        assert moe.workspace_size(cfg, T) <= 64 << 20
        x = inp["x"][:T].contiguous()
        got = {}
        for mode in ("workspace", "static"):
            o = _outputs(shape, T, out_dtype)
            kw = dict(logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], topk_idx=o["idx"], topk_w=o["w"],
                      expert_counts=o["counts"], logits_out=o["logits"])
            if mode == "workspace":
                moe.forward(cfg, x, inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], out=o["out"],
                            ws=moe.workspace(cfg, T), **kw)
            else:
                moe.forward_noalloc(cfg, x, inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], o["out"],
                                    **kw)
            torch.cuda.synchronize()
            got[mode] = o
        a, b = got["workspace"], got["static"]
        assert bool(torch.isfinite(a["out"].float()).all())
        for key in ("out", "idx", "w", "counts", "logits"):
            assert torch.equal(a[key], b[key]), (name, T, key)
        if shape.capacity_factor > 0:
            C = int(np.ceil(shape.capacity_factor * T * shape.k / shape.E))
            assert int(b["counts"].max().item()) <= C
        print("%s T=%d: identical outputs" % (name, T), flush=True)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    shape = CONFIGS["deepseek_v3_prefill"]
    cfg = moe.make_config(shape)
    x = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((16,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(cfg, x, w, w, w, w, out)
    assert e.value.status == -3 and "static scratch" in str(e.value)
