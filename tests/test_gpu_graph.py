"""The layer captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches) replays bit-identically to the eager call.

The library launches only kernels (and, in one corner, device-to-device
copies) on the caller's stream, allocates nothing and never synchronises, so
a caller may capture a layer call.  Each case captures one call, replays it
several times with eager work and synchronisations in between (the output
is poisoned before each replay), and checks every replay bit for bit against
the eager call -- the layer is deterministic -- then feeds a new input
through the captured buffer and checks the replay against a fresh eager call
on it.
"""
import pytest
import torch

import routing_expert_ffn_amd as moe
from workloads import TEST_SHAPES, make_inputs

pytestmark = pytest.mark.gpu


def _call(shape, cfg, inp, x, out, ws):
    if shape.dtype == "fp8":
        moe.forward_fp8(cfg, x, inp["w_router"], inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"],
                        inp["w_down"], inp["s_down"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"],
                        out=out, ws=ws)
    else:
        moe.forward(cfg, x, inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                    logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], out=out, ws=ws)


@pytest.mark.parametrize("name", ["v3_small", "v3_decode_small", "mixtral_small", "v2_small", "v3_fp8_small",
                                  "v3_decode_fp8_small"])
def test_layer_replays_from_a_graph(name):
    shape = TEST_SHAPES[name]
    print("case %s T=%d" % (name, shape.T), flush=True)
    inp = make_inputs(shape, device="cuda")
    cfg = moe.make_config(shape, out_dtype="bf16")
    T = shape.T
    ws_eager, ws_graph = moe.workspace(cfg, T), moe.workspace(cfg, T)
    ref = torch.empty((T, shape.H), dtype=torch.bfloat16, device="cuda")
    _call(shape, cfg, inp, inp["x"], ref, ws_eager)

    x = inp["x"].clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(shape, cfg, inp, x, out, ws_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(shape, cfg, inp, x, out, ws_graph)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)

    # a new batch through the captured input buffer
    x2 = torch.flip(inp["x"], dims=[0]).contiguous() * 0.5
    ref2 = torch.empty_like(ref)
    _call(shape, cfg, inp, x2, ref2, ws_eager)
    x.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    assert not torch.equal(ref2, ref)
    del g
