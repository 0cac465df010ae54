"""Every work item of the grouped expert GEMMs at the workloads' full sizes.

The expert GEMMs split the rows of each expert (routed, then shared) into row
tiles and the outputs into column tiles; the items are handed to the XCDs in
ranges and the last items of every range through a shared pool.  A skipped or
doubled item would leave stale rows that sampled-token tests can miss, so here
the workspace (which holds h) and y_rows are filled with NaN bytes before the
call, every row must come back finite, and the first and last row of every
(expert, row tile) -- every column tile of that row, in both projections --
are compared with the oracle's expert rows.  The layer being checked is the
one of "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个":
y = sum_k w_k * expert_k(x) + shared_expert(x), each expert a SwiGLU FFN.

The whole layer is then run with a NaN-filled workspace: every routed row is
read by exactly one (token, slot) and every shared row by its token, so a
finite output for every token shows that moe_forward's split rows (routed
bf16, shared fp32) were all written.
"""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_amd as moe
from tests.hostdata import to_oracle
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

BM = 256          # rows of a full row tile of the bf16 and FP8 expert GEMMs


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _tile_rows(off, T, k, E, S):
    """(row, expert) of the first and last row of every row tile."""
    out = []
    segs = [(off[e], off[e + 1], e) for e in range(E)]
    segs += [(T * k + s * T, T * k + (s + 1) * T, E + s) for s in range(S)]
    for a, b, e in segs:
        for r0 in range(a, b, BM):
            r1 = min(r0 + BM, b) - 1
            out.append((r0, e))
            if r1 != r0:
                out.append((r1, e))
    return np.array(out, dtype=np.int64)


# full widths at the workloads' batch sizes, and the DeepSeek-V3 shape at 2048
# and 4096 tokens, where every routed expert fits one row tile (non-temporal
# weights: gate/up per item, down per launch) while the shared expert spans
# several (default policy in gate/up)
@pytest.mark.parametrize("name,T", [("deepseek_v3_prefill", None), ("deepseek_v2", None), ("mixtral_8x7b", None),
                                    ("deepseek_v3_prefill_fp8", None), ("deepseek_v3_prefill", 2048),
                                    ("deepseek_v3_prefill", 4096), ("deepseek_v3_prefill_fp8", 1024)])
def test_every_gemm_work_item_full_size(name, T):
    shape = CONFIGS[name] if T is None else CONFIGS[name].with_(T=T)
    print("case", name, shape.T, flush=True)
    T, E, S, k, H = shape.T, shape.E, shape.S, shape.k, shape.H
    inp = make_inputs(shape, device="cuda")
    cfg = moe.make_config(shape, out_dtype="f32")
    ws = moe.workspace(cfg, T)
    idx, _ = moe.route(cfg, T, inp["x"], inp["w_router"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"],
                       ws=ws)
    counts, offsets, row_token, slot_row = moe.permute(cfg, idx, ws=ws)
    rows = T * k + S * T
    y = torch.full((rows, H), float("nan"), dtype=torch.float32, device="cuda")
    ws.fill_(0xFF)                       # h and every other workspace region: NaN / -1 bytes
    if shape.dtype == "fp8":
        moe.expert_ffn_fp8(cfg, inp["x"], inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"], inp["w_down"],
                           inp["s_down"], offsets, row_token, y_rows=y, ws=ws)
    else:
        moe.expert_ffn(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], offsets, row_token, y_rows=y, ws=ws)
    torch.cuda.synchronize()
    assigned = int(counts.sum().item())
    assert assigned == T * k                        # no capacity limit at these workloads
    finite = torch.isfinite(y).all(dim=1)
    assert bool(finite.all()), "%d expert rows not written" % int((~finite).sum().item())

    off = offsets.cpu().numpy()
    rt = row_token.cpu().numpy()
    sel = _tile_rows(off, T, k, E, S)
    r, e = sel[:, 0], sel[:, 1]
    tok = np.where(r < T * k, rt[np.minimum(r, T * k - 1)], (r - T * k) % T)
    assert np.all(tok >= 0)
    print("%s: checking %d rows (first and last of every row tile)" % (name, len(r)), flush=True)
    x_h = to_oracle(inp["x"])
    # each checked row as a token of a one-slot layer whose experts are the
    # routed and shared experts, gate 1
    one = shape.with_(E=E + S, S=0, k=1, G=1, topk_group=1)
    order = np.arange(len(r))
    if shape.dtype == "fp8":
        names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
        ref = oracle.forward_tokens_fp8(one, order, x_h[tok], e[:, None].astype(np.int32), np.ones((len(r), 1)),
                                        lambda ee: tuple(to_oracle(inp[n][ee]) for n in names))
    else:
        ref = oracle.forward_tokens(one, order, x_h[tok], e[:, None].astype(np.int32), np.ones((len(r), 1)),
                                    lambda ee: (to_oracle(inp["w_gate"][ee]), to_oracle(inp["w_up"][ee]),
                                                to_oracle(inp["w_down"][ee])))
    got = y[torch.from_numpy(r).cuda()].cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref) / rms
    worst = np.max(err, axis=1)
    print("%s: max err %.3g x RMS, mean %.3g" % (name, worst.max(), err.mean()), flush=True)
    if shape.dtype == "fp8":
        assert worst.max() <= 6e-2 and err.mean() <= 2e-3
    else:
        assert worst.max() <= 2e-2, (int(r[np.argmax(worst)]), int(e[np.argmax(worst)]))
    del y

    # the whole layer on a NaN-filled workspace
    ws.fill_(0xFF)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    cfg16 = moe.make_config(shape, out_dtype="bf16")
    if shape.dtype == "fp8":
        moe.forward_fp8(cfg16, inp["x"], inp["w_router"], inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"],
                        inp["w_down"], inp["s_down"], logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"],
                        out=out, ws=ws)
    else:
        moe.forward(cfg16, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                    logit_bias=inp["logit_bias"], sel_bias=inp["sel_bias"], out=out, ws=ws)
    torch.cuda.synchronize()
    bad = ~torch.isfinite(out.float()).all(dim=1)
    assert not bool(bad.any()), "%d tokens with a row that was not written" % int(bad.sum().item())
    del inp, ws, out
    torch.cuda.empty_cache()
