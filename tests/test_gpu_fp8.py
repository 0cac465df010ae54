"""FP8 experts on MI355X through the C ABI against the oracle: the 1 x 128
activation quantisation bit for bit, and the expert stage row by row.  (The
whole FP8 layer at reduced and full sizes runs in test_gpu_parity.py.)"""
import numpy as np
import pytest
import torch

import oracle
import routing_expert_ffn_amd as moe
from tests.hostdata import f32_to_bf16_bits, to_oracle
from workloads import TEST_SHAPES, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _bf16_bits_tensor(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("rows,K,stride", [(1, 128, 1), (37, 512, 4), (300, 7168, 59), (4, 2048, 16)])
def test_quantize_bit_exact(rows, K, stride):
    rng = np.random.default_rng(rows * 7 + K)
    mag = 2.0 ** rng.integers(-60, 60, (rows, K // 128))
    v = (rng.standard_normal((rows, K)) * np.repeat(mag, 128, axis=1)).astype(np.float32)
    if rows >= 37:
        v[1] = 0.0                                                   # all-zero tiles
        v[2, :128] = np.float32(2.0 ** -130)                          # subnormal-only tile (bf16 keeps it)
        v[3, 5] = np.float32(-0.0)
        v[4, :128] = np.float32(1.0625) * np.where(np.arange(128) % 2 == 0, 1, -1)   # ties after scaling
        v[4, 0] = np.float32(448.0 * 2.0 ** -7)
        v[5, :128] = rng.choice(np.array([448.0, -448.0, 3.5, 0.0], np.float32), 128) * np.float32(2.0 ** 20)
        v[6, 128:256] = np.float32(-(2.0 ** -126))
    bits = f32_to_bf16_bits(v)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    x = _bf16_bits_tensor(bits).cuda()
    codes, scales = moe.quantize_fp8(x, scale_stride=stride)
    torch.cuda.synchronize()
    oc, osc = oracle.quantize_e4m3(vals)
    assert np.array_equal(codes.cpu().numpy(), oc)
    s = scales.cpu().numpy()
    assert np.array_equal(s[:, :K // 128], osc)
    assert np.all(s[:, K // 128:] == 0)                               # bytes past K/128 untouched


def _codes(vals):
    return torch.from_numpy(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)


def _routing(shape, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(shape.E)[:shape.k] for _ in range(shape.T)]).astype(np.int32)
    for t in range(min(shape.T, 300)):            # expert 7 gets more than one full row tile
        if 7 not in idx[t]:
            idx[t, 0] = 7
    return idx


def _stage(shape, inp, idx):
    cfg = moe.make_config(shape)
    counts, offsets, row_token, slot_row = moe.permute(cfg, torch.from_numpy(idx).cuda())
    y = moe.expert_ffn_fp8(cfg, inp["x"], inp["w_gate"], inp["s_gate"], inp["w_up"], inp["s_up"], inp["w_down"],
                           inp["s_down"], offsets, row_token)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), offsets.cpu().numpy(), row_token.cpu().numpy()


def _expert_rows(shape, e, off, T):
    k, E = shape.k, shape.E
    return np.arange(off[e], off[e + 1]) if e < E else np.arange(T * k + (e - E) * T, T * k + (e - E + 1) * T)


def _oracle_rows(shape, inp, e, toks):
    """The oracle's expert e (routed or shared) on the listed tokens."""
    T = inp["x"].shape[0]
    one = np.full((T, 1), e if e < shape.E else -1, np.int32)
    sub = shape.with_(k=1, S=(e - shape.E + 1) if e >= shape.E else 0)
    names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
    return oracle.forward_tokens_fp8(sub, toks, to_oracle(inp["x"]), one, np.ones((T, 1)),
                                     lambda ee: tuple(to_oracle(inp[n][ee]) for n in names))


def _exact_inputs(shape, inp, seed, large_gate=False):
    """Codes and scales for which every product and partial sum is exact in
    the matrix cores (weights in {0, +-0.5, +-1} times 2^-6 .. 2^-4, x in
    {0, +-1, +-2} with a 7 in every 128-wide tile, which quantises exactly).
    large_gate: x in {1, 2} and W_gate in {0.5, 1} x 2^-1, so every gate value
    is at least 64 and silu(g) = g exactly in fp32 and fp64: h = g*u is then
    the same fp32 value on both sides and no h code can round differently."""
    T, E, S, H, I = shape.T, shape.E, shape.S, shape.H, shape.I
    rng = np.random.default_rng(seed)
    for n, shp in (("w_gate", (E + S, I, H)), ("w_up", (E + S, I, H)), ("w_down", (E + S, H, I))):
        sn = "s" + n[1:]
        if large_gate and n == "w_gate":
            inp[n] = _codes(rng.choice([0.5, 1.0], shp)).cuda()
            inp[sn] = torch.full(tuple(inp[sn].shape), 126, dtype=torch.uint8).cuda()
            continue
        inp[n] = _codes(rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], shp)).cuda()
        inp[sn] = torch.from_numpy(rng.integers(121, 124, tuple(inp[sn].shape)).astype(np.uint8)).cuda()
    vals = [1.0, 2.0] if large_gate else [-2.0, -1.0, 0.0, 1.0, 2.0]
    xv = rng.choice(vals, (T, H)).astype(np.float32)
    xv[:, ::128] = 7.0                           # tile maximum 7 = 448 * 2^-6: x quantises exactly
    inp["x"] = torch.from_numpy(xv).to(torch.bfloat16).cuda()


# Expert rows of exact-arithmetic inputs with large gate values: g and u are
# exact, silu(g) = g, so h and its E4M3 codes are the same on both sides;
# what remains is the fp32 rounding of the down projection's block sums.
EXACT_REL = 2e-4


def test_expert_stage_exact_arithmetic():
    """Codes and scales chosen so that every product and partial sum is exact
    in the matrix cores and h is the same value on both sides: the expert rows
    then match the oracle to rounding (within 2e-4 x RMS), on full and
    half-height row tiles and the shared expert."""
    shape = TEST_SHAPES["v3_fp8_small"].with_(T=600)
    inp = make_inputs(shape, device="cuda")
    E = shape.E
    T = shape.T
    _exact_inputs(shape, inp, 9, large_gate=True)
    idx = _routing(shape, 3)
    y, off, rt = _stage(shape, inp, idx)
    for e in (7, int(idx[100, 1]), E):
        rows = _expert_rows(shape, e, off, T)
        ref = _oracle_rows(shape, inp, e, rt[rows].astype(np.int64))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(y[rows] - ref) / rms
        print("expert %d: %d rows, max err %.3g x RMS" % (e, len(rows), err.max()))
        assert err.max() <= EXACT_REL


def test_h_codes_are_valid_roundings():
    """With W_down the identity (H == I), each expert row is the E4M3 value of
    h.  It must be a nearest rounding of the oracle's h, on the grid of an
    E4M3 value of its magnitude, up to the accumulation error of the FP8
    matrix cores: one v_mfma_scale_f32_32x32x64 block of 64 products was
    measured within 1.7e-4 of the sum of their magnitudes, so g and u may be
    off by 3e-4 x sum_k |x_k w_k| (fp32 across blocks adds far less).  Codes
    that differ from the oracle's must stay rare."""
    shape = TEST_SHAPES["v3_fp8_small"].with_(T=400, H=512, I=512)
    inp = make_inputs(shape, device="cuda")
    E, S, H = shape.E, shape.S, shape.H
    eye = np.zeros((E + S, H, H), np.float32)
    eye[:, np.arange(H), np.arange(H)] = 1.0
    inp["w_down"] = _codes(eye).cuda()
    inp["s_down"] = torch.full_like(inp["s_down"], 127)
    idx = _routing(shape, 4)
    y, off, rt = _stage(shape, inp, idx)
    for e in (7, E):
        rows = _expert_rows(shape, e, off, shape.T)
        ref = _oracle_rows(shape, inp, e, rt[rows].astype(np.int64))       # the oracle's dequantised h
        got = y[rows]
        # the unrounded h from the dequantised x and weights
        xv = (to_oracle(inp["x"])[rt[rows]].astype(np.uint32) << 16).view(np.float32)
        xc, xs = oracle.quantize_e4m3(xv)
        xq = oracle.e4m3_values(xc) * np.repeat(2.0 ** (xs.astype(np.float64) - 127), 128, axis=1)

        def deq(n):
            c = oracle.e4m3_values(to_oracle(inp["w_" + n][e]))
            sc = 2.0 ** (to_oracle(inp["s_" + n][e]).astype(np.float64) - 127)
            return c * np.kron(sc, np.ones((128, 128)))
        wg, wu = deq("gate"), deq("up")
        g, u = xq @ wg.T, xq @ wu.T
        sg = g / (1 + np.exp(-g))
        h = sg * u
        err_g, err_u = 3e-4 * (np.abs(xq) @ np.abs(wg).T), 3e-4 * (np.abs(xq) @ np.abs(wu).T)
        slack = 1.1 * np.abs(u) * err_g + np.abs(sg) * err_u + 1e-6 * np.abs(h)
        # E4M3 grid at the larger magnitude; subnormal grid of the tile below 2^-6 of its scale
        amax = np.maximum(np.abs(got), np.abs(ref)).reshape(len(rows), -1, 128).max(axis=2)
        p = np.repeat(np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / 448.0)), -127), 128, axis=1)
        mag = np.maximum(np.abs(got), np.abs(h))
        spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 3), 2.0 ** (p - 9))
        bad = np.abs(got - h) > 0.5 * spacing + slack
        assert not bad.any(), "%d h codes are not nearest roundings" % bad.sum()
        differ = np.mean(got != ref)
        print("expert %d: %d rows, %.4f of the h codes differ from the oracle's" % (e, len(rows), differ))
        assert differ < 0.05


def test_expert_stage_random_codes():
    """Random codes: the rows stay within the FP8 layer bar (max 6e-2, mean
    2e-3 of the RMS; the max is set by h codes that the GPU and the oracle
    round to neighbouring E4M3 values)."""
    shape = TEST_SHAPES["v3_fp8_small"].with_(T=300)
    inp = make_inputs(shape, device="cuda")
    idx = _routing(shape, 3)
    y, off, rt = _stage(shape, inp, idx)
    for e in (7, int(idx[100, 1]), shape.E):
        rows = _expert_rows(shape, e, off, shape.T)
        ref = _oracle_rows(shape, inp, e, rt[rows].astype(np.int64))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(y[rows] - ref) / rms
        print("expert %d: %d rows, max err %.3g, mean %.3g x RMS" % (e, len(rows), err.max(), err.mean()))
        assert err.max() <= 6e-2 and err.mean() <= 2e-3


def test_expert_stage_row_tile_boundaries():
    """FP8 experts whose row counts sit on and around the row-tile sizes:
    full 256-row tiles, last tiles of 129-192 rows (three 32-row blocks per
    wavefront) and short last tiles of at most 128 rows (half height, pairs
    of column tiles).  Exact-arithmetic inputs with large gate values, so h
    is the same on both sides and every row matches the oracle to rounding
    (random codes at I = 256 let single h codes round to neighbouring E4M3
    values on the two sides, which moves an output by up to ~0.1 x RMS)."""
    counts = [128, 256, 129, 1, 0, 127, 255, 257, 384, 160, 192, 193, 448, 449, 577]
    E = len(counts)
    T = max(counts)
    shape = TEST_SHAPES["v3_fp8_small"].with_(T=T, E=E, S=1, k=E, G=1, topk_group=1, H=256, I=256)
    idx = np.full((T, E), -1, np.int32)
    for t in range(T):
        es = [e for e in range(E) if t < counts[e]]
        idx[t, :len(es)] = es
    inp = make_inputs(shape, device="cuda")
    _exact_inputs(shape, inp, 21, large_gate=True)
    y, off, rt = _stage(shape, inp, idx)
    assert np.diff(off[:E + 1]).tolist() == counts
    for e in list(range(E)) + [E]:
        rows = _expert_rows(shape, e, off, T)
        if rows.size == 0:
            continue
        ref = _oracle_rows(shape, inp, e, rt[rows].astype(np.int64))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(y[rows] - ref) / rms
        assert err.max() <= EXACT_REL, (e, counts[e] if e < E else T, err.max())
