"""Pins of the oracle's FP8 expert path ("15. DeepSeek：MLA、MoE 与 MTP", section
"FP8 训练是训练配方，不是架构": E4M3 matrix inputs, one scale per 1 x 128
activation tile and per 128 x 128 weight block, UE8M0 scales as in V3.1).

The E4M3 decoding and the rounding of scaled values are checked against
hand-computed codes and against torch's float8_e4m3fn conversion (a library
routine); the layer against a construction with numpy block expansion and
against the bf16 layer where the quantisation is lossless."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.hostdata import f32_to_bf16_bits
from workloads import LayerShape


def _torch_e4m3_codes(v):
    """Round fp32 values to float8_e4m3fn with torch (nearest-even) -> codes."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


# ---- formats ----------------------------------------------------------------------

def test_e4m3_decode_hand_values():
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0,
            0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x70: 128.0, 0x78: 256.0, 0x6F: 120.0}
    for c, v in want.items():
        got = oracle.e4m3_values(np.array([c], np.uint8))[0]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(c)
    assert np.isnan(oracle.e4m3_values(np.array([0x7F, 0xFF], np.uint8))).all()
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(0) == 2.0 ** -127 and oracle.e8m0_value(254) == 2.0 ** 127


def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    a, b = oracle.e4m3_values(codes), _torch_e4m3_values(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok])
    pos = a[1:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 1..126 increase


# ---- quantisation of 1 x 128 tiles ----------------------------------------------------

def test_quantize_hand_tiles():
    z = [0.0] * 124
    v = np.array([[448.0, 0, 0, 0] + z,          # fits exactly: scale 2^0
                  [449.0, 0, 0, 0] + z,          # just above: scale 2^1, 449/2 -> 224
                  [1.75, 0, 0, 0] + z,           # 1.75 * 2^8 = 448: scale 2^-8
                  [1.7500001, 0, 0, 0] + z,      # one ulp more: scale 2^-7
                  [0.0, 0, 0, 0] + z,            # all zero: scale byte 0, codes 0
                  [1.0625, 1.1875, -1e-30, 3.0] + z],  # ties to even, negative zero
                 np.float32)
    codes, scales = oracle.quantize_e4m3(v)
    assert scales.ravel().tolist() == [127, 128, 119, 120, 0, 120]
    assert codes[:, :4].tolist() == [[0x7E, 0, 0, 0], [0x76, 0, 0, 0], [0x7E, 0, 0, 0], [0x76, 0, 0, 0],
                                     [0, 0, 0, 0], [0x70, 0x72, 0x80, 0x7C]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_matches_torch_rounding_and_minimal_scale(seed):
    rng = np.random.default_rng(seed)
    rows, K = 64, 512
    mag = 2.0 ** rng.integers(-40, 40, (rows, K // 128)).astype(np.float64)
    v = (rng.standard_normal((rows, K)) * np.repeat(mag, 128, axis=1)).astype(np.float32)
    v[3] = 0.0
    v[4, :128] = np.float32(2.0 ** -130)                 # subnormal-only tile
    v[5, 7] = np.float32(-0.0)
    v[6] = (rng.standard_normal(K) * 1e-3).astype(np.float32)
    v[6, 0] = np.float32(448 * 2.0 ** -12)               # amax exactly at a power-of-two boundary
    codes, scales = oracle.quantize_e4m3(v)
    p = scales.astype(np.int64) - 127
    amax = np.abs(v.astype(np.float64)).reshape(rows, K // 128, 128).max(axis=2)
    normal = amax >= 2.0 ** -126
    assert np.all(p[~normal] == -127)
    assert np.all(amax[normal] / 2.0 ** p[normal] <= 448.0)
    low = normal & (p > -127)
    assert np.all(amax[low] / 2.0 ** (p[low] - 1) > 448.0)   # the smallest such power of two
    scaled = v.astype(np.float64) / np.repeat(2.0 ** p, 128, axis=1)
    assert np.array_equal(codes, _torch_e4m3_codes(scaled.astype(np.float32)))
    # the scaled values are exact in fp32 (powers of two), so this is the rounding of v itself
    deq = oracle.e4m3_values(codes) * np.repeat(2.0 ** p, 128, axis=1)
    half = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(deq), 2.0 ** -6 * np.repeat(2.0 ** p, 128, axis=1)))) - 4)
    assert np.all(np.abs(deq - v) <= half * (1 + 1e-12))


# ---- the FP8 layer -----------------------------------------------------------------------

def _fp8_expert(rng, I, H, scale_jitter=True):
    """Random E4M3 codes (finite) and UE8M0 block scales of one expert."""
    def mat(rows, cols):
        codes = _torch_e4m3_codes(rng.standard_normal((rows, cols)).astype(np.float32) * 40.0)
        base = 127 - 6 - int(round(math.log2(math.sqrt(cols))))
        jitter = rng.integers(-2, 3, (rows // 128, cols // 128)) if scale_jitter else np.zeros((rows // 128, cols // 128))
        sc = (base + jitter).astype(np.uint8)
        return codes, sc
    g, sg = mat(I, H)
    u, su = mat(I, H)
    d, sd = mat(H, I)
    return g, sg, u, su, d, sd


def _dequant(codes, scales):
    return oracle.e4m3_values(codes) * np.kron(2.0 ** (scales.astype(np.float64) - 127), np.ones((128, 128)))


def test_fp8_layer_matches_block_expansion_with_library_rounding():
    """Dense numpy evaluation: block scales expanded with np.kron, activations
    quantised with torch's float8 conversion at the power-of-two tile scale."""
    H, I, E, S, k = 256, 384, 3, 1, 2
    shape = LayerShape("t", T=4, H=H, E=E, S=S, k=k, I=I, dtype="bf16")
    rng = np.random.default_rng(5)
    experts = [_fp8_expert(rng, I, H) for _ in range(E + S)]
    xf = rng.standard_normal((4, H)).astype(np.float32)
    xf[:, 128:] *= 30.0                                    # tiles of different magnitude
    xb = f32_to_bf16_bits(xf)
    x_val = (xb.astype(np.uint32) << 16).view(np.float32)
    idx = np.array([[0, 2], [1, -1], [2, 1], [0, 1]], np.int32)
    w = rng.uniform(0.1, 1.0, (4, k))

    def q_tiles(v32):
        v = v32.astype(np.float64).reshape(-1, 128)
        am = np.abs(v).max(axis=1)
        p = np.array([-127 if a < 2.0 ** -126 else max(-127, math.frexp(a)[1] - 1 - 8 + (2 * math.frexp(a)[0] > 1.75))
                      for a in am])
        c = _torch_e4m3_codes((v / 2.0 ** p[:, None]).astype(np.float32))
        return (_torch_e4m3_values(c) * 2.0 ** p[:, None]).reshape(v32.shape)

    ref = np.zeros((4, H))
    for t in range(4):
        xq = q_tiles(x_val[t])
        for j, e in list(enumerate(idx[t])) + [(None, E + s) for s in range(S)]:
            if e < 0:
                continue
            g, sg, u, su, d, sd = experts[e]
            gv, uv = _dequant(g, sg) @ xq, _dequant(u, su) @ xq
            h = (gv / (1.0 + np.exp(-gv)) * uv).astype(np.float32)
            ref[t] += (1.0 if j is None else w[t, j]) * (_dequant(d, sd) @ q_tiles(h))
    out = oracle.forward_tokens_fp8(shape, np.arange(4), xb, idx, w, lambda e: experts[e])
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_fp8_layer_with_exact_inputs_is_the_bf16_layer_up_to_h_rounding():
    """x tiles that quantise without loss and weights with one common scale: the FP8
    layer differs from the bf16 layer (same values) only by the rounding of h
    to E4M3, bounded element by element."""
    H, I = 256, 256
    shape = LayerShape("t", T=3, H=H, E=1, S=0, k=1, I=I, dtype="bf16")
    rng = np.random.default_rng(11)
    g, _, u, _, d, _ = _fp8_expert(rng, I, H, scale_jitter=False)
    one = np.full((2, 2), 117, np.uint8)                 # every block scaled by 2^-10
    # x: E4M3 values times 2^q per tile, each tile's largest magnitude exactly 448 * 2^q
    xc = _torch_e4m3_codes(rng.standard_normal((3, H)).astype(np.float32) * 60)
    xv = _torch_e4m3_values(xc)
    xv[:, 0], xv[:, 128] = 448.0, -448.0
    xv[:, 128:] *= 2.0 ** -9
    xv[:, :128] *= 2.0 ** -6
    xb = f32_to_bf16_bits(xv.astype(np.float32))
    assert np.array_equal((xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64), xv)
    idx = np.zeros((3, 1), np.int32)
    w = np.ones((3, 1))
    fp8 = oracle.forward_tokens_fp8(shape, np.arange(3), xb, idx, w, lambda e: (g, one, u, one, d, one))
    # the same layer in bf16 (all values here are exact in bf16)
    gv_, uv_, dv_ = (oracle.e4m3_values(m) * 2.0 ** -10 for m in (g, u, d))
    wg, wu, wd = (f32_to_bf16_bits(m.astype(np.float32)) for m in (gv_, uv_, dv_))
    bf = oracle.forward_tokens(shape, np.arange(3), xb, idx, w, lambda e: (wg, wu, wd))
    # bound: sum_i |W_down[n,i]| * (half spacing of h_i's tile grid)
    gv = gv_ @ xv.T
    uv = uv_ @ xv.T
    h = (gv / (1 + np.exp(-gv)) * uv).T.astype(np.float32)
    _, hs = oracle.quantize_e4m3(h)
    p = np.repeat(hs.astype(np.float64) - 127, 128, axis=1)
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(h), 2.0 ** (p - 6)))) - 3)
    bound = (np.abs(dv_) @ (0.5 * spacing).T).T
    diff = np.abs(fp8 - bf)
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-9)
    assert np.max(diff) > 0          # h rounding is real: the two layers are not identical
