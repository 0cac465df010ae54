"""Seeded synthetic inputs of a layer shape.

Distributions: x ~ N(0, 1); every weight ~ N(0, 1/fan_in) (router and gate/up:
fan_in = H; down: fan_in = I); optional selection bias ~ U(-a, a) in fp32;
optional Zipf(s) per-expert logit offset; FP8-expert layers draw E4M3 codes
and UE8M0 block scales instead of bf16 expert weights; for hash routing, token ids with
Zipf(1) frequencies over the vocabulary and a table of k distinct uniformly
drawn experts per id.  bf16 tensors are produced by
rounding fp32 draws to nearest-even (torch's conversion).

The random stream of each tensor is a torch Philox/CPU generator seeded from
(shape seed, tensor index), and weight tensors are drawn expert by expert, so
the bytes depend only on (shape, seed, device type).  Both the HIP path and the
oracle consume the same bytes: tests draw once and hand the same tensors (or
host copies of them) to both sides.
"""
import math

import numpy as np
import torch

_TENSORS = ("x", "w_router", "sel_bias", "zipf_perm", "w_gate", "w_up", "w_down", "token_ids", "tid2eid",
            "s_gate", "s_up", "s_down")


def _seed(base: int, name: str) -> int:
    return (base * 1_000_003 + 7919 * (_TENSORS.index(name) + 1)) & 0x7FFF_FFFF_FFFF


def _gen(device, base: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(base, name))
    return g


def _dtype(cfg):
    """dtype of x and the router weight (bf16 for FP8-expert layers)."""
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _fp8_matrix(shape, fan_in, g_codes, g_scales, device):
    """E4M3 codes [E+S, rows, cols] (uint8) and UE8M0 block scales [E+S,
    rows/128, cols/128]: codes of 40 * N(0,1) draws (torch's float8_e4m3fn
    conversion), block exponents 2^-(6 + log2 sqrt(fan_in)) +- 1 at random, so
    the values have about the spread of N(0, 1/fan_in)."""
    n, rows, cols = shape
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    for e in range(n):
        t = torch.randn((rows, cols), generator=g_codes, device=device, dtype=torch.float32).mul_(40.0)
        codes[e] = t.to(torch.float8_e4m3fn).view(torch.uint8)
    base = 127 - 6 - int(round(math.log2(math.sqrt(fan_in))))
    jitter = torch.randint(-1, 2, (n, rows // 128, cols // 128), generator=g_scales, device=device)
    return codes, (jitter + base).to(torch.uint8)


def _normal(shape, std, g, device, dtype):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def zipf_logit_offsets(E: int, s: float, seed: int) -> np.ndarray:
    """Centred log-pmf of a Zipf(s) law over E ranks, ranks assigned to experts
    by a seeded permutation.  Added to the router logits it skews the load the
    way the pages describe real traffic (a few experts take most tokens)."""
    ranks = np.random.Generator(np.random.PCG64(_seed(seed, "zipf_perm"))).permutation(E) + 1
    j = np.arange(1, E + 1, dtype=np.float64)
    logp = -s * np.log(ranks.astype(np.float64)) - math.log(np.sum(j ** -s))
    return (logp - logp.mean()).astype(np.float32)


def hash_table(vocab: int, E: int, k: int, seed: int) -> np.ndarray:
    """[vocab, k] int32 table of k distinct experts per row, uniform over the
    k-subsets of E in random order (rows with a repeat are drawn again)."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, "tid2eid")))
    tab = rng.integers(0, E, (vocab, k), dtype=np.int64)
    while True:
        srt = np.sort(tab, axis=1)
        bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0] if k > 1 else np.zeros(0, np.int64)
        if bad.size == 0:
            return tab.astype(np.int32)
        tab[bad] = rng.integers(0, E, (bad.size, k), dtype=np.int64)


def zipf_token_ids(T: int, vocab: int, seed: int, s: float = 1.0) -> np.ndarray:
    """[T] int32 token ids with Zipf(s) frequencies over the vocabulary (the
    rank-frequency law of text), ranks assigned to ids by a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, "token_ids")))
    p = np.arange(1, vocab + 1, dtype=np.float64) ** -s
    ranks = rng.choice(vocab, size=T, p=p / p.sum())
    return rng.permutation(vocab)[ranks].astype(np.int32)


def make_inputs(cfg, device="cpu", seed=None, T=None):
    """Return a dict of tensors on `device`:
    x [T,H], w_router [E,H], w_gate/w_up [E+S,I,H], w_down [E+S,H,I] in the
    layer dtype (FP8-expert layers: x and w_router bf16, the expert matrices
    E4M3 codes with s_gate/s_up [E+S,I/128,H/128] and s_down [E+S,H/128,I/128]
    UE8M0 block scales); sel_bias [E] fp32 or None; logit_bias [E] fp32 or None;
    with hash routing token_ids [T] and tid2eid [vocab,k] int32, else None."""
    base = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    dt = _dtype(cfg)
    H, E, S, I = cfg.H, cfg.E, cfg.S, cfg.I
    out = {}
    out["x"] = _normal((T, H), 1.0, _gen(device, base, "x"), device, dt)
    out["w_router"] = _normal((E, H), 1.0 / math.sqrt(H), _gen(device, base, "w_router"), device, dt)
    if cfg.sel_bias:
        g = _gen(device, base, "sel_bias")
        u = torch.rand((E,), generator=g, device=device, dtype=torch.float32)
        out["sel_bias"] = (u * (2.0 * cfg.sel_bias) - cfg.sel_bias).contiguous()
    else:
        out["sel_bias"] = None
    if cfg.zipf_s:
        out["logit_bias"] = torch.from_numpy(zipf_logit_offsets(E, cfg.zipf_s, base)).to(device)
    else:
        out["logit_bias"] = None
    vocab = getattr(cfg, "hash_vocab", 0)
    if vocab > 0:
        out["token_ids"] = torch.from_numpy(zipf_token_ids(T, vocab, base)).to(device)
        out["tid2eid"] = torch.from_numpy(hash_table(vocab, E, cfg.k, base)).to(device)
    else:
        out["token_ids"] = out["tid2eid"] = None
    if cfg.dtype == "fp8":
        for name, sname, shape, fan in (("w_gate", "s_gate", (I, H), H), ("w_up", "s_up", (I, H), H),
                                        ("w_down", "s_down", (H, I), I)):
            out[name], out[sname] = _fp8_matrix((E + S,) + shape, fan, _gen(device, base, name),
                                                _gen(device, base, sname), device)
        return out
    for name, shape, std in (("w_gate", (I, H), 1.0 / math.sqrt(H)),
                             ("w_up", (I, H), 1.0 / math.sqrt(H)),
                             ("w_down", (H, I), 1.0 / math.sqrt(I))):
        w = torch.empty((E + S,) + shape, device=device, dtype=dt)
        g = _gen(device, base, name)
        for e in range(E + S):
            w[e] = _normal(shape, std, g, device, dt)
        out[name] = w
    return out
