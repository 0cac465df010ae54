"""CPU oracle of the sparse MoE FFN layer (fp64, plain loops) -- Python glue.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library and never imports it.  The arithmetic lives in oracle.c (see its
header for the passages each step follows); this module only marshals numpy
arrays into it.

Inputs are numpy arrays: fp32 arrays for fp32 layers and uint16 arrays holding
bf16 bit patterns for bf16 layers.  `cfg` is any object with the attributes
H, E, S, k, G, topk_group, I, scoring, renorm, scale, capacity_factor, dtype
(and optionally drop_tokens).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=gnu11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("S", ctypes.c_int32), ("k", ctypes.c_int32),
                ("G", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("I", ctypes.c_int32),
                ("scoring", ctypes.c_int32), ("renorm", ctypes.c_int32), ("scale", ctypes.c_double),
                ("capacity_factor", ctypes.c_double), ("dtype", ctypes.c_int32), ("drop_tokens", ctypes.c_int32)]


_lib_override = None


def use_library(path=None):
    """Load the oracle from another build of oracle.c (the mutation tests use
    this to run the pins against copies with planted mistakes); None restores
    the default build."""
    global _lib, _lib_override
    _lib_override = path
    _lib = None


def _load():
    global _lib
    if _lib is None:
        path = _lib_override or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_exp32.restype = ctypes.c_float
        lib.oracle_exp32.argtypes = [ctypes.c_float]
        lib.oracle_sigmoid32.restype = ctypes.c_float
        lib.oracle_sigmoid32.argtypes = [ctypes.c_float]
        lib.oracle_sigmoid32_array.argtypes = [I64, P, P]
        lib.oracle_exp32_array.argtypes = [I64, P, P]
        lib.oracle_sqrtsoftplus32.restype = ctypes.c_float
        lib.oracle_sqrtsoftplus32.argtypes = [ctypes.c_float]
        lib.oracle_sqrtsoftplus32_array.argtypes = [I64, P, P]
        lib.oracle_hash_select.argtypes = [P, I64, P, P, P, I64, P, P, P]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_values.argtypes = [I64, P, P]
        lib.oracle_quantize_e4m3.argtypes = [I64, I64, P, P, P, I64]
        lib.oracle_forward_tokens_fp8.argtypes = [P, I64, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_router_logits.argtypes = [P, I64, P, P, P, P]
        lib.oracle_select.argtypes = [P, I64, P, P, P, P, P, P]
        lib.oracle_capacity.restype = I64
        lib.oracle_capacity.argtypes = [P, I64]
        lib.oracle_permute.argtypes = [P, I64, P, P, P, P, P]
        lib.oracle_expert_rows.argtypes = [P, I64, P, P, P, P, P]
        lib.oracle_forward_tokens.argtypes = [P, I64, P, P, P, P, P, P, P, P]
        lib.oracle_combine.argtypes = [P, I64, P, P, P, P]
        lib.oracle_balance_update.argtypes = [ctypes.c_int, P, P, ctypes.c_float, P, P]
        lib.oracle_moe_layer_params.restype = I64
        lib.oracle_moe_layer_params.argtypes = [I64, I64, I64, I64]
        lib.oracle_moe_active_params.restype = I64
        lib.oracle_moe_active_params.argtypes = [I64, I64, I64, I64, I64]
        _lib = lib
    return _lib


_SCORING = {"softmax": 0, "sigmoid": 1, "sqrtsoftplus": 2}


def _layer(cfg) -> _Layer:
    return _Layer(cfg.H, cfg.E, cfg.S, cfg.k, cfg.G, cfg.topk_group, cfg.I,
                  _SCORING[cfg.scoring], 1 if cfg.renorm else 0, float(cfg.scale),
                  float(cfg.capacity_factor), 0 if cfg.dtype == "f32" else 1,
                  1 if getattr(cfg, "drop_tokens", False) else 0)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _input(a, cfg):
    """Contiguous host array in the layer's input encoding."""
    a = np.ascontiguousarray(a)
    want = np.float32 if cfg.dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError("oracle input must be %s, got %s" % (want, a.dtype))
    return a


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def exp32(z):
    z = np.ascontiguousarray(z, dtype=np.float32)
    out = np.empty_like(z)
    _load().oracle_exp32_array(z.size, _ptr(z), _ptr(out))
    return out


def sigmoid32(l):
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.empty_like(l)
    _load().oracle_sigmoid32_array(l.size, _ptr(l), _ptr(out))
    return out


def sqrtsoftplus32(l):
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.empty_like(l)
    _load().oracle_sqrtsoftplus32_array(l.size, _ptr(l), _ptr(out))
    return out


def router_logits(cfg, x, w_router, logit_bias=None):
    x = _input(x, cfg)
    w_router = _input(w_router, cfg)
    T = x.shape[0]
    out = np.empty((T, cfg.E), dtype=np.float32)
    L = _layer(cfg)
    lb = _f32(logit_bias)
    _load().oracle_router_logits(ctypes.byref(L), T, _ptr(x), _ptr(w_router), _ptr(lb), _ptr(out))
    return out


def capacity(cfg, T):
    L = _layer(cfg)
    c = _load().oracle_capacity(ctypes.byref(L), T)
    return None if c < 0 else int(c)


def select(cfg, logits, sel_bias=None):
    """-> (idx int32 [T,k], w float64 [T,k], margin float64 [T], counts int32 [E])"""
    logits = _f32(logits)
    T = logits.shape[0]
    idx = np.empty((T, cfg.k), dtype=np.int32)
    w = np.empty((T, cfg.k), dtype=np.float64)
    margin = np.empty((T,), dtype=np.float64)
    counts = np.empty((cfg.E,), dtype=np.int32)
    L = _layer(cfg)
    sb = _f32(sel_bias)
    rc = _load().oracle_select(ctypes.byref(L), T, _ptr(logits), _ptr(sb), _ptr(idx), _ptr(w), _ptr(margin),
                               _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_select rejected the layer shape")
    return idx, w, margin, counts


def hash_select(cfg, logits, token_ids, tid2eid):
    """Hash routing: experts from rows of the table tid2eid [vocab, k] picked
    by token_ids [T]; gates from the logits.  -> (idx int32 [T,k], w float64
    [T,k], counts int32 [E])"""
    logits = _f32(logits)
    T = logits.shape[0]
    token_ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    tid2eid = np.ascontiguousarray(tid2eid, dtype=np.int32)
    if token_ids.shape != (T,) or tid2eid.ndim != 2 or tid2eid.shape[1] != cfg.k:
        raise ValueError("token_ids must be [T] and tid2eid [vocab, k]")
    idx = np.empty((T, cfg.k), dtype=np.int32)
    w = np.empty((T, cfg.k), dtype=np.float64)
    counts = np.empty((cfg.E,), dtype=np.int32)
    L = _layer(cfg)
    rc = _load().oracle_hash_select(ctypes.byref(L), T, _ptr(logits), _ptr(token_ids), _ptr(tid2eid),
                                    tid2eid.shape[0], _ptr(idx), _ptr(w), _ptr(counts))
    if rc == -2:
        raise ValueError("hash routing has no next-best expert: capacity needs drop mode")
    if rc != 0:
        raise ValueError("oracle_hash_select rejected the layer shape")
    return idx, w, counts


def permute(cfg, idx):
    """-> (counts [E], offsets [E+1], row_token [T*k+S*T], slot_row [T*k])"""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T = idx.shape[0]
    counts = np.empty((cfg.E,), dtype=np.int32)
    offsets = np.empty((cfg.E + 1,), dtype=np.int32)
    row_token = np.empty((T * cfg.k + cfg.S * T,), dtype=np.int32)
    slot_row = np.empty((T * cfg.k,), dtype=np.int32)
    L = _layer(cfg)
    rc = _load().oracle_permute(ctypes.byref(L), T, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(row_token),
                                _ptr(slot_row))
    if rc != 0:
        raise ValueError("oracle_permute: index out of range")
    return counts, offsets, row_token, slot_row.reshape(T, cfg.k)


def expert_rows(cfg, x_rows, wg, wu, wd):
    """y [n,H] (float64) of one expert applied to n rows."""
    x_rows = _input(x_rows, cfg)
    wg, wu, wd = _input(wg, cfg), _input(wu, cfg), _input(wd, cfg)
    n = x_rows.shape[0]
    y = np.empty((n, cfg.H), dtype=np.float64)
    L = _layer(cfg)
    _load().oracle_expert_rows(ctypes.byref(L), n, _ptr(x_rows), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(y))
    return y


def forward_tokens(cfg, tokens, x, idx, w, get_expert):
    """Layer output (float64 [n,H]) of the listed tokens given their selection.

    get_expert(e) -> (w_gate[e] [I,H], w_up[e] [I,H], w_down[e] [H,I]) host
    arrays; it is called once per expert the listed tokens need."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    x = _input(x, cfg)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n_exp = cfg.E + cfg.S
    need = set(range(cfg.E, n_exp))
    for t in tokens:
        need.update(int(e) for e in idx[t] if e >= 0)
    keep = {}
    ptrs = [(ctypes.c_void_p * n_exp)() for _ in range(3)]
    for e in sorted(need):
        mats = tuple(_input(m, cfg) for m in get_expert(e))
        keep[e] = mats
        for p, m in zip(ptrs, mats):
            p[e] = m.ctypes.data
    out = np.empty((tokens.size, cfg.H), dtype=np.float64)
    L = _layer(cfg)
    rc = _load().oracle_forward_tokens(ctypes.byref(L), tokens.size, _ptr(tokens), _ptr(x), _ptr(idx), _ptr(w),
                                       ptrs[0], ptrs[1], ptrs[2], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_forward_tokens: missing expert weights")
    return out


def e4m3_values(codes):
    """float64 values of E4M3 codes (NaN for the two NaN codes)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_e4m3_values(codes.size, _ptr(codes), _ptr(out))
    return out


def e8m0_value(b):
    return float(_load().oracle_e8m0_value(int(b)))


def quantize_e4m3(values):
    """fp32 [rows, K] (K % 128 == 0) -> (codes uint8 [rows, K], scale bytes
    uint8 [rows, K/128]) in 1 x 128 tiles."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    if v.ndim != 2 or v.shape[1] % 128 != 0:
        raise ValueError("values must be [rows, K] with K % 128 == 0")
    rows, K = v.shape
    codes = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty((rows, K // 128), dtype=np.uint8)
    if _load().oracle_quantize_e4m3(rows, K, _ptr(v), _ptr(codes), _ptr(scales), K // 128) != 0:
        raise ValueError("bad quantisation shape")
    return codes, scales


def forward_tokens_fp8(cfg, tokens, x, idx, w, get_expert):
    """Layer output (float64 [n,H]) of the listed tokens with FP8 experts.
    x: bf16 bits [T,H]; get_expert(e) -> (w_gate codes [I,H], gate scales
    [I/128,H/128], w_up codes, up scales, w_down codes [H,I], down scales
    [H/128,I/128]) as uint8 host arrays."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n_exp = cfg.E + cfg.S
    need = set(range(cfg.E, n_exp))
    for t in tokens:
        need.update(int(e) for e in idx[t] if e >= 0)
    keep = {}
    ptrs = [(ctypes.c_void_p * n_exp)() for _ in range(6)]
    for e in sorted(need):
        mats = tuple(np.ascontiguousarray(m, dtype=np.uint8) for m in get_expert(e))
        keep[e] = mats
        for p, m in zip(ptrs, mats):
            p[e] = m.ctypes.data
    out = np.empty((tokens.size, cfg.H), dtype=np.float64)
    L = _layer(cfg)
    rc = _load().oracle_forward_tokens_fp8(ctypes.byref(L), tokens.size, _ptr(tokens), _ptr(x), _ptr(idx), _ptr(w),
                                           *ptrs, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_forward_tokens_fp8: missing expert weights or bad shape")
    return out


def forward(cfg, x, w_router, w_gate, w_up, w_down, sel_bias=None, logit_bias=None, tokens=None,
            token_ids=None, tid2eid=None):
    """Whole layer: logits -> selection -> experts -> combine.  Returns a dict
    with logits, idx, w, margin, counts and out (float64, rows of `tokens`,
    all tokens by default).  With token_ids and tid2eid the selection is hash
    routing (margin is then +inf: no ranking decides it)."""
    logits = router_logits(cfg, x, w_router, logit_bias)
    if tid2eid is not None:
        idx, w, counts = hash_select(cfg, logits, token_ids, tid2eid)
        margin = np.full(logits.shape[0], np.inf)
    else:
        idx, w, margin, counts = select(cfg, logits, sel_bias)
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    out = forward_tokens(cfg, tokens, x, idx, w, lambda e: (w_gate[e], w_up[e], w_down[e]))
    return dict(logits=logits, idx=idx, w=w, margin=margin, counts=counts, out=out)


def combine(cfg, y_rows, slot_row, w):
    """out [T,H] (float64) from expert rows in the row space (see permute)."""
    slot_row = np.ascontiguousarray(slot_row, dtype=np.int32)
    T = slot_row.shape[0]
    y_rows = np.ascontiguousarray(y_rows, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    if y_rows.shape[0] < T * cfg.k + cfg.S * T or y_rows.shape[1] != cfg.H:
        raise ValueError("y_rows must be [T*k + S*T, H]")
    out = np.empty((T, cfg.H), dtype=np.float64)
    L = _layer(cfg)
    _load().oracle_combine(ctypes.byref(L), T, _ptr(y_rows), _ptr(slot_row), _ptr(w), _ptr(out))
    return out


def balance_update(counts, bias, gamma):
    """One auxiliary-loss-free balancing step.  counts [E] int, bias [E]
    fp32, gamma fp32 -> (new bias [E] fp32, share [E] float64, stats
    {entropy (nats), max_share, over, under})."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    E = counts.shape[0]
    share = np.empty(E, dtype=np.float64)
    stats = np.empty(4, dtype=np.float64)
    st = _load().oracle_balance_update(E, _ptr(counts), _ptr(b), ctypes.c_float(gamma), _ptr(share), _ptr(stats))
    if st != 0:
        raise ValueError("negative expert count")
    return b, share, {"entropy": stats[0], "max_share": stats[1], "over": int(stats[2]), "under": int(stats[3])}


def moe_layer_params(H, E, S, I):
    return int(_load().oracle_moe_layer_params(H, E, S, I))


def moe_active_params(H, E, S, k, I):
    return int(_load().oracle_moe_active_params(H, E, S, k, I))
