"""Python binding of libmoe.so, the gfx950 sparse MoE FFN layer (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  torch supplies device memory and the stream: outputs not passed in
are allocated with torch.empty, and every call enqueues on
torch.cuda.current_stream() unless a stream is given.  There is no fallback:
if libmoe.so is missing or cannot be loaded, using the binding raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRTSOFTPLUS = 0, 1, 2
SCORING = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID, "sqrtsoftplus": MOE_SCORE_SQRTSOFTPLUS}
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
          -4: "MOE_ERR_HIP"}

EXPORTS = ("moe_workspace_size", "moe_route", "moe_route_hash", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_forward_hash", "moe_forward_fp8", "moe_expert_ffn_fp8",
           "moe_quantize_fp8", "moe_balance_update", "moe_probe_mfma_bf16", "moe_probe_mfma_fp8", "moe_probe_read",
           "moe_last_error",
           "moe_version", "moe_timing_enable", "moe_timing_read", "moe_timing_only", "moe_kernel_name")


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("n_routed_experts", ctypes.c_int32),
                ("n_shared_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("scoring", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("capacity_factor", ctypes.c_double),
                ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("drop_tokens", ctypes.c_int32)]


def make_config(shape, out_dtype=None):
    """moe_config from a layer description (attributes H, E, S, k, G,
    topk_group, I, scoring, renorm, scale, capacity_factor, dtype and
    optionally drop_tokens)."""
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8}[shape.dtype]
    if out_dtype is None:
        od = MOE_F32 if dt == MOE_F32 else MOE_BF16
    else:
        od = MOE_F32 if out_dtype in ("f32", torch.float32, MOE_F32) else MOE_BF16
    return moe_config(shape.H, shape.E, shape.S, shape.k, shape.G, shape.topk_group, shape.I,
                      SCORING[shape.scoring],
                      1 if shape.renorm else 0, float(shape.scale), float(shape.capacity_factor), dt, od,
                      1 if getattr(shape, "drop_tokens", False) else 0)


_lib = None


def lib():
    """The loaded libmoe.so (torch is imported first so that the library binds
    to the HIP runtime torch already loaded)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe.so is not built (run __graft_entry__.build() or "
                              "python -m routing_expert_ffn_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        C = ctypes.POINTER(moe_config)
        for name in ("moe_workspace_size", "moe_route", "moe_route_hash", "moe_permute", "moe_expert_ffn",
                     "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_forward_hash", "moe_forward_fp8",
                     "moe_expert_ffn_fp8", "moe_quantize_fp8", "moe_balance_update", "moe_timing_enable",
                     "moe_timing_read", "moe_timing_only", "moe_probe_mfma_bf16", "moe_probe_mfma_fp8",
                     "moe_probe_read"):
            getattr(L, name).restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [C, I64, ctypes.POINTER(SZ)]
        L.moe_route.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_permute.argtypes = [C, I64, P, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn.argtypes = [C, I64, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_combine.argtypes = [C, I64, P, P, P, P, P]
        L.moe_balance_update.argtypes = [C, P, P, ctypes.c_float, P, P, P]
        L.moe_forward.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_forward_noalloc.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.moe_route_hash.argtypes = [C, I64, P, P, P, P, P, P, P, I64, P, P, P, P, SZ, P]
        L.moe_forward_hash.argtypes = [C, I64, P, P, P, P, P, I64, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_forward_fp8.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn_fp8.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_quantize_fp8.argtypes = [I64, I32, P, P, P, I32, P]
        L.moe_probe_mfma_bf16.argtypes = [I32, I32, I64, P, ctypes.POINTER(ctypes.c_double), P]
        L.moe_probe_mfma_fp8.argtypes = [I32, I32, I64, P, ctypes.POINTER(ctypes.c_double), P]
        L.moe_probe_read.argtypes = [I32, I32, P, SZ, P, P]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_version.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_timing_enable.argtypes = [I32]
        L.moe_timing_read.argtypes = [P, P, I32]
        L.moe_timing_only.argtypes = [I32]
        L.moe_kernel_name.restype = ctypes.c_char_p
        L.moe_kernel_name.argtypes = [I32]
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version():
    return lib().moe_version().decode()


def workspace_size(cfg, T):
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), int(T), ctypes.byref(n)))
    return n.value


def workspace(cfg, T, device="cuda"):
    return torch.empty(max(workspace_size(cfg, T), 256), dtype=torch.uint8, device=device)


def _dev(t):
    return t.device if t is not None else torch.device("cuda")


def route(cfg, T, x=None, w_router=None, logit_bias=None, sel_bias=None, logits_in=None, logits_out=None,
          topk_idx=None, topk_w=None, expert_counts=None, ws=None, stream=None):
    """-> (topk_idx [T,k] int32, topk_w [T,k] fp32)"""
    dev = _dev(x if x is not None else logits_in)
    k = cfg.top_k
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, T, dev)
    _check(lib().moe_route(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(sel_bias), _p(logits_in),
                           _p(logits_out), _p(topk_idx), _p(topk_w), _p(expert_counts), _p(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))
    return topk_idx, topk_w


def route_hash(cfg, T, token_ids, tid2eid, x=None, w_router=None, logit_bias=None, logits_in=None,
               logits_out=None, topk_idx=None, topk_w=None, expert_counts=None, ws=None, stream=None):
    """Hash routing: token_ids [T] int32, tid2eid [vocab,k] int32 (device).
    -> (topk_idx [T,k] int32, topk_w [T,k] fp32)"""
    dev = _dev(x if x is not None else logits_in)
    k = cfg.top_k
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, T, dev)
    _check(lib().moe_route_hash(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(logits_in),
                                _p(logits_out), _p(token_ids), _p(tid2eid), int(tid2eid.shape[0]), _p(topk_idx),
                                _p(topk_w), _p(expert_counts), _p(ws), ws.numel(), _stream(stream)))
    return topk_idx, topk_w


def permute(cfg, topk_idx, ws=None, stream=None):
    """-> (expert_counts [E], expert_offsets [E+1], row_token [T*k+S*T], slot_row [T,k])"""
    T = topk_idx.shape[0]
    dev = topk_idx.device
    E, k, S = cfg.n_routed_experts, cfg.top_k, cfg.n_shared_experts
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k + S * T, dtype=torch.int32, device=dev)
    slot_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(cfg, T, dev)
    _check(lib().moe_permute(ctypes.byref(cfg), T, _p(topk_idx), _p(counts), _p(offsets), _p(row_token),
                             _p(slot_row), _p(ws), ws.numel(), _stream(stream)))
    return counts, offsets, row_token, slot_row


def expert_ffn(cfg, x, w_gate, w_up, w_down, expert_offsets, row_token, y_rows=None, ws=None, stream=None):
    """-> y_rows [T*k+S*T, H] fp32"""
    T = x.shape[0]
    rows = T * cfg.top_k + cfg.n_shared_experts * T
    if y_rows is None:
        y_rows = torch.empty((rows, cfg.hidden_size), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(cfg, T, x.device)
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), T, _p(x), _p(w_gate), _p(w_up), _p(w_down), _p(expert_offsets),
                                _p(row_token), _p(y_rows), _p(ws), ws.numel(), _stream(stream)))
    return y_rows


def combine(cfg, T, y_rows, slot_row, topk_w, out=None, stream=None):
    """-> out [T,H] in cfg.out_dtype"""
    if out is None:
        dt = torch.float32 if cfg.out_dtype == MOE_F32 else torch.bfloat16
        out = torch.empty((T, cfg.hidden_size), dtype=dt, device=y_rows.device)
    _check(lib().moe_combine(ctypes.byref(cfg), T, _p(y_rows), _p(slot_row), _p(topk_w), _p(out),
                             _stream(stream)))
    return out


def balance_update(cfg, expert_counts, sel_bias=None, gamma=0.001, stream=None):
    """One auxiliary-loss-free balancing step: sel_bias [E] fp32 is updated in
    place (if given); -> (share [E] fp32, stats [4] fp32: entropy in nats,
    max share, experts above / below the mean load)."""
    dev = expert_counts.device
    share = torch.empty(cfg.n_routed_experts, dtype=torch.float32, device=dev)
    stats = torch.empty(4, dtype=torch.float32, device=dev)
    _check(lib().moe_balance_update(ctypes.byref(cfg), _p(expert_counts), _p(sel_bias), float(gamma), _p(share),
                                    _p(stats), _stream(stream)))
    return share, stats


def forward(cfg, x, w_router, w_gate, w_up, w_down, logit_bias=None, sel_bias=None, out=None, topk_idx=None,
            topk_w=None, expert_counts=None, logits_out=None, ws=None, stream=None):
    """The whole layer; -> out [T,H] in cfg.out_dtype."""
    T = x.shape[0]
    if out is None:
        dt = torch.float32 if cfg.out_dtype == MOE_F32 else torch.bfloat16
        out = torch.empty((T, cfg.hidden_size), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(cfg, T, x.device)
    _check(lib().moe_forward(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(sel_bias), _p(w_gate),
                             _p(w_up), _p(w_down), _p(out), _p(topk_idx), _p(topk_w), _p(expert_counts),
                             _p(logits_out), _p(ws), ws.numel(), _stream(stream)))
    return out


def forward_noalloc(cfg, x, w_router, w_gate, w_up, w_down, out, logit_bias=None, sel_bias=None, topk_idx=None,
                    topk_w=None, expert_counts=None, logits_out=None, stream=None):
    """The whole layer on the library's static device scratch (no workspace
    argument); `out` [T,H] in cfg.out_dtype is required.  -> out"""
    T = x.shape[0]
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(sel_bias),
                                     _p(w_gate), _p(w_up), _p(w_down), _p(out), _p(topk_idx), _p(topk_w),
                                     _p(expert_counts), _p(logits_out), _stream(stream)))
    return out


def forward_hash(cfg, x, w_router, w_gate, w_up, w_down, token_ids, tid2eid, logit_bias=None, out=None,
                 topk_idx=None, topk_w=None, expert_counts=None, logits_out=None, ws=None, stream=None):
    """The whole layer with hash routing; -> out [T,H] in cfg.out_dtype."""
    T = x.shape[0]
    if out is None:
        dt = torch.float32 if cfg.out_dtype == MOE_F32 else torch.bfloat16
        out = torch.empty((T, cfg.hidden_size), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(cfg, T, x.device)
    _check(lib().moe_forward_hash(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(token_ids),
                                  _p(tid2eid), int(tid2eid.shape[0]), _p(w_gate), _p(w_up), _p(w_down), _p(out),
                                  _p(topk_idx), _p(topk_w), _p(expert_counts), _p(logits_out), _p(ws), ws.numel(),
                                  _stream(stream)))
    return out


def forward_fp8(cfg, x, w_router, w_gate, s_gate, w_up, s_up, w_down, s_down, logit_bias=None, sel_bias=None,
                out=None, topk_idx=None, topk_w=None, expert_counts=None, logits_out=None, ws=None, stream=None):
    """The whole layer with FP8 experts (uint8 E4M3 codes and UE8M0 block
    scales); -> out [T,H] in cfg.out_dtype."""
    T = x.shape[0]
    if out is None:
        dt = torch.float32 if cfg.out_dtype == MOE_F32 else torch.bfloat16
        out = torch.empty((T, cfg.hidden_size), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(cfg, T, x.device)
    _check(lib().moe_forward_fp8(ctypes.byref(cfg), T, _p(x), _p(w_router), _p(logit_bias), _p(sel_bias),
                                 _p(w_gate), _p(s_gate), _p(w_up), _p(s_up), _p(w_down), _p(s_down), _p(out),
                                 _p(topk_idx), _p(topk_w), _p(expert_counts), _p(logits_out), _p(ws), ws.numel(),
                                 _stream(stream)))
    return out


def expert_ffn_fp8(cfg, x, w_gate, s_gate, w_up, s_up, w_down, s_down, expert_offsets, row_token, y_rows=None,
                   ws=None, stream=None):
    """-> y_rows [T*k+S*T, H] fp32 (FP8 experts)"""
    T = x.shape[0]
    rows = T * cfg.top_k + cfg.n_shared_experts * T
    if y_rows is None:
        y_rows = torch.empty((rows, cfg.hidden_size), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(cfg, T, x.device)
    _check(lib().moe_expert_ffn_fp8(ctypes.byref(cfg), T, _p(x), _p(w_gate), _p(s_gate), _p(w_up), _p(s_up),
                                    _p(w_down), _p(s_down), _p(expert_offsets), _p(row_token), _p(y_rows), _p(ws),
                                    ws.numel(), _stream(stream)))
    return y_rows


def quantize_fp8(x, scale_stride=None, stream=None):
    """bf16 [rows, K] -> (E4M3 codes uint8 [rows, K], UE8M0 scales uint8
    [rows, scale_stride]) in 1 x 128 tiles."""
    rows, K = x.shape
    ss = K // 128 if scale_stride is None else scale_stride
    codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    scales = torch.zeros((rows, ss), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_fp8(rows, K, _p(x), _p(codes), _p(scales), ss, _stream(stream)))
    return codes, scales


def probe_mfma_bf16(blocks, iters, sink, vary=True, stream=None):
    """Enqueue the sustained bf16 matrix-core probe (vary: four A and four B
    fragments in turn, else one fixed pair); `sink` is a float32 device
    tensor of at least blocks * 256 elements.  -> FLOPs of the launch."""
    assert sink.dtype == torch.float32 and sink.numel() >= blocks * 256
    f = ctypes.c_double(0.0)
    _check(lib().moe_probe_mfma_bf16(1 if vary else 0, int(blocks), int(iters), _p(sink), ctypes.byref(f),
                                     _stream(stream)))
    return f.value


def probe_mfma_fp8(blocks, iters, sink, vary=True, stream=None):
    """The same probe on the FP8 experts' scaled E4M3 matrix instruction.
    -> FLOPs of the launch."""
    assert sink.dtype == torch.float32 and sink.numel() >= blocks * 256
    f = ctypes.c_double(0.0)
    _check(lib().moe_probe_mfma_fp8(1 if vary else 0, int(blocks), int(iters), _p(sink), ctypes.byref(f),
                                    _stream(stream)))
    return f.value


def probe_read(buf, mode, blocks, sink, stream=None):
    """Enqueue the streaming read probe over the device tensor `buf` (mode 0
    plain loads, 1 non-temporal loads, 2 global->LDS copies, 3 the same
    non-temporal); `sink` is a float32 device tensor of at least blocks * 256
    elements.  -> bytes read."""
    assert sink.dtype == torch.float32 and sink.numel() >= blocks * 256
    n = buf.numel() * buf.element_size()
    _check(lib().moe_probe_read(int(mode), int(blocks), _p(buf), n, _p(sink), _stream(stream)))
    return n


def timing_enable(max_launches):
    _check(lib().moe_timing_enable(int(max_launches)))


def timing_only(name=None):
    """Bracket only the launches of the named kernel (None: every kernel)."""
    kid = -1
    if name is not None:
        i = 0
        while True:
            n = lib().moe_kernel_name(i)
            if n is None:
                raise ValueError("unknown kernel %r" % name)
            if n.decode() == name:
                kid = i
                break
            i += 1
    _check(lib().moe_timing_only(kid))


def timing_read(n_kernels=16):
    """-> {kernel name: (total ms, launches)} for the launches recorded since
    timing_enable (waits for them)."""
    ms = (ctypes.c_double * n_kernels)()
    cnt = (ctypes.c_int64 * n_kernels)()
    _check(lib().moe_timing_read(ms, cnt, n_kernels))
    out = {}
    for i in range(n_kernels):
        name = lib().moe_kernel_name(i)
        if name is None:
            break
        if cnt[i]:
            out[name.decode()] = (ms[i], cnt[i])
    return out
