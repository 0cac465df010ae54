// C ABI of the MoE layer (include/moe.h): validation, workspace layout and
// launch sequencing on the caller's stream.  No device memory is allocated
// here and nothing synchronises the host except moe_timing_read.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

// ---- per-kernel timing -------------------------------------------------------
struct Timing {
  int max = 0;
  int used = 0;
  int only = -1;  // kernel id whose launches are bracketed, -1 = every kernel
  std::vector<hipEvent_t> ev;
  std::vector<int> ids;
};
Timing g_timing;

template <class F>
hipError_t timed(int id, hipStream_t s, F&& f) {
  if (g_timing.max > 0 && g_timing.used < g_timing.max && (g_timing.only < 0 || g_timing.only == id)) {
    const int slot = g_timing.used++;
    hipEventRecord(g_timing.ev[2 * slot], s);
    const hipError_t err = f();
    hipEventRecord(g_timing.ev[2 * slot + 1], s);
    g_timing.ids[slot] = id;
    return err;
  }
  return f();
}

// ---- static scratch of moe_forward_noalloc ---------------------------------------
// The workspace of moe_forward_noalloc: a device array of the code object,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address of the current GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

// ---- configuration -------------------------------------------------------------
struct Dims {
  int64_t T;
  int H, E, S, k, G, gsz, topk_group, I, scoring, renorm, dtype, out_dtype;
  float scale;
  int capacity;   // <= 0: unlimited
  int drop;       // with a capacity: drop the overflow instead of re-routing
  int n_allowed;
  int esz;        // bytes per element of x (and the router weight)
  int xdt;        // dtype of x and the router weight: MOE_F32 or MOE_BF16
  int fp8;        // expert matrices are E4M3 codes with UE8M0 block scales
};

moe_status check_config(const moe_config* c, int64_t T, Dims& d) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  d.T = T;
  d.H = c->hidden_size;
  d.E = c->n_routed_experts;
  d.S = c->n_shared_experts;
  d.k = c->top_k;
  d.G = c->n_group;
  d.topk_group = c->topk_group;
  d.I = c->moe_intermediate_size;
  d.scoring = c->scoring;
  d.renorm = c->norm_topk_prob ? 1 : 0;
  d.scale = c->routed_scaling_factor;
  d.dtype = c->dtype;
  d.out_dtype = c->out_dtype;
  if (d.dtype != MOE_F32 && d.dtype != MOE_BF16 && d.dtype != MOE_FP8)
    return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32, MOE_BF16 or MOE_FP8");
  if (d.out_dtype != MOE_F32 && d.out_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "out_dtype must be MOE_F32 or MOE_BF16");
  if (d.scoring != MOE_SCORE_SOFTMAX && d.scoring != MOE_SCORE_SIGMOID && d.scoring != MOE_SCORE_SQRTSOFTPLUS)
    return fail(MOE_ERR_INVALID_ARG, "scoring must be MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID or MOE_SCORE_SQRTSOFTPLUS");
  if (d.H <= 0 || d.I <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden_size and moe_intermediate_size must be > 0");
  if (d.E < 1) return fail(MOE_ERR_INVALID_ARG, "n_routed_experts must be >= 1");
  if (d.E > 512) return fail(MOE_ERR_UNSUPPORTED, "n_routed_experts > 512 is not supported");
  if (d.S < 0) return fail(MOE_ERR_INVALID_ARG, "n_shared_experts must be >= 0");
  if (d.k < 1 || d.k > d.E) return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, n_routed_experts]");
  if (d.k > 32) return fail(MOE_ERR_UNSUPPORTED, "top_k > 32 is not supported");
  if (d.G < 1 || d.E % d.G != 0) return fail(MOE_ERR_INVALID_ARG, "n_group must divide n_routed_experts");
  if (d.G > 32) return fail(MOE_ERR_UNSUPPORTED, "n_group > 32 is not supported");
  d.gsz = d.E / d.G;
  if (d.G > 1 && d.gsz < 2) return fail(MOE_ERR_INVALID_ARG, "groups need at least 2 experts");
  if (d.topk_group < 1 || d.topk_group > d.G) return fail(MOE_ERR_INVALID_ARG, "topk_group must be in [1, n_group]");
  d.n_allowed = d.G > 1 ? d.topk_group * d.gsz : d.E;
  if (d.k > d.n_allowed) return fail(MOE_ERR_INVALID_ARG, "top_k exceeds the experts of the kept groups");
  if (!std::isfinite(d.scale)) return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor must be finite");
  if (!std::isfinite(c->capacity_factor)) return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if (d.dtype != MOE_F32) {
    if (d.H % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16 and FP8 layers need hidden_size % 256 == 0");
    if (d.I % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 and FP8 layers need moe_intermediate_size % 128 == 0");
  } else {
    if (d.H % 32 != 0) return fail(MOE_ERR_UNSUPPORTED, "fp32 layers need hidden_size % 32 == 0");
    if (d.I % 32 != 0) return fail(MOE_ERR_UNSUPPORTED, "fp32 layers need moe_intermediate_size % 32 == 0");
  }
  d.fp8 = d.dtype == MOE_FP8 ? 1 : 0;
  d.xdt = d.dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
  d.esz = d.xdt == MOE_BF16 ? 2 : 4;
  const int64_t rows = T * d.k + (int64_t)d.S * T;
  if (rows > 0x7FFFFFFF || T * (int64_t)d.E > 0x7FFFFFFF)
    return fail(MOE_ERR_UNSUPPORTED, "T*(k+S) and T*E must fit in int32");
  if (c->drop_tokens != 0 && c->drop_tokens != 1) return fail(MOE_ERR_INVALID_ARG, "drop_tokens must be 0 or 1");
  d.drop = c->drop_tokens;
  d.capacity = 0;
  if (c->capacity_factor > 0.0) {
    // C = ceil(((cf*T)*k)/E) evaluated in IEEE double, left to right, on the
    // caller's double factor (a decimal such as 1.2 is not representable in
    // fp32, and its fp32 value can make C one larger)
    const double cap = std::ceil(c->capacity_factor * (double)T * (double)d.k / (double)d.E);
    if (cap > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "capacity too large");
    d.capacity = (int)cap;
    if (d.capacity < 1 && T > 0) d.capacity = 1;
  }
  return MOE_OK;
}

struct Layout {
  size_t logits, rpart, cand, idx, w, counts, offsets, slot_row, row_token, chunk_cnt, chunk_base, seg_start, seg_len,
      f_prefix, h_prefix, pool, h, y, xq, sx, sxr, sh, sbg, sbu, sbd, dcnt, total;
};

// bytes of a grouped row-space scale array (4-step groups of K/128 blocks)
size_t grouped_scales(size_t rows, int nkb) { return ((size_t)(nkb + 3) / 4) * rows * 4; }
int pad4(int n) { return (n + 3) & ~3; }

// FP8 layers: x's tile scales per token ([T, H/128]); rows of the row space
// (the K-block-major scale arrays of the GEMMs are [K/128, rows])
int sx_stride(const Dims& d) { return d.H / 128; }
int64_t row_space(const Dims& d) { return d.T * d.k + (int64_t)d.S * d.T; }

Layout layout_of(const Dims& d) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t T = (size_t)d.T, E = d.E, S = d.S, k = d.k;
  const size_t rows = T * k + S * T;
  const size_t nchunks = (T + 63) / 64;
  L.logits = take(T * E * 4);
  // partial router logits of the K slices (bf16 router GEMM, small T)
  size_t nsplit = 1;
  if (d.xdt == MOE_BF16 && d.T > 0) {
    int sps;
    nsplit = (size_t)router_splits(d.T, d.H, d.E, &sps);
  }
  L.rpart = take(nsplit > 1 ? nsplit * T * E * 4 : 0);
  L.cand = take(d.capacity > 0 && !d.drop ? T * (size_t)d.n_allowed * 4 : 0);
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.slot_row = take(T * k * 4);
  L.row_token = take(rows * 4);
  L.chunk_cnt = take(nchunks * E * 4);
  L.chunk_base = take(nchunks * E * 4);
  L.seg_start = take((E + S) * 4);
  L.seg_len = take((E + S) * 4);
  L.f_prefix = take((E + S + 1) * 4);
  L.h_prefix = take((E + S + 1) * 4);
  L.pool = take(2 * 4);  // item counters of the two GEMMs' shared pools
  L.dcnt = take(E * 4);  // drop mode: assignments per expert before the limit
  L.h = take(rows * (size_t)d.I * (d.fp8 ? 1 : d.esz));  // FP8: E4M3 codes of h
  L.y = take(rows * (size_t)d.H * 4);  // expert outputs are fp32
  // FP8: x's codes and the scales of x and h
  L.xq = take(d.fp8 ? T * (size_t)d.H : 0);
  L.sx = take(d.fp8 ? T * (size_t)sx_stride(d) : 0);
  L.sxr = take(d.fp8 ? grouped_scales(rows, d.H / 128) : 0);
  L.sh = take(d.fp8 ? grouped_scales(rows, d.I / 128) : 0);
  // weight block scales with rows padded to 4 bytes (used when the caller's
  // rows are not already a multiple of 4 bytes)
  L.sbg = take(d.fp8 ? (E + S) * (size_t)(d.I / 128) * pad4(d.H / 128) : 0);
  L.sbu = take(d.fp8 ? (E + S) * (size_t)(d.I / 128) * pad4(d.H / 128) : 0);
  L.sbd = take(d.fp8 ? (E + S) * (size_t)(d.H / 128) * pad4(d.I / 128) : 0);
  L.total = off;
  return L;
}

template <class P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The bf16/FP8 gate/up GEMM gathers token rows through one buffer resource
// over x (bf16) or its E4M3 codes (FP8), whose byte size must fit in 31 bits.
moe_status check_gemm_x(const Dims& d) {
  if (d.dtype != MOE_F32 && d.T * (int64_t)d.H * (d.fp8 ? 1 : 2) > 0x7FFFFFFF)
    return fail(MOE_ERR_UNSUPPORTED, "T * hidden_size * element size must be below 2 GiB (x of bf16 and FP8 layers)");
  return MOE_OK;
}

moe_status check_ws(const Dims& d, void* ws, size_t ws_bytes, Layout& L) {
  L = layout_of(d);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes, got " +
                                       std::to_string(ws_bytes));
  return MOE_OK;
}

RouteParams route_params(const Dims& d) {
  RouteParams p;
  p.T = (int)d.T;
  p.H = d.H;
  p.E = d.E;
  p.k = d.k;
  p.G = d.G;
  p.gsz = d.gsz;
  p.topk_group = d.topk_group;
  p.scoring = d.scoring;
  p.renorm = d.renorm;
  p.scale = d.scale;
  p.capacity = d.capacity;
  p.n_allowed = d.n_allowed;
  return p;
}

// ---- stages (arguments already validated) -----------------------------------

// Router: logits_in -> selection kernel; bf16 -> router GEMM (logits, or
// partial logits of K slices) then the selection kernel, which adds the
// slices and logit_bias and writes the logits to a.logits_out (or the
// workspace); fp32 -> the fused fp32 router.
hipError_t run_router(const Dims& d, RouterArgs a, const void* x, const void* w_router, void* ws, const Layout& L,
                      hipStream_t s) {
  if (a.logits_in) return timed(K_ROUTE_SELECT, s, [&] { return launch_route_select(a, s); });
  if (d.xdt != MOE_BF16) return timed(K_ROUTER, s, [&] { return launch_router(a, d.xdt, s); });
  int sps;
  const int S = router_splits(d.T, d.H, d.E, &sps);
  float* lg = a.logits_out ? a.logits_out : at<float>(ws, L.logits);
  RouterGemmArgs g{};
  g.T = (int)d.T;
  g.H = d.H;
  g.E = d.E;
  g.S = S;
  g.sps = sps;
  g.x = x;
  g.w = w_router;
  g.out = S == 1 ? lg : at<float>(ws, L.rpart);
  hipError_t e = timed(K_ROUTER, s, [&] { return launch_router_gemm(g, s); });
  if (e != hipSuccess) return e;
  a.part = g.out;
  a.nsplit = S;
  a.logits_out = lg;
  return timed(K_ROUTE_SELECT, s, [&] { return launch_route_select(a, s); });
}

// Hash routing inputs (null table: learned routing).
struct HashTable {
  const int32_t* token_ids = nullptr;
  const int32_t* tid2eid = nullptr;
  int64_t vocab = 0;
};

moe_status check_hash(const Dims& d, const int32_t* token_ids, const int32_t* tid2eid, int64_t vocab) {
  if (vocab < 0) return fail(MOE_ERR_INVALID_ARG, "vocab must be >= 0");
  if (vocab > INT64_MAX / 32) return fail(MOE_ERR_INVALID_ARG, "vocab too large");
  if (d.T > 0 && !token_ids) return fail(MOE_ERR_INVALID_ARG, "token_ids is required");
  if (d.T > 0 && vocab > 0 && !tid2eid) return fail(MOE_ERR_INVALID_ARG, "tid2eid is required when vocab > 0");
  if (d.capacity > 0 && !d.drop)
    return fail(MOE_ERR_INVALID_ARG, "hash routing has no next-best expert: a capacity needs drop_tokens = 1");
  return MOE_OK;
}

moe_status do_route(const Dims& d, const void* x, const void* w_router, const float* logit_bias,
                    const float* sel_bias, const float* logits_in, float* logits_out, int32_t* topk_idx,
                    float* topk_w, int32_t* counts, void* ws, const Layout& L, hipStream_t s,
                    const HashTable* hash = nullptr) {
  RouterArgs a{};
  if (hash) {
    a.hash = 1;
    a.token_ids = hash->token_ids;
    a.tid2eid = hash->tid2eid;
    a.vocab = hash->vocab;
  }
  a.p = route_params(d);
  a.x = x;
  a.w_router = w_router;
  a.logit_bias = logit_bias;
  a.sel_bias = sel_bias;
  a.logits_in = logits_in;
  a.logits_out = logits_out;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.counts = nullptr;
  hipError_t e;
  if (d.capacity > 0 && d.drop) {
    // drop mode: unlimited top-k and gates, then the capacity pass drops
    // late assignments in place
    a.p.capacity = 0;
    if (logits_in && logits_out) {
      e = hipMemcpyAsync(logits_out, logits_in, sizeof(float) * d.T * d.E, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "logits copy");
      a.logits_out = nullptr;
    }
    e = run_router(d, a, x, w_router, ws, L, s);
    if (e != hipSuccess) return hip_fail(e, "router kernel launch");
    // the permutation of the unlimited top-k gives every assignment its rank
    // among its expert's assignments in token order; ranks >= C are dropped
    PermuteArgs pa{};
    pa.T = (int)d.T;
    pa.E = d.E;
    pa.k = d.k;
    pa.S = d.S;
    pa.nchunks = (int)((d.T + 63) / 64);
    pa.topk_idx = topk_idx;
    pa.chunk_cnt = at<int32_t>(ws, L.chunk_cnt);
    pa.chunk_base = at<int32_t>(ws, L.chunk_base);
    pa.counts = at<int32_t>(ws, L.dcnt);
    pa.offsets = at<int32_t>(ws, L.offsets);
    pa.row_token = at<int32_t>(ws, L.row_token);
    pa.slot_row = at<int32_t>(ws, L.slot_row);
    e = timed(K_PERM_COUNT, s, [&] { return launch_perm_count(pa, s); });
    if (e == hipSuccess) e = timed(K_PERM_SCAN, s, [&] { return launch_perm_scan(pa, s); });
    if (e == hipSuccess) e = timed(K_PERM_SCATTER, s, [&] { return launch_perm_scatter(pa, s); });
    if (e != hipSuccess) return hip_fail(e, "permute launch");
    DropArgs dr{};
    dr.T = (int)d.T;
    dr.E = d.E;
    dr.k = d.k;
    dr.capacity = d.capacity;
    dr.topk_idx = topk_idx;
    dr.topk_w = topk_w;
    dr.slot_row = pa.slot_row;
    dr.offsets = pa.offsets;
    dr.full_counts = pa.counts;
    dr.counts = counts;
    e = timed(K_CAPACITY, s, [&] { return launch_drop(dr, s); });
    if (e != hipSuccess) return hip_fail(e, "drop kernel launch");
    return MOE_OK;
  }
  if (d.capacity > 0) {
    // the capacity pass reads the logits (gates of the final selection)
    float* lg = logits_out ? logits_out : at<float>(ws, L.logits);
    if (logits_in) lg = const_cast<float*>(logits_in);
    a.logits_out = logits_in ? nullptr : lg;
    a.cand = at<int32_t>(ws, L.cand);
    e = run_router(d, a, x, w_router, ws, L, s);
    if (e != hipSuccess) return hip_fail(e, "router kernel launch");
    if (logits_in && logits_out) {
      e = hipMemcpyAsync(logits_out, logits_in, sizeof(float) * d.T * d.E, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "logits copy");
    }
    CapacityArgs c{};
    c.p = a.p;
    c.logits = lg;
    c.cand = a.cand;
    c.topk_idx = topk_idx;
    c.topk_w = topk_w;
    c.counts = counts;
    e = timed(K_CAPACITY, s, [&] { return launch_capacity(c, s); });
    if (e != hipSuccess) return hip_fail(e, "capacity kernel launch");
    return MOE_OK;
  }
  if (counts) {
    e = timed(K_FILL, s, [&] { return launch_fill_i32(counts, d.E, 0, s); });
    if (e != hipSuccess) return hip_fail(e, "fill kernel launch");
    a.counts = counts;
  }
  if (logits_in && logits_out) {
    e = hipMemcpyAsync(logits_out, logits_in, sizeof(float) * d.T * d.E, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "logits copy");
    a.logits_out = nullptr;
  }
  e = run_router(d, a, x, w_router, ws, L, s);
  if (e != hipSuccess) return hip_fail(e, "router kernel launch");
  return MOE_OK;
}

moe_status do_permute(const Dims& d, const int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* row_token,
                      int32_t* slot_row, void* ws, const Layout& L, hipStream_t s) {
  PermuteArgs a{};
  a.T = (int)d.T;
  a.E = d.E;
  a.k = d.k;
  a.S = d.S;
  a.nchunks = (int)((d.T + 63) / 64);
  a.topk_idx = topk_idx;
  a.chunk_cnt = at<int32_t>(ws, L.chunk_cnt);
  a.chunk_base = at<int32_t>(ws, L.chunk_base);
  a.counts = counts;
  a.offsets = offsets;
  a.row_token = row_token;
  a.slot_row = slot_row;
  hipError_t e = timed(K_PERM_COUNT, s, [&] { return launch_perm_count(a, s); });
  if (e != hipSuccess) return hip_fail(e, "permute count launch");
  e = timed(K_PERM_SCAN, s, [&] { return launch_perm_scan(a, s); });
  if (e != hipSuccess) return hip_fail(e, "permute scan launch");
  e = timed(K_PERM_SCATTER, s, [&] { return launch_perm_scatter(a, s); });
  if (e != hipSuccess) return hip_fail(e, "permute scatter launch");
  return MOE_OK;
}

// UE8M0 block scales of FP8 expert matrices.
struct Fp8Scales {
  const uint8_t* gate;  // [E+S, I/128, H/128]
  const uint8_t* up;    // [E+S, I/128, H/128]
  const uint8_t* down;  // [E+S, H/128, I/128]
};

// Expert FFNs: y_rows [T*k+S*T, H] fp32; or, with y16 set (bf16 and FP8
// layers inside moe_forward), the routed rows [T*k, H] in bf16 to y16 and the
// shared rows [S*T, H] fp32 to y_rows.  FP8 layers (f8 set) first quantise x
// in 1 x 128 tiles into the workspace.
moe_status do_ffn(const Dims& d, const void* x, const void* w_gate, const void* w_up, const void* w_down,
                  const int32_t* offsets, const int32_t* row_token, void* y_rows, void* ws, const Layout& L,
                  hipStream_t s, void* y16 = nullptr, const Fp8Scales* f8 = nullptr) {
  hipError_t e;
  if (f8) {
    QuantArgs q{};
    q.rows = d.T;
    q.K = d.H;
    q.in = x;
    q.codes = at<uint8_t>(ws, L.xq);
    q.scales = at<uint8_t>(ws, L.sx);
    q.sstride = sx_stride(d);
    e = timed(K_QUANT, s, [&] { return launch_quantize_fp8(q, s); });
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    RowScaleArgs r{};
    r.n_rows = (int)row_space(d);
    r.nkb = d.H / 128;
    r.row_token = row_token;
    r.sx = q.scales;
    r.out = at<uint8_t>(ws, L.sxr);
    e = timed(K_ROWSCALE, s, [&] { return launch_row_scales(r, s); });
    if (e != hipSuccess) return hip_fail(e, "row scales launch");
  }
  Fp8Scales wsc{};  // weight scales as the GEMMs read them (rows of 4-byte multiples)
  if (f8) {
    auto usable = [](const uint8_t* p, int nkb) { return nkb % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (usable(f8->gate, d.H / 128) && usable(f8->up, d.H / 128) && usable(f8->down, d.I / 128)) {
      wsc = *f8;
    } else {
      ScalePackArgs pk{};
      const int64_t n_exp = d.E + d.S;
      pk.m[0] = {n_exp * (d.I / 128), d.H / 128, f8->gate, at<uint8_t>(ws, L.sbg)};
      pk.m[1] = {n_exp * (d.I / 128), d.H / 128, f8->up, at<uint8_t>(ws, L.sbu)};
      pk.m[2] = {n_exp * (d.H / 128), d.I / 128, f8->down, at<uint8_t>(ws, L.sbd)};
      e = timed(K_ROWSCALE, s, [&] { return launch_pack_scales(pk, s); });
      if (e != hipSuccess) return hip_fail(e, "scale pack launch");
      wsc = {pk.m[0].dst, pk.m[1].dst, pk.m[2].dst};
    }
  }
  const int BM = gemm_bm(d.dtype);
  ScheduleArgs sa{};
  sa.T = (int)d.T;
  sa.E = d.E;
  sa.S = d.S;
  sa.k = d.k;
  sa.BM = BM;
  sa.half_rows = gemm_half_rows(d.dtype);
  sa.offsets = offsets;
  sa.seg_start = at<int32_t>(ws, L.seg_start);
  sa.seg_len = at<int32_t>(ws, L.seg_len);
  sa.f_prefix = at<int32_t>(ws, L.f_prefix);
  sa.h_prefix = at<int32_t>(ws, L.h_prefix);
  sa.pool = at<int32_t>(ws, L.pool);
  e = timed(K_SCHEDULE, s, [&] { return launch_schedule(sa, s); });
  if (e != hipSuccess) return hip_fail(e, "schedule launch");
  const int64_t bound = gemm_mtile_bound((int)d.T, d.E, d.S, d.k, BM);
  GemmArgs g{};
  g.n_exp = d.E + d.S;
  g.seg_start = sa.seg_start;
  g.seg_len = sa.seg_len;
  g.f_prefix = sa.f_prefix;
  g.h_prefix = sa.h_prefix;
  g.row_token = row_token;
  // bf16 and FP8 kernels share each GEMM's last items between the XCDs
  // (the fp32 kernel has no LDS to broadcast the counter)
  g.pool = d.dtype != MOE_F32 ? sa.pool : nullptr;
  // (the gate/up GEMM chooses the weights' cache policy per item, from the
  // item's expert; the down GEMM per launch, below)
  void* h = at<void>(ws, L.h);
  // gate/up + SwiGLU
  g.K = d.H;
  g.N = d.I;
  g.n_tiles = d.dtype != MOE_F32 ? d.I / 128 : d.I / 32;
  g.a = x;
  g.a_bytes = (uint32_t)(d.T * d.H * (f8 ? 1 : d.esz));
  g.b0 = w_gate;
  g.b1 = w_up;
  g.c = h;
  if (f8) {
    g.a = at<uint8_t>(ws, L.xq);
    g.sa = at<uint8_t>(ws, L.sxr);
    g.n_rows = (int)row_space(d);
    g.sb0 = wsc.gate;
    g.sb1 = wsc.up;
    g.sc = at<uint8_t>(ws, L.sh);
  }
  if (bound * g.n_tiles > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "too many GEMM tiles");
  e = timed(K_GATEUP, s, [&] { return launch_gateup(g, d.dtype, bound, s); });
  if (e != hipSuccess) return hip_fail(e, "gate/up GEMM launch");
  // down
  if (g.pool) g.pool = sa.pool + 1;
  g.K = d.I;
  g.N = d.H;
  g.n_tiles = d.dtype != MOE_F32 ? d.H / 256 : d.H / 32;
  g.a = h;
  g.b0 = w_down;
  g.b1 = nullptr;
  if (f8) {
    g.sa = at<uint8_t>(ws, L.sh);
    g.n_rows = (int)row_space(d);
    g.sb0 = wsc.down;
    g.sb1 = nullptr;
    g.sc = nullptr;
  }
  g.c = y_rows;
  g.c16 = y16;
  // the down GEMM's weights stream past the caches (non-temporal copies)
  // when each weight tile is read by one item: at most BM tokens (every
  // expert segment fits one row tile: a token takes an expert at most once,
  // a shared expert has T rows), or, for bf16 weights, when the routed
  // experts average at most BM/2 rows (most fit one row tile; the shared
  // experts' tiles are then re-read from HBM, measured cheaper than sending
  // the routed weights through the caches: V3 shape down 1.43 -> 1.27 ms at
  // 512 tokens, 1.84 -> 1.80 ms at 4096; for FP8 weights it was slower)
  g.stream_b = d.T <= BM || (d.dtype == MOE_BF16 && d.T * d.k <= (int64_t)(BM / 2) * d.E) ? 1 : 0;
  // at short K (I <= 4096: 32 or fewer steps per item) the h rows' copies are
  // the ones that arrive late: three h stages and two weight stages (measured
  // on the DeepSeek-V2/V3/V4 shapes: down 2-4 % faster; at the Mixtral
  // shape's K = 14336 and when the weights stream once, 8-9 % slower)
  g.a3 = d.dtype == MOE_BF16 && !g.stream_b && d.I <= 4096 ? 1 : 0;
  g.n_routed = d.E;
  g.routed_rows = (int)(d.T * d.k);
  if (bound * g.n_tiles > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "too many GEMM tiles");
  e = timed(K_DOWN, s, [&] { return launch_down(g, d.dtype, bound, s); });
  if (e != hipSuccess) return hip_fail(e, "down GEMM launch");
  return MOE_OK;
}

// y_routed: [T*k, H] fp32, or bf16 when routed_bf16; y_shared: [S*T, H] fp32.
moe_status do_combine(const Dims& d, const void* y_routed, bool routed_bf16, const float* y_shared,
                      const int32_t* slot_row, const float* topk_w, void* out, hipStream_t s) {
  CombineArgs a{};
  a.T = (int)d.T;
  a.H = d.H;
  a.k = d.k;
  a.S = d.S;
  a.y_routed = y_routed;
  a.routed_bf16 = routed_bf16 ? 1 : 0;
  a.y_shared = y_shared;
  a.slot_row = slot_row;
  a.topk_w = topk_w;
  a.out = out;
  const hipError_t e = timed(K_COMBINE, s, [&] { return launch_combine(a, d.dtype, d.out_dtype, s); });
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

// The whole layer (learned routing, or hash routing when `hash` is set; FP8
// expert matrices when `f8` is set).
moe_status forward_impl(const Dims& d, const void* x, const void* w_router, const float* logit_bias,
                        const float* sel_bias, const void* w_gate, const void* w_up, const void* w_down, void* out,
                        int32_t* topk_idx, float* topk_w, int32_t* expert_counts, float* logits_out, void* ws,
                        size_t ws_bytes, hipStream_t s, const HashTable* hash, const Fp8Scales* f8 = nullptr) {
  moe_status st;
  if (d.fp8 != (f8 != nullptr))
    return fail(MOE_ERR_INVALID_ARG, d.fp8 ? "MOE_FP8 layers run through moe_forward_fp8"
                                           : "moe_forward_fp8 needs dtype MOE_FP8");
  if (d.T == 0) return MOE_OK;
  if (f8 && (!f8->gate || !f8->up || !f8->down)) return fail(MOE_ERR_INVALID_ARG, "NULL scale argument");
  if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return fail(MOE_ERR_INVALID_ARG, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(out))
    return fail(MOE_ERR_INVALID_ARG, "x, weights and out must be 16-byte aligned");
  st = check_gemm_x(d);
  if (st != MOE_OK) return st;
  Layout L{};
  st = check_ws(d, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* w = topk_w ? topk_w : at<float>(ws, L.w);
  int32_t* counts = expert_counts ? expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  void* y = at<void>(ws, L.y);
  st = do_route(d, x, w_router, logit_bias, sel_bias, nullptr, logits_out, idx, w, nullptr, ws, L, s, hash);
  if (st != MOE_OK) return st;
  st = do_permute(d, idx, counts, offsets, row_token, slot_row, ws, L, s);
  if (st != MOE_OK) return st;
  if (d.dtype != MOE_F32 && d.S >= 1) {
    // routed expert rows in bf16, shared expert rows in fp32, in the
    // expert-row region: with a shared expert, whose unweighted fp32 row
    // carries much of each output, the bf16 rounding of the gate-weighted
    // routed rows stays small against the output (measured: 0.0074 ->
    // 0.0090 of RMS at the DeepSeek-V3 prefill shape); without one, every
    // output is a sum of rounded rows and all rows stay fp32
    void* y16 = y;
    float* y32 = reinterpret_cast<float*>(static_cast<char*>(y) + (size_t)d.T * d.k * d.H * 2);
    st = do_ffn(d, x, w_gate, w_up, w_down, offsets, row_token, y32, ws, L, s, y16, f8);
    if (st != MOE_OK) return st;
    return do_combine(d, y16, true, y32, slot_row, w, out, s);
  }
  st = do_ffn(d, x, w_gate, w_up, w_down, offsets, row_token, y, ws, L, s, nullptr, f8);
  if (st != MOE_OK) return st;
  return do_combine(d, y, false, static_cast<const float*>(y) + (int64_t)d.T * d.k * d.H, slot_row, w, out, s);
}

}  // namespace

// ---- kernel names --------------------------------------------------------------
const char* kernel_name(int id) {
  static const char* names[K_COUNT] = {"fill",          "router",          "router_select", "capacity",
                                       "permute_count", "permute_scan",    "permute_scatter", "schedule",
                                       "gateup_swiglu", "down",            "combine",         "balance",
                                       "quantize",      "row_scales"};
  return (id >= 0 && id < K_COUNT) ? names[id] : nullptr;
}

// ---- exported ------------------------------------------------------------------
extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes) {
  Dims d;
  const moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout_of(d).total;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* logit_bias,
                     const float* sel_bias, const float* logits_in, float* logits_out, int32_t* topk_idx,
                     float* topk_w, int32_t* expert_counts, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits_in && (!x || !w_router)) return fail(MOE_ERR_INVALID_ARG, "x and w_router are required without logits_in");
  if (!logits_in && (!aligned16(x) || !aligned16(w_router)))
    return fail(MOE_ERR_INVALID_ARG, "x and w_router must be 16-byte aligned");
  if (!topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "topk_idx and topk_w are required");
  Layout L{};
  // the workspace holds the capacity candidates, and for bf16 layers the
  // router GEMM's logits and K-slice partials
  if (d.capacity > 0 || (!logits_in && d.xdt == MOE_BF16)) {
    st = check_ws(d, ws, ws_bytes, L);
    if (st != MOE_OK) return st;
  }
  return do_route(d, x, w_router, logit_bias, sel_bias, logits_in, logits_out, topk_idx, topk_w, expert_counts, ws, L,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                       void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets) return fail(MOE_ERR_INVALID_ARG, "expert_counts and expert_offsets are required");
  if (T > 0 && (!topk_idx || !row_token || !slot_row))
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, row_token and slot_row are required");
  Layout L{};
  st = check_ws(d, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // empty batch: every expert has zero rows
    hipError_t e = launch_fill_i32(expert_counts, d.E, 0, s);
    if (e == hipSuccess) e = launch_fill_i32(expert_offsets, d.E + 1, 0, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fill kernel launch");
  }
  return do_permute(d, topk_idx, expert_counts, expert_offsets, row_token, slot_row, ws, L, s);
}

moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const void* w_gate, const void* w_up,
                          const void* w_down, const int32_t* expert_offsets, const int32_t* row_token, void* y_rows,
                          void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !expert_offsets || !row_token || !y_rows)
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(y_rows))
    return fail(MOE_ERR_INVALID_ARG, "x, weights and y_rows must be 16-byte aligned");
  if (d.fp8) return fail(MOE_ERR_INVALID_ARG, "MOE_FP8 layers run through moe_expert_ffn_fp8");
  st = check_gemm_x(d);
  if (st != MOE_OK) return st;
  Layout L{};
  st = check_ws(d, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  return do_ffn(d, x, w_gate, w_up, w_down, expert_offsets, row_token, y_rows, ws, L, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_fp8(const moe_config* cfg, int64_t T, const void* x, const uint8_t* w_gate,
                              const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                              const uint8_t* s_down, const int32_t* expert_offsets, const int32_t* row_token,
                              void* y_rows, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (!d.fp8) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_fp8 needs dtype MOE_FP8");
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !s_gate || !s_up || !s_down || !expert_offsets || !row_token || !y_rows)
    return fail(MOE_ERR_INVALID_ARG, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(y_rows))
    return fail(MOE_ERR_INVALID_ARG, "x, weights and y_rows must be 16-byte aligned");
  st = check_gemm_x(d);
  if (st != MOE_OK) return st;
  Layout L{};
  st = check_ws(d, ws, ws_bytes, L);
  if (st != MOE_OK) return st;
  const Fp8Scales f8{s_gate, s_up, s_down};
  return do_ffn(d, x, w_gate, w_up, w_down, expert_offsets, row_token, y_rows, ws, L, static_cast<hipStream_t>(stream),
                nullptr, &f8);
}

moe_status moe_quantize_fp8(int64_t rows, int32_t K, const void* in, uint8_t* codes, uint8_t* scales,
                            int32_t scale_stride, void* stream) {
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows < 0");
  if (K <= 0 || K % 128 != 0) return fail(MOE_ERR_INVALID_ARG, "K must be a positive multiple of 128");
  if (scale_stride < K / 128) return fail(MOE_ERR_INVALID_ARG, "scale_stride < K/128");
  if (rows == 0) return MOE_OK;
  if (!in || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL tensor argument");
  if (!aligned16(in) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0)
    return fail(MOE_ERR_INVALID_ARG, "in must be 16-byte and codes 8-byte aligned");
  QuantArgs q{};
  q.rows = rows;
  q.K = K;
  q.in = in;
  q.codes = codes;
  q.scales = scales;
  q.sstride = scale_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(K_QUANT, s, [&] { return launch_quantize_fp8(q, s); });
  return e == hipSuccess ? MOE_OK : hip_fail(e, "quantize launch");
}

moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, const int32_t* slot_row,
                       const float* topk_w, void* out, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!y_rows || !slot_row || !topk_w || !out) return fail(MOE_ERR_INVALID_ARG, "NULL tensor argument");
  if (!aligned16(y_rows) || !aligned16(out)) return fail(MOE_ERR_INVALID_ARG, "y_rows and out must be 16-byte aligned");
  const float* shared = static_cast<const float*>(y_rows) + (int64_t)d.T * d.k * d.H;
  return do_combine(d, y_rows, false, shared, slot_row, topk_w, out, static_cast<hipStream_t>(stream));
}

moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* logit_bias,
                       const float* sel_bias, const void* w_gate, const void* w_up, const void* w_down, void* out,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_counts, float* logits_out, void* ws,
                       size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  return forward_impl(d, x, w_router, logit_bias, sel_bias, w_gate, w_up, w_down, out, topk_idx, topk_w,
                      expert_counts, logits_out, ws, ws_bytes, static_cast<hipStream_t>(stream), nullptr);
}

moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                               const float* logit_bias, const float* sel_bias, const void* w_gate, const void* w_up,
                               const void* w_down, void* out, int32_t* topk_idx, float* topk_w,
                               int32_t* expert_counts, float* logits_out, void* stream) {
  Dims d;
  const moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  if (d.fp8) return fail(MOE_ERR_INVALID_ARG, "MOE_FP8 layers run through moe_forward_fp8");
  const size_t need = layout_of(d).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "this layer and batch need " + std::to_string(need) +
                                       " bytes of workspace; the static scratch holds " +
                                       std::to_string(kScratchBytes) + ": call moe_forward with a workspace");
  if (T == 0) return MOE_OK;
  void* ws = nullptr;
  const moe_status sst = scratch_of_current_device(&ws);
  if (sst != MOE_OK) return sst;
  return forward_impl(d, x, w_router, logit_bias, sel_bias, w_gate, w_up, w_down, out, topk_idx, topk_w,
                      expert_counts, logits_out, ws, kScratchBytes, static_cast<hipStream_t>(stream), nullptr);
}

moe_status moe_forward_fp8(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                           const float* logit_bias, const float* sel_bias, const uint8_t* w_gate, const uint8_t* s_gate,
                           const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                           void* out, int32_t* topk_idx, float* topk_w, int32_t* expert_counts, float* logits_out,
                           void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  const Fp8Scales f8{s_gate, s_up, s_down};
  return forward_impl(d, x, w_router, logit_bias, sel_bias, w_gate, w_up, w_down, out, topk_idx, topk_w,
                      expert_counts, logits_out, ws, ws_bytes, static_cast<hipStream_t>(stream), nullptr, &f8);
}

moe_status moe_route_hash(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                          const float* logit_bias, const float* logits_in, float* logits_out, const int32_t* token_ids,
                          const int32_t* tid2eid, int64_t vocab, int32_t* topk_idx, float* topk_w,
                          int32_t* expert_counts, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  st = check_hash(d, token_ids, tid2eid, vocab);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits_in && (!x || !w_router)) return fail(MOE_ERR_INVALID_ARG, "x and w_router are required without logits_in");
  if (!logits_in && (!aligned16(x) || !aligned16(w_router)))
    return fail(MOE_ERR_INVALID_ARG, "x and w_router must be 16-byte aligned");
  if (!topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "topk_idx and topk_w are required");
  Layout L{};
  if (!logits_in && d.xdt == MOE_BF16) {
    st = check_ws(d, ws, ws_bytes, L);
    if (st != MOE_OK) return st;
  }
  const HashTable h{token_ids, tid2eid, vocab};
  return do_route(d, x, w_router, logit_bias, nullptr, logits_in, logits_out, topk_idx, topk_w, expert_counts, ws, L,
                  static_cast<hipStream_t>(stream), &h);
}

moe_status moe_forward_hash(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                            const float* logit_bias, const int32_t* token_ids, const int32_t* tid2eid, int64_t vocab,
                            const void* w_gate, const void* w_up, const void* w_down, void* out, int32_t* topk_idx,
                            float* topk_w, int32_t* expert_counts, float* logits_out, void* ws, size_t ws_bytes,
                            void* stream) {
  Dims d;
  moe_status st = check_config(cfg, T, d);
  if (st != MOE_OK) return st;
  st = check_hash(d, token_ids, tid2eid, vocab);
  if (st != MOE_OK) return st;
  const HashTable h{token_ids, tid2eid, vocab};
  return forward_impl(d, x, w_router, logit_bias, nullptr, w_gate, w_up, w_down, out, topk_idx, topk_w,
                      expert_counts, logits_out, ws, ws_bytes, static_cast<hipStream_t>(stream), &h);
}

moe_status moe_balance_update(const moe_config* cfg, const int32_t* expert_counts, float* sel_bias, float gamma,
                              float* share, float* stats, void* stream) {
  Dims d;
  moe_status st = check_config(cfg, 0, d);
  if (st != MOE_OK) return st;
  if (!expert_counts) return fail(MOE_ERR_INVALID_ARG, "expert_counts is required");
  if (!(gamma >= 0.0f) || gamma == INFINITY) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite and >= 0");
  BalanceArgs a{};
  a.E = d.E;
  a.counts = expert_counts;
  a.bias = sel_bias;
  a.gamma = gamma;
  a.share = share;
  a.stats = stats;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(K_BALANCE, s, [&] { return launch_balance(a, s); });
  if (e != hipSuccess) return hip_fail(e, "balance kernel launch");
  return MOE_OK;
}

static moe_status probe_mfma(int fp8, int32_t vary, int32_t blocks, int64_t iters, float* sink, double* flops,
                             void* stream) {
  if (vary != 0 && vary != 1) return fail(MOE_ERR_INVALID_ARG, "vary must be 0 or 1");
  if (blocks < 1 || blocks > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "blocks must be in [1, 2^20]");
  if (iters < 1) return fail(MOE_ERR_INVALID_ARG, "iters must be >= 1");
  if (!sink || !flops) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  *flops = (double)blocks * (double)iters * probe_mfma_flops_per_iter_block(fp8);
  const hipError_t e = launch_probe_mfma(fp8, vary, blocks, iters, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "MFMA probe launch");
}

moe_status moe_probe_mfma_bf16(int32_t vary, int32_t blocks, int64_t iters, float* sink, double* flops,
                               void* stream) {
  return probe_mfma(0, vary, blocks, iters, sink, flops, stream);
}

moe_status moe_probe_mfma_fp8(int32_t vary, int32_t blocks, int64_t iters, float* sink, double* flops,
                              void* stream) {
  return probe_mfma(1, vary, blocks, iters, sink, flops, stream);
}

moe_status moe_probe_read(int32_t mode, int32_t blocks, const void* buf, size_t bytes, float* sink, void* stream) {
  if (mode < 0 || mode > 3) return fail(MOE_ERR_INVALID_ARG, "mode must be 0, 1, 2 or 3");
  if (blocks < 1 || blocks > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "blocks must be in [1, 2^20]");
  if (!buf || !sink) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!aligned16(buf) || bytes % 16 != 0 || bytes == 0)
    return fail(MOE_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a positive multiple of 16");
  const hipError_t e =
      launch_probe_read(mode, blocks, buf, (int64_t)(bytes / 16), sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "read probe launch");
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "routing_expert_ffn_amd 0.1.0 (gfx950)"; }

moe_status moe_timing_enable(int32_t max_launches) {
  for (hipEvent_t e : g_timing.ev) hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.ids.clear();
  g_timing.max = 0;
  g_timing.used = 0;
  if (max_launches <= 0) return MOE_OK;
  g_timing.ev.resize(2 * (size_t)max_launches);
  g_timing.ids.resize(max_launches);
  for (auto& e : g_timing.ev) {
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
  }
  g_timing.max = max_launches;
  return MOE_OK;
}

moe_status moe_timing_read(double* ms, int64_t* launches, int32_t n_kernels) {
  if (!ms || !launches || n_kernels < 0) return fail(MOE_ERR_INVALID_ARG, "bad timing buffers");
  for (int i = 0; i < n_kernels; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  for (int slot = 0; slot < g_timing.used; ++slot) {
    hipError_t err = hipEventSynchronize(g_timing.ev[2 * slot + 1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
    float t = 0.0f;
    err = hipEventElapsedTime(&t, g_timing.ev[2 * slot], g_timing.ev[2 * slot + 1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
    const int id = g_timing.ids[slot];
    if (id < n_kernels) {
      ms[id] += t;
      launches[id] += 1;
    }
  }
  g_timing.used = 0;
  return MOE_OK;
}

const char* moe_kernel_name(int32_t id) { return kernel_name(id); }

moe_status moe_timing_only(int32_t kernel_id) {
  if (kernel_id < -1 || kernel_id >= K_COUNT) return fail(MOE_ERR_INVALID_ARG, "kernel_id must be -1 or a kernel id");
  g_timing.only = kernel_id;
  return MOE_OK;
}

}  // extern "C"
