// Fused router of the MoE layer for gfx950: router GEMM on the matrix cores,
// scoring, group-limited top-k and gates, one wavefront per token in
// registers; plus the serial capacity pass.
//
// What is computed ("15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家
// 怎样选 8 个"; "MoE架构揭秘", section 3.1; "GPT-4 Has 1.8 Trillion Parameters.
// It Uses 2% of Them Per Token", section 2.2):
//   l = x W_r^T (+ logit_bias)
//   softmax scoring: rank the fp32 logits; sigmoid scoring: rank
//   c = fl32(sigmoid32(l) + sel_bias); sqrt(softplus) scoring (same page,
//   section "V4：放弃潜向量，改用压缩注意力"): c = fl32(sqrtsoftplus32(l) + sel_bias)
//   hash routing (same V4 section): experts from a fixed token-id table, the
//   logits only give the gates
//   G > 1: group score = fl32(best + second best c of the group), keep the
//   topk_group best groups, rank only their experts
//   top-k in rank order (ties: lower index), gates per moe.h
//   capacity: tokens in order take their best-ranked allowed experts with room.
//
// This translation unit is compiled without floating-point contraction so the
// fp32 sigmoid and sqrt(softplus) below are exactly the documented sequences
// of roundings.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace {

// e^z for z <= 0 from correctly rounded fp32 operations: n = rint(z*log2e),
// r = z - n*ln2 (ln2 in two parts, fused), e^r by the degree-7 Taylor
// polynomial in Horner form with fused multiply-adds, result scaled by 2^n.
__device__ __forceinline__ float exp32_nonpos(float z) {
  const float t = z * 0x1.715476p+0f;
  const float n = __builtin_rintf(t);
  float r = __builtin_fmaf(-n, 0x1.62e4p-1f, z);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float q = 0x1.a01a02p-13f;
  q = __builtin_fmaf(q, r, 0x1.6c16c2p-10f);
  q = __builtin_fmaf(q, r, 0x1.111112p-7f);
  q = __builtin_fmaf(q, r, 0x1.555556p-5f);
  q = __builtin_fmaf(q, r, 0x1.555556p-3f);
  q = __builtin_fmaf(q, r, 0x1p-1f);
  q = __builtin_fmaf(q, r, 0x1p+0f);
  q = __builtin_fmaf(q, r, 0x1p+0f);
  return __builtin_amdgcn_ldexpf(q, (int)n);
}

// Selection sigmoid: logit clamped to [-80, 80] (keeps everything normal),
// 1/(1+e^-l) for l >= 0 and e^l/(1+e^l) for l < 0.
__device__ __forceinline__ float sigmoid32(float l) {
  l = l > 80.0f ? 80.0f : l;
  l = l < -80.0f ? -80.0f : l;
  if (l >= 0.0f) {
    const float e = exp32_nonpos(-l);
    const float d = 1.0f + e;
    return 1.0f / d;
  }
  const float e = exp32_nonpos(l);
  const float d = 1.0f + e;
  return e / d;
}

// log(1 + u) for 0 < u <= 1: 2 atanh(z) with z = u / (2 + u) <= 1/3; the odd
// series of atanh in w = z^2 through the w^7 term (coefficients 1/(2j+1)
// rounded to fp32), Horner form with fused multiply-adds.
__device__ __forceinline__ float log1p32_unit(float u) {
  const float d = 2.0f + u;
  const float z = u / d;
  const float w = z * z;
  float q = 0x1.111112p-4f;
  q = __builtin_fmaf(q, w, 0x1.3b13b2p-4f);
  q = __builtin_fmaf(q, w, 0x1.745d18p-4f);
  q = __builtin_fmaf(q, w, 0x1.c71c72p-4f);
  q = __builtin_fmaf(q, w, 0x1.24924ap-3f);
  q = __builtin_fmaf(q, w, 0x1.99999ap-3f);
  q = __builtin_fmaf(q, w, 0x1.555556p-2f);
  q = __builtin_fmaf(q, w, 0x1p+0f);
  const float z2 = z + z;
  return z2 * q;
}

// Selection sqrt(softplus): softplus(l) = max(l, 0) + log(1 + e^-a) with
// a = min(|l|, 80), then the correctly rounded fp32 square root.
__device__ __forceinline__ float sqrtsoftplus32(float l) {
  float a = __builtin_fabsf(l);
  a = a > 80.0f ? 80.0f : a;
  const float u = exp32_nonpos(-a);
  const float sp = (l > 0.0f ? l : 0.0f) + log1p32_unit(u);
  return __builtin_sqrtf(sp);
}

// Unbiased score of scoring 1 (sigmoid) or 2 (sqrt(softplus)).
__device__ __forceinline__ float score32(int scoring, float l) {
  return scoring == 2 ? sqrtsoftplus32(l) : sigmoid32(l);
}

__device__ __forceinline__ float ordered_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// The two largest of a multiset of ordered values, (m1 >= m2), merged with
// another such pair.
__device__ __forceinline__ void top2_merge(uint32_t& m1, uint32_t& m2, uint32_t o1, uint32_t o2) {
  const uint32_t hi = m1 > o1 ? m1 : o1, lo = m1 > o1 ? o1 : m1;
  const uint32_t r2 = m2 > o2 ? m2 : o2;
  m2 = lo > r2 ? lo : r2;
  m1 = hi;
}

template <int CTRL>
__device__ __forceinline__ void top2_step(uint32_t& m1, uint32_t& m2) {
  top2_merge(m1, m2, dpp_u32<CTRL>(m1), dpp_u32<CTRL>(m2));
}

// Selection scores of one token: lane holds experts e = j*64 + lane.
template <int NJ>
__device__ __forceinline__ void token_scores(const RouteParams& p, const float* lrow, const float* sel_bias,
                                             int lane, uint64_t (&key)[NJ]) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * MOE_WAVE + lane;
    key[j] = 0;
    if (e < p.E) {
      const float l = lrow[e];
      float c;
      if (p.scoring != 0) {
        const float s = score32(p.scoring, l);
        const float b = sel_bias ? sel_bias[e] : 0.0f;
        c = s + b;
      } else {
        c = l;
      }
      key[j] = rank_key(c, e);
    }
  }
  if (p.G <= 1) return;
  const int gsz = p.gsz;
  uint64_t kept = 0;
  if ((gsz & (gsz - 1)) == 0 && gsz >= 2 && gsz <= MOE_WAVE && p.G * gsz == p.E) {
    // power-of-two groups inside a register: the expert of (j, lane) is in
    // group j*R + lane/gsz, R = 64/gsz.  Each group's two best values are
    // merged in place across its gsz lanes (the top two of a multiset, so an
    // equal value at another index is the second best); the group score is
    // the fp32 sum of the two; lane g then takes group g's score.
    const int R = MOE_WAVE / gsz;
    float my_gs = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint32_t m1 = (uint32_t)(key[j] >> 32), m2 = 0;
      top2_step<kDppQuadXor1>(m1, m2);
      if (gsz >= 4) top2_step<kDppQuadXor2>(m1, m2);
      if (gsz >= 8) top2_step<kDppHalfMirror>(m1, m2);
      if (gsz >= 16) top2_step<kDppMirror>(m1, m2);
      if (gsz >= 32) {
        // rows (16 lanes) 0+1 and 2+3 (gsz 32), or all four (gsz 64)
        uint32_t a1 = __builtin_amdgcn_readlane(m1, 0), a2 = __builtin_amdgcn_readlane(m2, 0);
        uint32_t b1 = __builtin_amdgcn_readlane(m1, 32), b2 = __builtin_amdgcn_readlane(m2, 32);
        top2_merge(a1, a2, __builtin_amdgcn_readlane(m1, 16), __builtin_amdgcn_readlane(m2, 16));
        top2_merge(b1, b2, __builtin_amdgcn_readlane(m1, 48), __builtin_amdgcn_readlane(m2, 48));
        if (gsz == 64) {
          top2_merge(a1, a2, b1, b2);
          b1 = a1;
          b2 = a2;
        }
        m1 = lane < 32 ? a1 : b1;
        m2 = lane < 32 ? a2 : b2;
      }
      const float gs = ordered_to_float(m1) + ordered_to_float(m2);
      const float t = __shfl(gs, (lane % R) * gsz);
      if (lane / R == j) my_gs = t;
    }
    // keep the topk_group groups of highest (score, lower index) key: a
    // group is kept when fewer than topk_group keys beat it
    const uint64_t gkey = lane < p.G ? rank_key(my_gs, lane) : 0;
    int above = 0;
    for (int g = 0; g < p.G; ++g) above += readlane_u64(gkey, g) > gkey ? 1 : 0;
    kept = __ballot(lane < p.G && above < p.topk_group);
  } else {
    // group scores: best and second best key of each group (an equal value
    // at another index counts as the second best)
    float my_gs = 0.0f;
    for (int g = 0; g < p.G; ++g) {
      uint64_t b1 = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = j * MOE_WAVE + lane;
        if (key[j] && e / gsz == g && key[j] > b1) b1 = key[j];
      }
      b1 = wave_max_u64(b1);
      uint64_t b2 = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = j * MOE_WAVE + lane;
        if (key[j] && e / gsz == g && key[j] != b1 && key[j] > b2) b2 = key[j];
      }
      b2 = wave_max_u64(b2);
      const float v1 = ordered_to_float((uint32_t)(b1 >> 32));
      const float v2 = ordered_to_float((uint32_t)(b2 >> 32));
      const float gs = v1 + v2;
      if (lane == g) my_gs = gs;
    }
    uint64_t gkey = lane < p.G ? rank_key(my_gs, lane) : 0;
    for (int i = 0; i < p.topk_group; ++i) {
      const uint64_t m = wave_max_u64(gkey);
      const int g = key_expert(m);
      kept |= 1ull << g;
      if (lane == g) gkey = 0;
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * MOE_WAVE + lane;
    if (key[j] && !((kept >> (e / gsz)) & 1ull)) key[j] = 0;
  }
}

// Gate of the expert lane i holds for slot i (lanes >= k or empty slots: 0).
template <int NJ>
__device__ __forceinline__ float token_gate(const RouteParams& p, const float* lrow, int my_e, int lane) {
  const bool mine = lane < p.k && my_e >= 0;
  float g = 0.0f;
  if (p.scoring != 0) {
    const float s = mine ? score32(p.scoring, lrow[my_e]) : 0.0f;
    if (p.renorm) {
      const float tot = wave_sum_f32(s);
      g = mine ? s / tot : 0.0f;
    } else {
      g = s;
    }
  } else if (p.renorm) {
    // softmax renormalised over the selection = softmax of the chosen logits
    const float l = mine ? lrow[my_e] : 0.0f;
    const float m0 = wave_max_f32(mine ? l : -INFINITY);
    const float ex = mine ? expf(l - m0) : 0.0f;
    const float tot = wave_sum_f32(ex);
    g = mine ? ex / tot : 0.0f;
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = j * MOE_WAVE + lane;
      if (e < p.E) mx = fmaxf(mx, lrow[e]);
    }
    mx = wave_max_f32(mx);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = j * MOE_WAVE + lane;
      if (e < p.E) z += expf(lrow[e] - mx);
    }
    z = wave_sum_f32(z);
    g = mine ? expf(lrow[my_e] - mx) / z : 0.0f;
  }
  return g * p.scale;
}

// Top-k of one token by repeated wavefront argmax; lane i ends with slot i.
template <int NJ>
__device__ __forceinline__ int token_topk(const RouteParams& p, uint64_t (&key)[NJ], int lane) {
  int my_e = -1;
  for (int i = 0; i < p.k; ++i) {
    uint64_t local = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) local = key[j] > local ? key[j] : local;
    const uint64_t m = wave_max_u64(local);
    const int e = m ? key_expert(m) : -1;
    if (lane == i) my_e = e;
    if (e >= 0 && (e & (MOE_WAVE - 1)) == lane) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (j == (e >> 6)) key[j] = 0;
    }
  }
  return my_e;
}

// The value of lane ^ s (s < 64; s is a constant once the sort is
// unrolled): DPP inside rows of 16 lanes for s <= 8 (row_ror:n gives lane i
// the value of lane (i - n) mod 16, so s = 4 takes the rotations by 12 and by
// 4 for the lanes below and above their partner, s = 8 the rotation by 8),
// a bpermute across rows.
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v, int lane, int s) {
  if (s == 1) return dpp_u64<kDppQuadXor1>(v);
  if (s == 2) return dpp_u64<kDppQuadXor2>(v);
  if (s == 4) {
    const uint64_t up = dpp_u64<0x12C>(v), down = dpp_u64<0x124>(v);
    return (lane & 4) ? down : up;
  }
  if (s == 8) return dpp_u64<0x128>(v);
  return __shfl_xor(v, s);
}

// Descending bitonic sort of the 64*NJ keys of the wavefront; element
// i = j*64 + lane ends holding rank i.
template <int NJ>
__device__ __forceinline__ void wave_bitonic_desc(uint64_t (&key)[NJ], int lane) {
  constexpr int N = NJ * MOE_WAVE;
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t nk[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i = j * MOE_WAVE + lane;
        uint64_t other;
        if (stride >= MOE_WAVE)
          other = key[j ^ (stride / MOE_WAVE)];
        else
          other = lane_xor_u64(key[j], lane, stride);
        const bool lower = (i & stride) == 0;
        const bool desc = (i & size) == 0;
        const bool keep_max = lower == desc;
        const uint64_t mx = key[j] > other ? key[j] : other;
        const uint64_t mn = key[j] > other ? other : key[j];
        nk[j] = keep_max ? mx : mn;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) key[j] = nk[j];
    }
  }
}

// Route token t from its logits row (lane holds experts j*64 + lane): group
// limit and top-k with gates, or in capacity mode the ranked candidates.
template <int NJ>
__device__ __forceinline__ void route_token(const RouterArgs& a, const float* lrow, int t, int lane) {
  const RouteParams& p = a.p;
  if (a.hash) {
    // hash routing: row token_ids[t] of the table chooses, the logits only
    // weight; an entry out of [0, E) or repeating an earlier entry of the
    // row, and every entry of an id outside the table, leave the slot empty
    const int64_t id = a.token_ids[t];
    const bool in_table = id >= 0 && id < a.vocab;
    const int raw = (lane < p.k && in_table) ? a.tid2eid[id * p.k + lane] : -1;
    int my_e = (raw >= 0 && raw < p.E) ? raw : -1;
    for (int j = 0; j + 1 < p.k; ++j) {
      const int rj = __shfl(raw, j);
      if (j < lane && rj == my_e) my_e = -1;
    }
    const float g = token_gate<NJ>(p, lrow, my_e, lane);
    if (lane < p.k) {
      a.topk_idx[(int64_t)t * p.k + lane] = my_e;
      a.topk_w[(int64_t)t * p.k + lane] = my_e >= 0 ? g : 0.0f;
      if (a.counts && my_e >= 0) atomicAdd(&a.counts[my_e], 1);
    }
    return;
  }
  uint64_t key[NJ];
  token_scores<NJ>(p, lrow, a.sel_bias, lane, key);
  if (p.capacity > 0) {
    wave_bitonic_desc<NJ>(key, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i = j * MOE_WAVE + lane;
      if (i < p.n_allowed) a.cand[(int64_t)t * p.n_allowed + i] = key_expert(key[j]);
    }
  } else {
    const int my_e = token_topk<NJ>(p, key, lane);
    const float g = token_gate<NJ>(p, lrow, my_e, lane);
    if (lane < p.k) {
      a.topk_idx[(int64_t)t * p.k + lane] = my_e;
      a.topk_w[(int64_t)t * p.k + lane] = my_e >= 0 ? g : 0.0f;
      if (a.counts && my_e >= 0) atomicAdd(&a.counts[my_e], 1);
    }
  }
}

// ---- bf16 router: GEMM kernel, then one wavefront per token -----------------

// Router GEMM tile: 64 tokens x 128*NB experts (wave w: experts w*32*NB ..,
// all 64 tokens, 2 x NB MFMA blocks of 32x32) over one K slice.  x rows and
// weight rows are staged in LDS in the swizzled 128-byte row format, two
// stages, the next step copied while the current one computes.
template <int NB>
__global__ __launch_bounds__(256) void router_gemm_kernel(RouterGemmArgs a) {
  constexpr int EP = 128 * NB;
  constexpr int A_BYTES = 64 * 128;
  constexpr int STAGE = A_BYTES + EP * 128;
  constexpr int B_PER_WAVE = EP / 8 / 4;
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 64;
  const int nk = a.H / 64;
  const int kb = blockIdx.y * a.sps, ke = min(nk, kb + a.sps);
  const int lrow = lane >> 3;
  const bf16* x = static_cast<const bf16*>(a.x);
  const bf16* w = static_cast<const bf16*>(a.w);
  uint32_t aoff[2], boff[B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave * 2 + i) * 8 + lrow;
    const int tok = min(t0 + r, a.T - 1);
    aoff[i] = (uint32_t)tok * (uint32_t)a.H + ((lane & 7) ^ swz_of_row(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_PER_WAVE; ++i) {
    const int r = (wave * B_PER_WAVE + i) * 8 + lrow;
    const int e = min(r, a.E - 1);
    boff[i] = (uint32_t)e * (uint32_t)a.H + ((lane & 7) ^ swz_of_row(r)) * 8;
  }
  char* const a_dst = lds + wave * 2 * 1024;
  char* const b_dst = lds + A_BYTES + wave * B_PER_WAVE * 1024;
  f32x16 acc[2][NB];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
  // fragment rows are congruent to lane mod 16: the swizzled slot depends on
  // the lane and the 16-wide sub-step only
  int slot[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) slot[kk] = ((kk * 2 + (lane >> 5)) ^ swz_of_row(lane & 15)) << 4;
  const int arow = (lane & 31) * 128;
  const int brow = A_BYTES + (wave * 32 * NB + (lane & 31)) * 128;

  if (kb < ke) {
#pragma unroll
    for (int i = 0; i < 2; ++i) copy16(x + kb * 64 + aoff[i], a_dst + i * 1024);
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) copy16(w + kb * 64 + boff[i], b_dst + i * 1024);
  }
  for (int ks = kb; ks < ke; ++ks) {
    const int cur = (ks - kb) & 1;
    // step ks has landed for every wave, and every wave is done with the
    // other stage (read in the previous step)
    wait_vmem_upto<0>();
    __syncthreads();
    if (ks + 1 < ke) {
      const int k1 = (ks + 1) * 64;
#pragma unroll
      for (int i = 0; i < 2; ++i) copy16(x + k1 + aoff[i], a_dst + (cur ^ 1) * STAGE + i * 1024);
#pragma unroll
      for (int i = 0; i < B_PER_WAVE; ++i) copy16(w + k1 + boff[i], b_dst + (cur ^ 1) * STAGE + i * 1024);
    }
    const char* st = lds + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 fa[2], fb[NB];
#pragma unroll
      for (int m = 0; m < 2; ++m) fa[m] = *reinterpret_cast<const bf16x8*>(st + arow + m * 32 * 128 + slot[kk]);
#pragma unroll
      for (int n = 0; n < NB; ++n) fb[n] = *reinterpret_cast<const bf16x8*>(st + brow + n * 32 * 128 + slot[kk]);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[n], acc[m][n], 0, 0, 0);
    }
  }
  float* out = a.out + (int64_t)blockIdx.y * a.T * a.E;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int e = wave * 32 * NB + n * 32 + (lane & 31);
    if (e >= a.E) continue;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (tok < a.T) out[(int64_t)tok * a.E + e] = acc[m][n][r];
      }
  }
}

// Router GEMM for large batches: 128 tokens x 128*NB experts per workgroup
// (wave w: experts w*32*NB .., all 128 tokens, 4 x NB MFMA blocks), one
// workgroup per compute unit.  x is the operand streamed from HBM, so it
// gets the deeper pipeline (and the non-temporal policy: each x byte is
// read by one workgroup): four x stages (copied three steps ahead) and
// three weight stages (two steps ahead; the weights are re-read from L2),
// 160 KB of LDS for NB = 2.
constexpr int kRgTokens = 128, kRgAStages = 4, kRgBStages = 3;

template <int NB>
__global__ __launch_bounds__(256) void router_gemm_big_kernel(RouterGemmArgs a) {
  constexpr int EP = 128 * NB;
  constexpr int A_STAGE = kRgTokens * 128, B_STAGE = EP * 128;
  constexpr int A_PER_WAVE = kRgTokens / 8 / 4, B_PER_WAVE = EP / 8 / 4;
  constexpr int MB = kRgTokens / 32;
  __shared__ __attribute__((aligned(1024))) char lds[kRgAStages * A_STAGE + kRgBStages * B_STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRgTokens;
  const int nk = a.H / 64;
  const int kb = blockIdx.y * a.sps, ke = min(nk, kb + a.sps);
  const int lrow = lane >> 3;
  const bf16* x = static_cast<const bf16*>(a.x);
  const bf16* w = static_cast<const bf16*>(a.w);
  uint32_t aoff[A_PER_WAVE], boff[B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int r = (wave * A_PER_WAVE + i) * 8 + lrow;
    const int tok = min(t0 + r, a.T - 1);
    aoff[i] = (uint32_t)tok * (uint32_t)a.H + ((lane & 7) ^ swz_of_row(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_PER_WAVE; ++i) {
    const int r = (wave * B_PER_WAVE + i) * 8 + lrow;
    const int e = min(r, a.E - 1);
    boff[i] = (uint32_t)e * (uint32_t)a.H + ((lane & 7) ^ swz_of_row(r)) * 8;
  }
  char* const a_dst = lds + wave * A_PER_WAVE * 1024;
  char* const b_dst = lds + kRgAStages * A_STAGE + wave * B_PER_WAVE * 1024;
  // copies of iteration i (i may precede kb: the prologue): x of step i+3
  // and weights of step i+2, each when inside the slice
  auto issue = [&](int i) {
    const int ka = i + 3, kw = i + 2;
    if (ka < ke) {
#pragma unroll
      for (int q = 0; q < A_PER_WAVE; ++q)
        copy16_nt(x + ka * 64 + aoff[q], a_dst + (ka % kRgAStages) * A_STAGE + q * 1024);
    }
    if (kw >= kb && kw < ke) {
#pragma unroll
      for (int q = 0; q < B_PER_WAVE; ++q) copy16(w + kw * 64 + boff[q], b_dst + (kw % kRgBStages) * B_STAGE + q * 1024);
    }
  };
  f32x16 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
  int slot[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) slot[kk] = ((kk * 2 + (lane >> 5)) ^ swz_of_row(lane & 15)) << 4;
  const int arow = (lane & 31) * 128;
  const int brow = (wave * 32 * NB + (lane & 31)) * 128;

  for (int i = kb - 3; i < kb; ++i) issue(i);
  for (int ks = kb; ks < ke; ++ks) {
    // in issue order, the copies after the weights of step ks are x of step
    // ks+2 and weights of step ks+1 (when inside the slice): wait until only
    // those are in flight, so x and weights of step ks have landed; the
    // barrier then also frees the stages read in step ks-1
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of step ks-1 are done
    if (ks + 2 < ke)
      wait_vmem_upto<A_PER_WAVE + B_PER_WAVE>();
    else if (ks + 1 < ke)
      wait_vmem_upto<B_PER_WAVE>();
    else
      wait_vmem_upto<0>();
    __builtin_amdgcn_s_barrier();
    issue(ks);
    const char* sa = lds + (ks % kRgAStages) * A_STAGE;
    const char* sb = lds + kRgAStages * A_STAGE + (ks % kRgBStages) * B_STAGE;
    // fragments of sub-step kk+1 are read while sub-step kk's MFMAs run
    bf16x8 fa[2][MB], fb[2][NB];
    auto read = [&](int kk, bf16x8(&ra)[MB], bf16x8(&rb)[NB]) {
#pragma unroll
      for (int m = 0; m < MB; ++m) ra[m] = *reinterpret_cast<const bf16x8*>(sa + arow + m * 32 * 128 + slot[kk]);
#pragma unroll
      for (int n = 0; n < NB; ++n) rb[n] = *reinterpret_cast<const bf16x8*>(sb + brow + n * 32 * 128 + slot[kk]);
    };
    read(0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][m], fb[kk & 1][n], acc[m][n], 0, 0, 0);
      if (kk < 3) {
        // one fragment read after each MFMA (left alone, the scheduler puts
        // all reads first and waits for them)
        constexpr int NR = MB + NB, NM = MB * NB;
#pragma unroll
        for (int i = 0; i < (NR < NM ? NR : NM); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
        if (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  float* out = a.out + (int64_t)blockIdx.y * a.T * a.E;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int e = wave * 32 * NB + n * 32 + (lane & 31);
    if (e >= a.E) continue;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (tok < a.T) out[(int64_t)tok * a.E + e] = acc[m][n][r];
      }
  }
}

// Selection: one wavefront per token.  The token's logits are the sum of its
// nsplit partial rows (in slice order) plus logit_bias, or logits_in as
// given; they are written to logits_out when set, kept in LDS, and routed.
template <int NJ>
__global__ __launch_bounds__(256) void route_select_kernel(RouterArgs a) {
  __shared__ float lds_rows[4][NJ * MOE_WAVE];
  const RouteParams& p = a.p;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.T) return;
  float* lrow = lds_rows[wave];
  const int64_t stride = (int64_t)p.T * p.E;
  if (!a.logits_in && a.nsplit > 1 && (p.E & 3) == 0 && (reinterpret_cast<uintptr_t>(a.part) & 15) == 0) {
    // several K slices: lane l adds the slices of experts 4*(l + 64*q) .. +3
    // with 16-byte loads, slices in order, eight loads in flight
    for (int e0 = 4 * lane; e0 < p.E; e0 += 4 * MOE_WAVE) {
      const float* src = a.part + (int64_t)t * p.E + e0;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int sl = 0; sl < a.nsplit; sl += 8) {
        f32x4 q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (sl + i < a.nsplit) q[i] = *reinterpret_cast<const f32x4*>(src + (sl + i) * stride);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (sl + i < a.nsplit) v += q[i];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = v[c];
        if (a.logit_bias) x += a.logit_bias[e0 + c];
        lrow[e0 + c] = x;
        if (a.logits_out) a.logits_out[(int64_t)t * p.E + e0 + c] = x;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = j * MOE_WAVE + lane;
      if (e >= p.E) continue;
      float v;
      if (a.logits_in) {
        v = a.logits_in[(int64_t)t * p.E + e];
      } else {
        v = 0.0f;
        for (int sl = 0; sl < a.nsplit; ++sl) v += a.part[(int64_t)t * p.E + e + sl * stride];
        if (a.logit_bias) v += a.logit_bias[e];
      }
      lrow[e] = v;
      if (a.logits_out) a.logits_out[(int64_t)t * p.E + e] = v;
    }
  }
  // the row is read across lanes below: the wave's LDS writes complete first
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  route_token<NJ>(a, lrow, t, lane);
}

// ---- fp32 layers: fused router ------------------------------------------------

constexpr int kRouterTokens = 32;

// One workgroup: 32 tokens x all experts.  The GEMM runs on 32x32 MFMA tiles
// (wave w owns expert blocks w, w+4, ...), the tile of logits goes to LDS,
// then each wave routes tokens w, w+4, ... .
template <typename Tin, int NJ>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  extern __shared__ float lds_logits[];
  constexpr int EP = NJ * MOE_WAVE;
  constexpr int NB = (2 * NJ + 3) / 4;  // 32-wide expert blocks per wave
  const RouteParams& p = a.p;
  const int t0 = blockIdx.x * kRouterTokens;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  if (a.logits_in == nullptr) {
    f32x16 acc[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    const int tok = min(t0 + (lane & 31), p.T - 1);
    const Tin* x = static_cast<const Tin*>(a.x);
    const Tin* w = static_cast<const Tin*>(a.w_router);
    if constexpr (sizeof(Tin) == 2) {
      const Tin* xa = x + (int64_t)tok * p.H + (lane >> 5) * 8;
      const Tin* wb[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int e = min((wave + 4 * q) * 32 + (lane & 31), p.E - 1);
        wb[q] = w + (int64_t)e * p.H + (lane >> 5) * 8;
      }
#pragma unroll 4
      for (int k0 = 0; k0 < p.H; k0 += 16) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xa + k0);
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          if ((wave + 4 * q) * 32 < p.E) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wb[q] + k0);
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[q], 0, 0, 0);
          }
        }
      }
    } else {
      const float* xa = reinterpret_cast<const float*>(x) + (int64_t)tok * p.H + (lane >> 5);
      const float* wb[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int e = min((wave + 4 * q) * 32 + (lane & 31), p.E - 1);
        wb[q] = reinterpret_cast<const float*>(w) + (int64_t)e * p.H + (lane >> 5);
      }
      for (int k0 = 0; k0 < p.H; k0 += 2) {
        const float av = xa[k0];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          if ((wave + 4 * q) * 32 < p.E) acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, wb[q][k0], acc[q], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int col = (wave + 4 * q) * 32 + (lane & 31);
      if ((wave + 4 * q) * 32 >= EP) continue;
      const float lb = (a.logit_bias && col < p.E) ? a.logit_bias[col] : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        lds_logits[row * EP + col] = acc[q][r] + lb;
      }
    }
  } else {
    for (int i = threadIdx.x; i < kRouterTokens * EP; i += blockDim.x) {
      const int r = i / EP, c = i % EP;
      const int t = t0 + r;
      lds_logits[i] = (t < p.T && c < p.E) ? a.logits_in[(int64_t)t * p.E + c] : 0.0f;
    }
  }
  __syncthreads();

  if (a.logits_out) {
    for (int i = threadIdx.x; i < kRouterTokens * p.E; i += blockDim.x) {
      const int r = i / p.E, c = i % p.E;
      const int t = t0 + r;
      if (t < p.T) a.logits_out[(int64_t)t * p.E + c] = lds_logits[r * EP + c];
    }
  }

  for (int r = wave; r < kRouterTokens; r += 4) {
    const int t = t0 + r;
    if (t >= p.T) break;
    route_token<NJ>(a, lds_logits + r * EP, t, lane);
  }
}

// Capacity pass for small batches (a serial walk; cheaper than rounds when
// experts fill about as often as tokens arrive), one workgroup of kCapWaves
// wavefronts, tokens in chunks of `chunk`: every thread copies the chunk's ranked candidates to LDS; wave 0
// then serves the chunk's tokens in index order (lane r of a step looks at
// rank base+r; candidates with room are taken in rank order until k are
// chosen; counts live in LDS); all threads store the chunk's selections.
constexpr int kCapWaves = 8;

template <int NJ>
__global__ __launch_bounds__(kCapWaves * 64) void capacity_serial_kernel(CapacityArgs a, int chunk) {
  extern __shared__ int32_t lds_cap[];
  const RouteParams& p = a.p;
  const int NA = p.n_allowed;
  int32_t* cnt = lds_cap;                   // [E]
  int32_t* cand = cnt + p.E;                // [chunk][NA]
  int32_t* sel = cand + chunk * NA;         // [chunk][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < p.E; e += kCapWaves * 64) cnt[e] = 0;
  for (int t0 = 0; t0 < p.T; t0 += chunk) {
    const int nt = min(chunk, p.T - t0);
    __syncthreads();  // previous chunk's gates are done with sel
    {
      // eight loads in flight per thread (a load, then its LDS store, one
      // at a time would put a memory round trip per element on the chain)
      const int n = nt * NA;
      const int32_t* src = a.cand + (int64_t)t0 * NA;
      for (int i0 = tid; i0 < n; i0 += 8 * kCapWaves * 64) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * kCapWaves * 64, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * kCapWaves * 64 < n) cand[i0 + u * kCapWaves * 64] = v[u];
      }
    }
    __syncthreads();
    if (wave == 0) {
      // the first 64 ranked candidates of 8 tokens are read ahead into
      // registers; the serial chain per token is then one LDS gather of the
      // counts, a ballot and the count updates
      for (int tb = 0; tb < nt; tb += 8) {
        int c0[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c0[i] = lane < NA ? cand[min(tb + i, nt - 1) * NA + lane] : -1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tt = tb + i;
          if (tt >= nt) break;
          const int32_t* c = cand + tt * NA;
          int32_t* s = sel + tt * p.k;
          int got = 0;
          for (int base = 0; base < NA && got < p.k; base += MOE_WAVE) {
            const int r = base + lane;
            const int e = base == 0 ? c0[i] : (r < NA ? c[r] : -1);
            const bool room = e >= 0 && cnt[e] < p.capacity;
            const uint64_t m = __ballot(room);
            const int need = p.k - got;
            const int pre = __popcll(m & ((1ull << lane) - 1ull));
            if (room && pre < need) {
              atomicAdd(&cnt[e], 1);
              s[got + pre] = e;
            }
            const int avail = __popcll(m);
            got += avail < need ? avail : need;
          }
          if (lane >= got && lane < p.k) s[lane] = -1;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < nt * p.k; i += kCapWaves * 64) a.topk_idx[(int64_t)t0 * p.k + i] = sel[i];
  }
  __syncthreads();
  if (a.counts)
    for (int e = tid; e < p.E; e += kCapWaves * 64) a.counts[e] = cnt[e];
}

// Capacity pass (first come, first served in token order: each token takes
// its best-ranked allowed experts that hold fewer than C tokens), one
// workgroup, exact, in rounds over blocks of up to 64 tokens:
//   1. every token of the block picks its first k candidates among the
//      experts not full at the start of the round (8 lanes per token, the
//      counts in LDS);
//   2. per expert, a 64-bit mask of the block's tokens that picked it;
//   3. a token's picks are final when each picked expert still has room
//      after the block's earlier picks (count + popcount of the mask below
//      the token < C): experts only fill, so its first k candidates among
//      the experts with room at the round start are then exactly its first k
//      among those with room when it is served.  The first token that fails
//      (never the block's first) ends the round;
//   4. the tokens before it are committed (counts += their picks) and the
//      next round starts at it.
// A round commits 64 tokens unless an expert fills inside the block, which
// happens at most once per expert, so there are at most T/64 + E rounds.
// The gates follow in capacity_gates_kernel, one wavefront per token.  (Drop
// mode needs no pass at all: see drop_kernel in permute.hip.)
constexpr int kCapThreads = 512;
constexpr int kCapBlock = 64;

template <int NJ>
__global__ __launch_bounds__(kCapThreads) void capacity_kernel(CapacityArgs a) {
  extern __shared__ int32_t lds_cap[];
  const RouteParams& p = a.p;
  const int E = p.E, k = p.k, NA = p.n_allowed, C = p.capacity;
  int32_t* cnt = lds_cap;                                        // [E]
  uint64_t* mask = reinterpret_cast<uint64_t*>(cnt + ((E + 1) & ~1));  // [E]
  int32_t* tent = reinterpret_cast<int32_t*>(mask + E);          // [64][k]
  int32_t* t_end = tent + kCapBlock * k;                          // [1]
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < E; e += kCapThreads) {
    cnt[e] = 0;
    mask[e] = 0;
  }
  __syncthreads();
  for (int t0 = 0; t0 < p.T;) {
    const int nb = min(kCapBlock, p.T - t0);
    // 1. picks among the experts with room at the round start
    const int tt = tid >> 3, sub = tid & 7;
    if (tt < nb) {
      const int32_t* c = a.cand + (int64_t)(t0 + tt) * NA;
      int got = 0;
      for (int base = 0; got < k && base < NA; base += 8) {
        const int r = base + sub;
        const int e = r < NA ? c[r] : -1;
        const bool room = e >= 0 && cnt[e] < C;
        const uint32_t m8 = (uint32_t)(__ballot(room) >> (lane & ~7)) & 0xFFu;
        const int need = k - got;
        const int pre = __popc(m8 & ((1u << sub) - 1u));
        if (room && pre < need) tent[tt * k + got + pre] = e;
        got += min(__popc(m8), need);
      }
      for (int j = got + sub; j < k; j += 8) tent[tt * k + j] = -1;
    }
    __syncthreads();
    // 2. per-expert masks of the block's picks
    for (int i = tid; i < nb * k; i += kCapThreads) {
      const int e = tent[i];
      if (e >= 0) atomicOr((unsigned long long*)&mask[e], 1ull << (i / k));
    }
    __syncthreads();
    // 3. the first token whose picks do not all still have room
    if (tid < kCapBlock) {
      bool bad = false;
      if (tid < nb) {
        const uint64_t below = (1ull << tid) - 1ull;
        for (int j = 0; j < k; ++j) {
          const int e = tent[tid * k + j];
          if (e >= 0 && cnt[e] + __popcll(mask[e] & below) >= C) bad = true;
        }
      }
      const uint64_t bm = __ballot(bad);
      if (tid == 0) *t_end = bm ? __ffsll((long long)bm) - 1 : nb;
    }
    __syncthreads();
    // 4. commit the tokens before it, clear the masks for the next round
    const int ne = *t_end;
    const uint64_t keep = ne >= 64 ? ~0ull : (1ull << ne) - 1ull;
    for (int e = tid; e < E; e += kCapThreads) {
      cnt[e] += __popcll(mask[e] & keep);
      mask[e] = 0;
    }
    for (int i = tid; i < ne * k; i += kCapThreads) a.topk_idx[(int64_t)t0 * k + i] = tent[i];
    t0 += ne;
    __syncthreads();
  }
  if (a.counts)
    for (int e = tid; e < E; e += kCapThreads) a.counts[e] = cnt[e];
}

// Gates of the final (capacity-limited) selection, one wavefront per token.
template <int NJ>
__global__ __launch_bounds__(256) void capacity_gates_kernel(CapacityArgs a) {
  const RouteParams& p = a.p;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int my_e = lane < p.k ? a.topk_idx[(int64_t)t * p.k + lane] : -1;
  const float g = token_gate<NJ>(p, a.logits + (int64_t)t * p.E, my_e, lane);
  if (lane < p.k) a.topk_w[(int64_t)t * p.k + lane] = my_e >= 0 ? g : 0.0f;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <typename Tin, int NJ>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t s) {
  const int grid = (a.p.T + kRouterTokens - 1) / kRouterTokens;
  const size_t lds = sizeof(float) * kRouterTokens * NJ * MOE_WAVE;
  hipLaunchKernelGGL((router_kernel<Tin, NJ>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_router_d(const RouterArgs& a, hipStream_t s) {
  const int nj = (a.p.E + MOE_WAVE - 1) / MOE_WAVE;
  if (nj <= 1) return launch_router_t<Tin, 1>(a, s);
  if (nj <= 2) return launch_router_t<Tin, 2>(a, s);
  if (nj <= 4) return launch_router_t<Tin, 4>(a, s);
  return launch_router_t<Tin, 8>(a, s);
}

template <int NB>
hipError_t launch_router_gemm_t(const RouterGemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)a.S);
  hipLaunchKernelGGL((router_gemm_kernel<NB>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NJ>
hipError_t launch_route_select_t(const RouterArgs& a, hipStream_t s) {
  const int grid = (a.p.T + 3) / 4;
  hipLaunchKernelGGL((route_select_kernel<NJ>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NJ>
hipError_t launch_capacity_t(const CapacityArgs& a, hipStream_t s) {
  if (a.p.T < 8 * a.p.E) {
    // small batch: serial walk.  chunk: candidates and selections of as many
    // tokens as fit, with the counts, in 64 KB of LDS (n_allowed <= E <= 512,
    // k <= 32)
    const int NA = a.p.n_allowed;
    const int chunk = std::max(1, std::min(a.p.T, 15360 / (NA + a.p.k)));
    const size_t lds = sizeof(int32_t) * ((size_t)a.p.E + (size_t)chunk * NA + (size_t)chunk * a.p.k);
    hipLaunchKernelGGL((capacity_serial_kernel<NJ>), dim3(1), dim3(kCapWaves * 64), lds, s, a, chunk);
  } else {
    // rounds: counts, masks, the block's picks and the round's end (at most
    // 14 KB)
    const size_t lds = sizeof(int32_t) * (size_t)((a.p.E + 1) & ~1) + sizeof(uint64_t) * a.p.E +
                       sizeof(int32_t) * ((size_t)kCapBlock * a.p.k + 1);
    hipLaunchKernelGGL((capacity_kernel<NJ>), dim3(1), dim3(kCapThreads), lds, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((capacity_gates_kernel<NJ>), dim3((a.p.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, int dtype, hipStream_t s) {
  if (a.p.T <= 0) return hipSuccess;
  return dtype == 1 ? launch_router_d<bf16>(a, s) : launch_router_d<float>(a, s);
}

// Large batches (at least 64 tiles of 128 tokens, at most 256 experts) take
// the 128-token kernel, one workgroup per compute unit.
static bool router_big_tiles(int64_t T, int E) { return E <= 256 && (T + kRgTokens - 1) / kRgTokens >= 64; }

int router_splits(int64_t T, int H, int E, int* sps) {
  // enough (token tile, K slice) workgroups to fill the compute units: the
  // GEMM streams x from HBM, so its speed is the bytes in flight per CU.
  // 64-token tiles at two workgroups per CU (80 KB of LDS each, one step of
  // prefetch), or 128-token tiles at one (three steps of x in flight); K is
  // split into slices of whole 64-wide steps, at most 32 slices
  const int nk = H / 64;
  const bool big = router_big_tiles(T, E);
  const int64_t tiles = big ? (T + kRgTokens - 1) / kRgTokens : (T + 63) / 64;
  const int64_t want = big ? 256 : 512;
  int S = 1;
  if (tiles < want) S = (int)std::min<int64_t>((want + tiles - 1) / tiles, 32);
  S = std::min(S, nk);
  const int per = (nk + S - 1) / S;
  *sps = per;
  return (nk + per - 1) / per;
}

template <int NB>
hipError_t launch_router_gemm_big_t(const RouterGemmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T + kRgTokens - 1) / kRgTokens), (unsigned)a.S);
  hipLaunchKernelGGL((router_gemm_big_kernel<NB>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const RouterGemmArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (router_big_tiles(a.T, a.E)) return a.E <= 128 ? launch_router_gemm_big_t<1>(a, s) : launch_router_gemm_big_t<2>(a, s);
  if (a.E <= 128) return launch_router_gemm_t<1>(a, s);
  if (a.E <= 256) return launch_router_gemm_t<2>(a, s);
  return launch_router_gemm_t<4>(a, s);
}

hipError_t launch_route_select(const RouterArgs& a, hipStream_t s) {
  if (a.p.T <= 0) return hipSuccess;
  const int nj = (a.p.E + MOE_WAVE - 1) / MOE_WAVE;
  if (nj <= 1) return launch_route_select_t<1>(a, s);
  if (nj <= 2) return launch_route_select_t<2>(a, s);
  if (nj <= 4) return launch_route_select_t<4>(a, s);
  return launch_route_select_t<8>(a, s);
}

hipError_t launch_capacity(const CapacityArgs& a, hipStream_t s) {
  if (a.p.T <= 0) return hipSuccess;
  const int nj = (a.p.E + MOE_WAVE - 1) / MOE_WAVE;
  if (nj <= 1) return launch_capacity_t<1>(a, s);
  if (nj <= 2) return launch_capacity_t<2>(a, s);
  if (nj <= 4) return launch_capacity_t<4>(a, s);
  return launch_capacity_t<8>(a, s);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}
