// Grouped expert GEMMs of the MoE layer for gfx950.
//
// Each expert is a SwiGLU FFN y = W_down (silu(W_gate x) * W_up x) ("MoE on
// KnightLi的博客", activation-function section; gate/up/down matrices of
// "15. DeepSeek：MLA、MoE 与 MTP", section "671B 和 37B 的参数账").  Shared
// experts are extra experts that see every token.
//
// Work is a flat list of tiles (expert, column tile, row tile) built on the
// device from the permutation offsets, so no host synchronisation is needed:
//   gate/up  rows of an expert gather x rows through row_token; the block
//            computes 128 h-columns of gate AND the same 128 of up, and the
//            epilogue writes h = silu(g) * u (bf16) -- SwiGLU fused between
//            the two projections;
//   down     h rows are contiguous per expert; y_rows = h W_down^T (fp32).
// bf16 tiles: 4 wavefronts, block tile BM x 256 (B rows) x 64 (K), each wave
// WM x 128 on v_mfma_f32_32x32x16_bf16, operands double-buffered in LDS with
// an XOR swizzle (conflict-free 16-byte reads), global loads for step k+1 in
// flight while step k computes.  Tiles are mapped so that each XCD (one L2)
// walks a contiguous range of logical tiles, row tiles of one (expert, column
// tile) being adjacent: the weight tile is fetched once per XCD and reused
// from L2 by the expert's row tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace {

constexpr int kBK = 64;     // K elements per LDS stage
constexpr int kBNB = 256;   // B rows per block tile
constexpr int kWM = 128;    // rows per wavefront (bf16 path); BM = 2 * kWM

// Logical tile of this workgroup: XCD-contiguous order over [0, total).
__device__ __forceinline__ bool tile_of_block(const GemmArgs& a, int BM, int& e, int& nt, int& row0, int& rows) {
  const int total = a.mt_prefix[a.n_exp] * a.n_tiles;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  const int xcd = bid & 7, q = total >> 3, r = total & 7;
  const int L = xcd * q + min(xcd, r) + (bid >> 3);
  int lo = 0, hi = a.n_exp;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.mt_prefix[mid] * a.n_tiles <= L)
      lo = mid;
    else
      hi = mid;
  }
  e = lo;
  const int local = L - a.mt_prefix[e] * a.n_tiles;
  const int me = a.mt_prefix[e + 1] - a.mt_prefix[e];
  nt = local / me;
  const int mt = local - nt * me;
  row0 = a.seg_start[e] + mt * BM;
  rows = min(BM, a.seg_len[e] - mt * BM);
  return true;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int WM, bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_gemm_bf16(GemmArgs a) {
  constexpr int BM = 2 * WM;
  constexpr int MB = WM / 32;
  constexpr int A_LOADS = BM * 8 / 256;
  constexpr int B_LOADS = kBNB * 8 / 256;
  constexpr int STAGE = (BM + kBNB) * kBK * 2;  // bytes
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  int e, nt, row0, rows;
  if (!tile_of_block(a, BM, e, nt, row0, rows)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ch = tid & 7, rbase = tid >> 3;
  const int K = a.K;

  const bf16* aptr[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int rr = min(rbase + 32 * i, rows - 1);
    if constexpr (GATEUP) {
      const int tok = a.row_token[row0 + rr];
      aptr[i] = static_cast<const bf16*>(a.a) + (int64_t)tok * K + ch * 8;
    } else {
      aptr[i] = static_cast<const bf16*>(a.a) + (int64_t)(row0 + rr) * K + ch * 8;
    }
  }
  const bf16* bptr[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int rb = rbase + 32 * i;
    if constexpr (GATEUP) {
      const int n = nt * 128 + (rb & 127);
      const bf16* mat = static_cast<const bf16*>(rb < 128 ? a.b0 : a.b1);
      bptr[i] = mat + ((int64_t)e * a.N + n) * K + ch * 8;
    } else {
      const int n = nt * kBNB + rb;
      bptr[i] = static_cast<const bf16*>(a.b0) + ((int64_t)e * a.N + n) * K + ch * 8;
    }
  }

  u32x4 ra[A_LOADS], rb[B_LOADS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i] + k0);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + k0);
  };
  auto lstore = [&](int stage) {
    char* sa = lds + stage * STAGE;
    char* sb = sa + BM * kBK * 2;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<u32x4*>(sa + swz(rbase + 32 * i, ch)) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<u32x4*>(sb + swz(rbase + 32 * i, ch)) = rb[i];
  };

  f32x16 acc[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;

  const int wr = wave & 1, wc = wave >> 1;
  int brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if constexpr (GATEUP)
      brow[n] = (n < 2 ? wc * 64 + n * 32 : 128 + wc * 64 + (n - 2) * 32) + (lane & 31);
    else
      brow[n] = wc * 128 + n * 32 + (lane & 31);
  }

  const int nk = K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const char* sa = lds + (kt & 1) * STAGE;
    const char* sb = sa + BM * kBK * 2;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 af[MB], bfv[4];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int row = wr * WM + m * 32 + (lane & 31);
        af[m] = *reinterpret_cast<const bf16x8*>(sa + swz(row, chunk));
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) bfv[n] = *reinterpret_cast<const bf16x8*>(sb + swz(brow[n], chunk));
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfv[n], acc[m][n], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore((kt + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int m = 0; m < MB; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wr * WM + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= rows) continue;
      if constexpr (GATEUP) {
        bf16* orow = static_cast<bf16*>(a.c) + (int64_t)(row0 + row) * a.N;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float g = acc[m][n][r], u = acc[m][n + 2][r];
          const float hv = g / (1.0f + __expf(-g)) * u;
          orow[nt * 128 + wc * 64 + n * 32 + (lane & 31)] = (bf16)hv;
        }
      } else {
        // expert outputs stay fp32 until the combine (bf16 here would put a
        // second rounding of every expert output into the layer result)
        float* orow = static_cast<float*>(a.c) + (int64_t)(row0 + row) * a.N;
#pragma unroll
        for (int n = 0; n < 4; ++n) orow[nt * kBNB + wc * 128 + n * 32 + (lane & 31)] = acc[m][n][r];
      }
    }
  }
}

// fp32 layers: one wavefront per 32 x 32 output tile on v_mfma_f32_32x32x2_f32,
// operands straight from global memory (tiny layers only).
template <bool GATEUP>
__global__ __launch_bounds__(64) void expert_gemm_f32(GemmArgs a) {
  int e, nt, row0, rows;
  if (!tile_of_block(a, 32, e, nt, row0, rows)) return;
  const int lane = threadIdx.x;
  const int K = a.K;
  const int rr = min(lane & 31, rows - 1);
  const float* ap;
  if constexpr (GATEUP)
    ap = static_cast<const float*>(a.a) + (int64_t)a.row_token[row0 + rr] * K + (lane >> 5);
  else
    ap = static_cast<const float*>(a.a) + (int64_t)(row0 + rr) * K + (lane >> 5);
  const int n = nt * 32 + (lane & 31);
  const float* b0 = static_cast<const float*>(a.b0) + ((int64_t)e * a.N + n) * K + (lane >> 5);
  const float* b1 = GATEUP ? static_cast<const float*>(a.b1) + ((int64_t)e * a.N + n) * K + (lane >> 5) : nullptr;
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 2) {
    const float av = ap[k0];
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0[k0], acc0, 0, 0, 0);
    if constexpr (GATEUP) acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1[k0], acc1, 0, 0, 0);
  }
  float* out = static_cast<float*>(a.c);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row >= rows) continue;
    float v = acc0[r];
    if constexpr (GATEUP) v = v / (1.0f + expf(-v)) * acc1[r];
    out[(int64_t)(row0 + row) * a.N + n] = v;
  }
}

// Segments of every expert and the exclusive prefix of their row-tile counts.
__global__ __launch_bounds__(1024) void schedule_kernel(ScheduleArgs a) {
  __shared__ int32_t buf[2][1024];
  const int tid = threadIdx.x;
  const int n_exp = a.E + a.S;
  int carry = 0;
  for (int e0 = 0; e0 < n_exp; e0 += 1024) {
    const int e = e0 + tid;
    int mt = 0;
    if (e < n_exp) {
      int start, len;
      if (e < a.E) {
        start = a.offsets[e];
        len = a.offsets[e + 1] - start;
      } else {
        start = a.T * a.k + (e - a.E) * a.T;
        len = a.T;
      }
      a.seg_start[e] = start;
      a.seg_len[e] = len;
      mt = (len + a.BM - 1) / a.BM;
    }
    // inclusive Hillis-Steele scan over the 1024 entries
    int cur = 0;
    buf[cur][tid] = mt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = buf[cur][tid] + (tid >= off ? buf[cur][tid - off] : 0);
      buf[cur ^ 1][tid] = v;
      cur ^= 1;
      __syncthreads();
    }
    const int incl = buf[cur][tid];
    if (e < n_exp) a.mt_prefix[e] = carry + incl - mt;
    if (e == n_exp - 1) a.mt_prefix[n_exp] = carry + incl;
    carry += buf[cur][1023];
    __syncthreads();
  }
}

}  // namespace

int gemm_bm(int dtype) { return dtype == 1 ? 2 * kWM : 32; }

int64_t gemm_mtile_bound(int T, int E, int S, int k, int BM) {
  // sum_e ceil(n_e / BM) <= (sum_e n_e + E*(BM-1)) / BM, sum_e n_e <= T*k
  return ((int64_t)T * k + (int64_t)E * (BM - 1)) / BM + (int64_t)S * ((T + BM - 1) / BM);
}

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s) {
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((expert_gemm_bf16<kWM, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((expert_gemm_f32<true>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s) {
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((expert_gemm_bf16<kWM, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((expert_gemm_f32<false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}
