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

constexpr int kBK = 64;                // K elements per LDS stage
constexpr int kRowBytes = kBK * 2;     // bytes of one tile row in LDS
constexpr int kStages = 2;             // LDS stages (2 x 64 KB)
constexpr bool kPrefetchL2 = false;    // warm L2 two steps ahead of each copy (measured: no gain)
constexpr int kBNB = 256;              // B rows per block tile
constexpr int kWM = 128;               // rows per wavefront (bf16 path); BM = 2 * kWM

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

typedef __attribute__((address_space(3))) void lds_void_t;

// Wait until at most N of this wavefront's vector-memory operations (here the
// global->LDS copies, which complete in order) are outstanding:
// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Tiles live in LDS as rows of 128 bytes (64 bf16 of K) whose eight 16-byte
// chunks are permuted: chunk c of row r sits in slot c ^ sw(r) with
// sw(r) = (r % 8) ^ ((r / 8) % 2).  Sixteen consecutive rows read at one chunk
// then touch 16 distinct 16-byte bank groups, and so do any eight within a
// 128-byte window: fragment reads are free of LDS bank conflicts.
__device__ __forceinline__ int swz_of_row(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// One global->LDS copy of 16 bytes per lane: lane L reads src and writes LDS
// bytes [dst + 16*L, dst + 16*L + 16) (dst is the same for the whole wave).
__device__ __forceinline__ void copy16(const bf16* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

// N copies: copy i reads base + off[i] and fills the 1 KB of LDS at dst + i*1024.
template <int N>
__device__ __forceinline__ void copy_rows(const bf16* base, const uint32_t (&off)[N], char* dst) {
#pragma unroll
  for (int i = 0; i < N; ++i) copy16(base + off[i], dst + i * 1024);
}

// MFMA operand fragments of one 16-wide K step from the swizzled LDS tiles.
template <int MB>
__device__ __forceinline__ void load_frags(const char* sa, int arow, const int (&brow)[4], int slot, int a_bytes,
                                           bf16x8 (&fa)[MB], bf16x8 (&fb)[4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m) fa[m] = *reinterpret_cast<const bf16x8*>(sa + arow + m * 32 * kRowBytes + slot);
#pragma unroll
  for (int n = 0; n < 4; ++n) fb[n] = *reinterpret_cast<const bf16x8*>(sa + a_bytes + brow[n] + slot);
}

template <int MB>
__device__ __forceinline__ void mfma_step(const bf16x8 (&fa)[MB], const bf16x8 (&fb)[4], f32x16 (&acc)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[n], acc[m][n], 0, 0, 0);
}

// Interleave the MFMAs and LDS reads of one 16-wide K step: one read after
// each of the first MB+4 MFMAs, so the reads land while the rest execute.
template <int MB>
__device__ __forceinline__ void interleave_reads() {
#pragma unroll
  for (int i = 0; i < MB + 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MB * 4 - (MB + 4), 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Pipeline per K step of 64 (two LDS stages): the four 16-wide sub-steps run
// their MFMAs while the next sub-step's fragments are read.  The one barrier
// per step sits before the last sub-step, once every wave has read its last
// fragments of the current stage: the stage is then refilled with step kt+2
// while the last MFMAs run and step kt+1's first fragments are read, so the
// matrix cores do not wait for the barrier or for the first LDS reads.
// LDS of one stage: the A tile region is sized for full row tiles (2 * kWM
// rows); half tiles use its first half.
constexpr int kABytes = 2 * kWM * kRowBytes;
constexpr int kStageBytes = kABytes + kBNB * kRowBytes;

// One output tile: rows [row0, row0 + rows) of expert e, column tile nt.  WM
// is the row count per wavefront: kWM for a full tile (2*kWM rows), kWM/2 for
// a tile of at most kWM rows (an expert's last, short row tile), which then
// costs half the MFMAs instead of computing padding.
template <int WM, bool GATEUP>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, char* lds, int e, int nt, int row0, int rows) {
  constexpr int BM = 2 * WM;
  constexpr int MB = WM / 32;
  constexpr int A_BYTES = kABytes;
  constexpr int STAGE = kStageBytes;
  constexpr int A_PER_WAVE = BM / 8 / 4;    // 8-row groups of A each wave copies
  constexpr int B_PER_WAVE = kBNB / 8 / 4;  // 8-row groups of B each wave copies

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  // a copy writes 64 lanes x 16 bytes = 8 rows of 128 bytes: lane L lands in
  // row L/8 of its group, slot L%8, so it fetches chunk (L%8) ^ sw(row)
  const int lrow = lane >> 3;

  const bf16* abase;
  uint32_t aoff[A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int r = (wave * A_PER_WAVE + i) * 8 + lrow;
    const int rr = min(r, rows - 1);
    const int chunk = (lane & 7) ^ swz_of_row(r);
    if constexpr (GATEUP)
      aoff[i] = (uint32_t)a.row_token[row0 + rr] * (uint32_t)K + chunk * 8;
    else
      aoff[i] = (uint32_t)rr * (uint32_t)K + chunk * 8;
  }
  if constexpr (GATEUP)
    abase = static_cast<const bf16*>(a.a);
  else
    abase = static_cast<const bf16*>(a.a) + (int64_t)row0 * K;

  const bf16* bbase;
  uint32_t boff[B_PER_WAVE];
  if constexpr (GATEUP) {
    // waves 0-1 copy the 128 gate rows, waves 2-3 the 128 up rows
    bbase = static_cast<const bf16*>(wave < 2 ? a.b0 : a.b1) + ((int64_t)e * a.N + nt * 128) * K;
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int rb = ((wave & 1) * B_PER_WAVE + i) * 8 + lrow;
      boff[i] = (uint32_t)rb * (uint32_t)K + ((lane & 7) ^ swz_of_row(rb)) * 8;
    }
  } else {
    bbase = static_cast<const bf16*>(a.b0) + ((int64_t)e * a.N + nt * kBNB) * K;
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int rb = (wave * B_PER_WAVE + i) * 8 + lrow;
      boff[i] = (uint32_t)rb * (uint32_t)K + ((lane & 7) ^ swz_of_row(rb)) * 8;
    }
  }
  char* const a_dst = lds + wave * A_PER_WAVE * 1024;
  char* const b_dst = lds + A_BYTES + wave * B_PER_WAVE * 1024;
  // L2 warm-up: two steps before a stage is copied, each lane touches one
  // 16-byte piece of one A row and one B row of it (64 rows per wave), so the
  // copy itself hits L2; the pieces land in a per-wave scratch kilobyte.
  char* const junk = lds + kStages * STAGE + wave * 1024;
  uint32_t pa_off, pb_off;
  {
    const int r = wave * 64 + lane;
    const int rr = min(r, rows - 1);
    if constexpr (GATEUP) {
      pa_off = (uint32_t)a.row_token[row0 + rr] * (uint32_t)K;
      pb_off = (uint32_t)((wave & 1) * 64 + lane) * (uint32_t)K;
    } else {
      pa_off = (uint32_t)rr * (uint32_t)K;
      pb_off = (uint32_t)r * (uint32_t)K;
    }
  }

  f32x16 acc[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;

  const int wr = wave & 1, wc = wave >> 1;
  // fragment rows: A row wr*WM + m*32 + lane%32, B row brow[n] + lane%32; all
  // are congruent to lane mod 16, so the swizzled slot only depends on lane
  const int arow = (wr * WM + (lane & 31)) * kRowBytes;
  int brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if constexpr (GATEUP)
      brow[n] = ((n < 2 ? wc * 64 + n * 32 : 128 + wc * 64 + (n - 2) * 32) + (lane & 31)) * kRowBytes;
    else
      brow[n] = (wc * 128 + n * 32 + (lane & 31)) * kRowBytes;
  }
  int slot[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) slot[kk] = ((kk * 2 + (lane >> 5)) ^ swz_of_row(lane & 15)) << 4;

  const int nk = K / kBK;
  // prologue: steps 0 and 1 in flight (and step 3 warmed), wait for step 0
  copy_rows<A_PER_WAVE>(abase, aoff, a_dst);
  copy_rows<B_PER_WAVE>(bbase, boff, b_dst);
  if (nk > 1) {
    copy_rows<A_PER_WAVE>(abase + kBK, aoff, a_dst + STAGE);
    copy_rows<B_PER_WAVE>(bbase + kBK, boff, b_dst + STAGE);
  }
  if (kPrefetchL2 && nk > 3) {
    copy16(abase + 3 * kBK + pa_off, junk);
    copy16(bbase + 3 * kBK + pb_off, junk);
  }
  if (nk > 3)
    wait_vmem_upto<A_PER_WAVE + B_PER_WAVE + (kPrefetchL2 ? 2 : 0)>();
  else if (nk > 1)
    wait_vmem_upto<A_PER_WAVE + B_PER_WAVE>();
  else
    wait_vmem_upto<0>();
  __builtin_amdgcn_s_barrier();

  bf16x8 fa0[MB], fb0[4], fa1[MB], fb1[4];
  load_frags<MB>(lds, arow, brow, slot[0], A_BYTES, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const char* sa = lds + cur * STAGE;
    load_frags<MB>(sa, arow, brow, slot[1], A_BYTES, fa1, fb1);
    mfma_step<MB>(fa0, fb0, acc);
    interleave_reads<MB>();
    load_frags<MB>(sa, arow, brow, slot[2], A_BYTES, fa0, fb0);
    mfma_step<MB>(fa1, fb1, acc);
    interleave_reads<MB>();
    load_frags<MB>(sa, arow, brow, slot[3], A_BYTES, fa1, fb1);
    mfma_step<MB>(fa0, fb0, acc);
    interleave_reads<MB>();
    // this wave's reads of the current stage are done and step kt+1 has
    // landed (it is the only copy in flight); after the barrier every wave
    // is past the current stage
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    // only the warm-up of step kt+3 was issued after step kt+1's copies
    if (kPrefetchL2 && kt + 3 < nk)
      wait_vmem_upto<2>();
    else
      wait_vmem_upto<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kPrefetchL2 && kt + 4 < nk) {
      const int k4 = (kt + 4) * kBK;
      copy16(abase + k4 + pa_off, junk);
      copy16(bbase + k4 + pb_off, junk);
    }
    // last sub-step: the freed stage is refilled with step kt+2 (the last two
    // steps re-copy step nk-1, which keeps this region branch-free), step
    // kt+1's first fragments are read (after the last step: a stage that is
    // never used, harmless), and both interleave with the MFMAs
    {
      const int k2 = min(kt + 2, nk - 1) * kBK;
      copy_rows<A_PER_WAVE>(abase + k2, aoff, a_dst + cur * STAGE);
      copy_rows<B_PER_WAVE>(bbase + k2, boff, b_dst + cur * STAGE);
    }
    load_frags<MB>(lds + (cur ^ 1) * STAGE, arow, brow, slot[0], A_BYTES, fa0, fb0);
    mfma_step<MB>(fa1, fb1, acc);
#pragma unroll
    for (int i = 0; i < MB + 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global->LDS copy
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global->LDS copy
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MB * 4 - (MB + 4), 0);
    __builtin_amdgcn_sched_barrier(0);
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

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_gemm_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes + (kPrefetchL2 ? 4096 : 0)];
  int e, nt, row0, rows;
  if (!tile_of_block(a, 2 * kWM, e, nt, row0, rows)) return;
  if (rows > kWM)
    gemm_tile<kWM, GATEUP>(a, lds, e, nt, row0, rows);
  else
    gemm_tile<kWM / 2, GATEUP>(a, lds, e, nt, row0, rows);
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
    hipLaunchKernelGGL((expert_gemm_bf16<true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((expert_gemm_f32<true>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s) {
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL((expert_gemm_bf16<false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((expert_gemm_f32<false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}
