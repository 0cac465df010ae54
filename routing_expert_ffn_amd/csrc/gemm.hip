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
// WM x 128 on v_mfma_f32_32x32x16_bf16, operands staged in LDS (two A and
// three B stages) with an XOR swizzle (conflict-free 16-byte reads), the
// copies for step k+2 in flight while step k computes.  Work items (see
// work_of_block) are ordered so that each XCD (one L2) walks a contiguous
// range in which the row tiles sharing a weight tile, and the column tiles
// sharing an input row tile, run side by side and re-read the shared operand
// from L2.
#include "common.hpp"
#include "gemm_sched.hpp"
#include "kernels.hpp"

namespace {

constexpr int kBK = 64;                // K elements per LDS stage
constexpr int kRowBytes = kBK * 2;     // bytes of one tile row in LDS
constexpr int kBNB = 256;              // B rows per block tile
constexpr int kWM = 128;               // rows per wavefront (bf16 path); BM = 2 * kWM
// LDS: two A stages (input rows) and three B stages (weight rows), 32 KB
// each, 160 KB in all.  Both operands are copied two steps ahead of use: B
// into the stage freed one step earlier (three stages), A right after the
// barrier that frees its stage (two stages).  The down GEMM at short K swaps
// the roles (gemm_tile's A3).
constexpr int kAStage = 2 * kWM * kRowBytes;
constexpr int kBStage = kBNB * kRowBytes;
constexpr int kAStages = 2, kBStages = 3;
constexpr int kLdsBytes = kAStages * kAStage + kBStages * kBStage;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup");
// epilogue staging: one region per wavefront for its bf16 sub-tile of up to
// kWM rows x 128 columns, rows padded by 16 bytes
constexpr int kEpWave = kWM * (128 * 2 + 16);
static_assert(4 * kEpWave <= kLdsBytes, "epilogue staging fits in the stages");

// Copies I0 .. I0+N-1 of a wave's group: copy i reads base + off[i] and
// fills the 1 KB of LDS at dst + i*1024 (NT: non-temporal).
template <bool NT, int I0, int N, int M>
__device__ __forceinline__ void copy_rows(const bf16* base, const uint32_t (&off)[M], char* dst) {
  static_assert(I0 + N <= M, "copy range");
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) {
    if constexpr (NT)
      copy16_nt(base + off[i], dst + i * 1024);
    else
      copy16(base + off[i], dst + i * 1024);
  }
}

// The same through a buffer resource: copy i reads byte voff[i] + soff
// (zeros for a row past the tile's end, whose offset is out of range).
template <int I0, int N, int M>
__device__ __forceinline__ void copy_rows_buf(__amdgpu_buffer_rsrc_t r, const uint32_t (&voff)[M], uint32_t soff,
                                              char* dst) {
  static_assert(I0 + N <= M, "copy range");
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) copy16_buf(r, voff[i], soff, dst + i * 1024);
}

// MFMA operand fragments of one 16-wide K step from the swizzled LDS tiles
// (sa: A stage, sb: B stage).
template <int MB>
__device__ __forceinline__ void load_frags(const char* sa, const char* sb, int arow, const int (&brow)[4], int slot,
                                           bf16x8 (&fa)[MB], bf16x8 (&fb)[4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m) fa[m] = *reinterpret_cast<const bf16x8*>(sa + arow + m * 32 * kRowBytes + slot);
#pragma unroll
  for (int n = 0; n < 4; ++n) fb[n] = *reinterpret_cast<const bf16x8*>(sb + brow[n] + slot);
}

template <int MB>
__device__ __forceinline__ void mfma_step(const bf16x8 (&fa)[MB], const bf16x8 (&fb)[4], f32x16 (&acc)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[m], fb[n], acc[m][n], 0, 0, 0);
}

// Interleave one 16-wide K step: a fragment read after each of the first
// MB+4 MFMAs, so the reads land while the rest execute, then the NC
// global->LDS copies of the sub-step one per MFMA (the compiler keeps LDS
// reads and copies in program order, so the reads are written first).  The
// copy stream is spread over the whole K step: bunched, it queues behind the
// address unit and stalls the wave's in-order issue, MFMAs included.
template <int MB, int NC>
__device__ __forceinline__ void interleave_reads() {
  // NR fragment reads against MB*4 MFMAs: one read after each MFMA while both
  // last (a one-block tile has one more read than MFMAs), then the copies
  constexpr int NR = MB + 4, NP = NR < MB * 4 ? NR : MB * 4;
  constexpr int NM = MB * 4 - NP;  // MFMAs left after the reads
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
  }
  if (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);              // 1 copy
  }
  if (NM > NC) __builtin_amdgcn_sched_group_barrier(0x008, NM - NC, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Pipeline per K step of 64: the four 16-wide sub-steps run their MFMAs
// while the next sub-step's fragments are read.  The one barrier per step
// sits before the last sub-step, once every wave has read its last fragments
// of the current stages, so the matrix cores wait neither for the barrier nor
// for the first LDS reads of the next step.  The copies refilling the freed
// stages: B of step kt+2 in sub-steps 0 to 2 of step kt (B has three
// stages, so its stage was freed by the previous barrier), A of step kt+2 in
// the last sub-step, right after the barrier that frees its stage.  Before
// the barrier of step kt a wave waits until only B of step kt+2 is in
// flight, so every copy has at least a full step to land.

// One output tile: rows [row0, row0 + rows) of expert e, column tile nt.  WM
// is the row count per wavefront: kWM for a full tile (2*kWM rows); for an
// expert's last row tile 3*kWM/4 when it has at most 3*kWM/2 rows, kWM/2 when
// it has at most kWM and kWM/4 when it has at most kWM/2, which then costs
// three quarters, half or a quarter of the MFMAs instead of computing padding.
// A3: three A stages and two B stages instead of two and three (A copied two
// steps ahead in sub-steps 0-2, B right after the barrier that frees its
// stage): at short K the input rows' copies are the ones that arrive late.
template <int WM, bool GATEUP, bool NTB, bool A3 = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, char* lds, int e, int nt, int row0, int rows) {
  constexpr int AS = A3 ? 3 : 2, BS = A3 ? 2 : 3;  // A and B stages
  constexpr int BM = 2 * WM;
  constexpr int MB = WM / 32;
  constexpr int A_PER_WAVE = BM / 8 / 4;    // 8-row groups of A each wave copies
  constexpr int B_PER_WAVE = kBNB / 8 / 4;  // 8-row groups of B each wave copies

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  // a copy writes 64 lanes x 16 bytes = 8 rows of 128 bytes: lane L lands in
  // row L/8 of its group, slot L%8, so it fetches chunk (L%8) ^ sw(row)
  const int lrow = lane >> 3;

  // A rows through a buffer resource (byte offsets): the rows of the tile
  // past `rows` read as zeros, so padding rows cost no memory traffic and
  // feed zeros to the matrix cores
  __amdgpu_buffer_rsrc_t arsrc;
  uint32_t aoff[A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int r = (wave * A_PER_WAVE + i) * 8 + lrow;
    const uint32_t chunk = (uint32_t)((lane & 7) ^ swz_of_row(r)) * 16u;
    if constexpr (GATEUP)
      aoff[i] = r < rows ? (uint32_t)a.row_token[row0 + r] * (uint32_t)(2 * K) + chunk : kOutOfRange;
    else
      aoff[i] = r < rows ? (uint32_t)r * (uint32_t)(2 * K) + chunk : kOutOfRange;
  }
  if constexpr (GATEUP)
    arsrc = raw_rsrc(a.a, a.a_bytes);
  else
    arsrc = raw_rsrc(static_cast<const bf16*>(a.a) + (int64_t)row0 * K, (uint32_t)rows * (uint32_t)(2 * K));

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
  char* const b_lds = lds + AS * kAStage;
  char* const a_dst = lds + wave * A_PER_WAVE * 1024;
  char* const b_dst = b_lds + wave * B_PER_WAVE * 1024;

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
  if constexpr (A3) {
    // prologue: A and B of steps 0 and 1 in the order of the main loop (A
    // of a step before its B), then wait for step 0
    constexpr int AH = (A_PER_WAVE * 3 + 7) / 8, AH2 = 2 * AH;  // A copies in sub-steps 0 / 1 / 2
    constexpr int N1 = AH2 <= A_PER_WAVE ? AH : A_PER_WAVE - AH;
    constexpr int I2 = AH2 <= A_PER_WAVE ? AH2 : A_PER_WAVE, N2 = A_PER_WAVE - I2;
    copy_rows_buf<0, A_PER_WAVE>(arsrc, aoff, 0, a_dst);
    copy_rows<NTB, 0, B_PER_WAVE>(bbase, boff, b_dst);
    copy_rows_buf<0, A_PER_WAVE>(arsrc, aoff, min(1, nk - 1) * kRowBytes, a_dst + kAStage);
    copy_rows<NTB, 0, B_PER_WAVE>(bbase + min(1, nk - 1) * kBK, boff, b_dst + kBStage);
    wait_vmem_upto<A_PER_WAVE + B_PER_WAVE>();
    __builtin_amdgcn_s_barrier();

    bf16x8 fa0[MB], fb0[4], fa1[MB], fb1[4];
    int sai = 0;  // A stage of step kt (kt mod 3)
    load_frags<MB>(lds, b_lds, arow, brow, slot[0], fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
      const char* sa = lds + sai * kAStage;
      const char* sb = b_lds + (kt & 1) * kBStage;
      const int san = sai == AS - 1 ? 0 : sai + 1;  // A stage of step kt+1
      const int saf = san == AS - 1 ? 0 : san + 1;  // A stage of step kt+2 (free)
      const uint32_t an = min(kt + 2, nk - 1) * kRowBytes;
      // sub-steps 0, 1 and 2: A of step kt+2 into the stage freed at the last
      // barrier
      load_frags<MB>(sa, sb, arow, brow, slot[1], fa1, fb1);
      copy_rows_buf<0, AH>(arsrc, aoff, an, a_dst + saf * kAStage);
      mfma_step<MB>(fa0, fb0, acc);
      interleave_reads<MB, AH>();
      load_frags<MB>(sa, sb, arow, brow, slot[2], fa0, fb0);
      copy_rows_buf<AH, N1>(arsrc, aoff, an, a_dst + saf * kAStage);
      mfma_step<MB>(fa1, fb1, acc);
      interleave_reads<MB, N1>();
      load_frags<MB>(sa, sb, arow, brow, slot[3], fa1, fb1);
      copy_rows_buf<I2, N2>(arsrc, aoff, an, a_dst + saf * kAStage);
      mfma_step<MB>(fa0, fb0, acc);
      interleave_reads<MB, N2>();
      // this wave's reads of the current stages are done and A and B of step
      // kt+1 have landed (only A of step kt+2 was issued after them)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      wait_vmem_upto<A_PER_WAVE>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // last sub-step: B of step kt+2 into the B stage just freed, and step
      // kt+1's first fragments
      load_frags<MB>(lds + san * kAStage, b_lds + ((kt + 1) & 1) * kBStage, arow, brow, slot[0], fa0, fb0);
      copy_rows<NTB, 0, B_PER_WAVE>(bbase + min(kt + 2, nk - 1) * kBK, boff, b_dst + (kt & 1) * kBStage);
      mfma_step<MB>(fa1, fb1, acc);
      interleave_reads<MB, B_PER_WAVE>();
      sai = san;
    }
  } else {
    constexpr int BH = (B_PER_WAVE * 3 + 7) / 8, BH2 = 2 * BH;  // B copies in sub-steps 0 / 1 / 2
    // prologue: A and B of steps 0 and 1 in the order of the main loop (B of a
    // step before its A; indices clamped to the last step: a re-copy lands in
    // a stage that is not read again), then wait for step 0
    copy_rows_buf<0, A_PER_WAVE>(arsrc, aoff, 0, a_dst);
    copy_rows<NTB, 0, B_PER_WAVE>(bbase, boff, b_dst);
    copy_rows<NTB, 0, B_PER_WAVE>(bbase + min(1, nk - 1) * kBK, boff, b_dst + kBStage);
    copy_rows_buf<0, A_PER_WAVE>(arsrc, aoff, min(1, nk - 1) * kRowBytes, a_dst + kAStage);
    wait_vmem_upto<A_PER_WAVE + B_PER_WAVE>();
    __builtin_amdgcn_s_barrier();

    bf16x8 fa0[MB], fb0[4], fa1[MB], fb1[4];
    int sbi = 0;  // B stage of step kt (kt mod 3)
    load_frags<MB>(lds, b_lds, arow, brow, slot[0], fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
      const char* sa = lds + (kt & 1) * kAStage;
      const char* sb = b_lds + sbi * kBStage;
      const int sbn = sbi == BS - 1 ? 0 : sbi + 1;  // B stage of step kt+1
      const int sbf = sbn == BS - 1 ? 0 : sbn + 1;  // B stage of step kt+2 (free)
      const bf16* const bn = bbase + min(kt + 2, nk - 1) * kBK;
      // sub-steps 0, 1 and 2: B of step kt+2 (3 + 3 + 2 copies) into the stage
      // freed at the last barrier
      load_frags<MB>(sa, sb, arow, brow, slot[1], fa1, fb1);
      copy_rows<NTB, 0, BH>(bn, boff, b_dst + sbf * kBStage);
      mfma_step<MB>(fa0, fb0, acc);
      interleave_reads<MB, BH>();
      load_frags<MB>(sa, sb, arow, brow, slot[2], fa0, fb0);
      copy_rows<NTB, BH, BH>(bn, boff, b_dst + sbf * kBStage);
      mfma_step<MB>(fa1, fb1, acc);
      interleave_reads<MB, BH>();
      load_frags<MB>(sa, sb, arow, brow, slot[3], fa1, fb1);
      copy_rows<NTB, BH2, B_PER_WAVE - BH2>(bn, boff, b_dst + sbf * kBStage);
      mfma_step<MB>(fa0, fb0, acc);
      interleave_reads<MB, B_PER_WAVE - BH2>();
      // this wave's reads of the current stages are done and A and B of step
      // kt+1 have landed (copies complete in issue order; only B of step kt+2
      // was issued after them); after the barrier every wave is past the
      // current stages and sees step kt+1
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      wait_vmem_upto<B_PER_WAVE>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // last sub-step: A of step kt+2 into the A stage just freed, and step
      // kt+1's first fragments (after the last step: harmless reads of unused
      // stages).  Every copy thus has a full step or more before the barrier
      // that needs it.
      load_frags<MB>(lds + ((kt + 1) & 1) * kAStage, b_lds + sbn * kBStage, arow, brow, slot[0], fa0, fb0);
      copy_rows_buf<0, A_PER_WAVE>(arsrc, aoff, min(kt + 2, nk - 1) * kRowBytes, a_dst + (kt & 1) * kAStage);
      mfma_step<MB>(fa1, fb1, acc);
      interleave_reads<MB, A_PER_WAVE>();
      sbi = sbn;
    }
  }
  // no copy may still be writing LDS when the stages are reused or released
  wait_vmem_upto<0>();

  // Epilogue through LDS for the bf16 outputs (h, routed expert rows): once
  // every wave is done with the stages, each wave stages its sub-tile in an
  // LDS region of its own (rows padded by 16 bytes against bank conflicts)
  // and writes it back as whole row segments with 16-byte stores -- an
  // eighth of the store instructions of writing the MFMA layout (one value
  // per lane, rows apart) directly, which kept the address unit busy for
  // several microseconds per tile.  fp32 rows (shared experts) are written
  // directly: staging them in two passes cost more registers than it saved.
  __syncthreads();
  char* const ep = lds + wave * kEpWave;
  const int rl = 4 * (lane >> 5), cl = lane & 31;  // the lane's row offset and column in a 32 x 32 block
  const int rows_w = rows - wr * WM;               // rows of this wave's sub-tile that exist (may be <= 0)
  if constexpr (GATEUP) {
    // h = silu(g) * u: WM rows x 64 columns (h columns wc*64 .. +63 of the tile's 128)
    constexpr int P = 64 * 2 + 16;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float g = acc[m][n][r], u = acc[m][n + 2][r];
          *reinterpret_cast<bf16*>(ep + (m * 32 + 8 * (r >> 2) + rl + (r & 3)) * P + (n * 32 + cl) * 2) =
              (bf16)swiglu(g, u);
        }
    bf16* const cw = static_cast<bf16*>(a.c) + (int64_t)(row0 + wr * WM) * a.N + nt * 128 + wc * 64;
#pragma unroll
    for (int i = 0; i < WM * 8 / 64; ++i) {
      const int idx = i * 64 + lane, row = idx >> 3, ch = idx & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ep + row * P + ch * 16);
      if (row < rows_w) *reinterpret_cast<u32x4*>(cw + (int64_t)row * a.N + ch * 8) = v;
    }
  } else if (a.c16 == nullptr || e >= a.n_routed) {
    // fp32 expert rows written directly from the MFMA layout
    float* const cw = static_cast<float*>(a.c) + ((int64_t)(row0 + wr * WM) - (a.c16 ? a.routed_rows : 0)) * a.N +
                      nt * kBNB + wc * 128 + cl;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m * 32 + 8 * (r >> 2) + rl + (r & 3);
        if (row >= rows_w) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) cw[(int64_t)row * a.N + n * 32] = acc[m][n][r];
      }
  } else {
    // bf16 routed rows: WM rows x 128 columns
    constexpr int P = 128 * 2 + 16;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          *reinterpret_cast<bf16*>(ep + (m * 32 + 8 * (r >> 2) + rl + (r & 3)) * P + (n * 32 + cl) * 2) =
              (bf16)acc[m][n][r];
    bf16* const cw = static_cast<bf16*>(a.c16) + (int64_t)(row0 + wr * WM) * a.N + nt * kBNB + wc * 128;
#pragma unroll
    for (int i = 0; i < WM * 16 / 64; ++i) {
      const int idx = i * 64 + lane, row = idx >> 4, ch = idx & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ep + row * P + ch * 16);
      if (row < rows_w) *reinterpret_cast<u32x4*>(cw + (int64_t)row * a.N + ch * 8) = v;
    }
  }
}

// Weight cache policy.  NT = 2 (gate/up): per item -- the weights of an
// expert whose rows fit one row tile are read by that item only and are
// copied with the non-temporal policy (they stream past the caches), an
// expert with several row tiles re-reads each weight tile from L2.  NT = 1:
// every item non-temporal (down launches whose weight tiles are read once, or
// mostly once); NT = 0: the default policy.  (The down GEMM keeps one policy
// per launch: with both forms of its tile in one kernel its registers spill
// and it runs slower.)
template <int WM, bool GATEUP, int NT, bool A3>
__device__ __forceinline__ void gemm_tile_of(const GemmArgs& a, char* lds, const Work& w, int nt) {
  if (NT == 1 || (NT == 2 && w.single))
    gemm_tile<WM, GATEUP, true, A3>(a, lds, w.e, nt, w.row0, w.rows);
  else
    gemm_tile<WM, GATEUP, false, A3>(a, lds, w.e, nt, w.row0, w.rows);
}

template <bool GATEUP, int NT, bool A3>
__global__ __launch_bounds__(256, 1) void expert_gemm_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  Work w;
  if (!work_of_block(a, 2 * kWM, w, reinterpret_cast<int*>(lds))) return;
  if (!w.pair) {
    // an expert's last row tile of 129-192 rows runs three 32-row blocks per
    // wavefront instead of four (a quarter less MFMA work on padding rows)
    if (w.rows > 3 * kWM / 2)
      gemm_tile_of<kWM, GATEUP, NT, A3>(a, lds, w, w.nt);
    else
      gemm_tile_of<3 * kWM / 4, GATEUP, NT, A3>(a, lds, w, w.nt);
  } else if (w.rows > kWM / 2) {
    gemm_tile_of<kWM / 2, GATEUP, NT, A3>(a, lds, w, w.nt);
    if (w.nt + 1 < a.n_tiles) {
      __syncthreads();  // every wave is past its last reads of the LDS stages
      gemm_tile_of<kWM / 2, GATEUP, NT, A3>(a, lds, w, w.nt + 1);
    }
  } else {
    // a short tile of at most 64 rows: one 32-row block per wavefront
    gemm_tile_of<kWM / 4, GATEUP, NT, A3>(a, lds, w, w.nt);
    if (w.nt + 1 < a.n_tiles) {
      __syncthreads();
      gemm_tile_of<kWM / 4, GATEUP, NT, A3>(a, lds, w, w.nt + 1);
    }
  }
}

// fp32 layers: one wavefront per 32 x 32 output tile on v_mfma_f32_32x32x2_f32,
// operands straight from global memory (tiny layers only).
template <bool GATEUP>
__global__ __launch_bounds__(64) void expert_gemm_f32(GemmArgs a) {
  Work w;
  if (!work_of_block(a, 32, w)) return;  // half_rows = 0: never a pair
  const int e = w.e, nt = w.nt, row0 = w.row0, rows = w.rows;
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

// Segments of every expert and the exclusive prefixes of its full and short
// row-tile counts; clears the pool counters of the two GEMMs that follow.
__global__ __launch_bounds__(1024) void schedule_kernel(ScheduleArgs a) {
  __shared__ int32_t bf[2][1024], bh[2][1024];
  const int tid = threadIdx.x;
  if (tid < 2) a.pool[tid] = 0;  // the two GEMMs' pool counters
  const int n_exp = a.E + a.S;
  int carry_f = 0, carry_h = 0;
  for (int e0 = 0; e0 < n_exp; e0 += 1024) {
    const int e = e0 + tid;
    int nf = 0, nh = 0;
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
      const int nrt = (len + a.BM - 1) / a.BM;
      nh = (nrt > 0 && len - (nrt - 1) * a.BM <= a.half_rows) ? 1 : 0;
      nf = nrt - nh;
    }
    // inclusive Hillis-Steele scans over the 1024 entries
    int cur = 0;
    bf[cur][tid] = nf;
    bh[cur][tid] = nh;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int vf = bf[cur][tid] + (tid >= off ? bf[cur][tid - off] : 0);
      const int vh = bh[cur][tid] + (tid >= off ? bh[cur][tid - off] : 0);
      bf[cur ^ 1][tid] = vf;
      bh[cur ^ 1][tid] = vh;
      cur ^= 1;
      __syncthreads();
    }
    const int incl_f = bf[cur][tid], incl_h = bh[cur][tid];
    if (e < n_exp) {
      a.f_prefix[e] = carry_f + incl_f - nf;
      a.h_prefix[e] = carry_h + incl_h - nh;
    }
    if (e == n_exp - 1) {
      a.f_prefix[n_exp] = carry_f + incl_f;
      a.h_prefix[n_exp] = carry_h + incl_h;
    }
    carry_f += bf[cur][1023];
    carry_h += bh[cur][1023];
    __syncthreads();
  }
}

}  // namespace

// tile geometry per input dtype: fp32 (0) 32-row tiles; bf16 (1) and FP8
// experts (2) 256-row tiles with half- or quarter-height last tiles
int gemm_bm(int dtype) { return dtype != 0 ? 2 * kWM : 32; }

int gemm_half_rows(int dtype) { return dtype != 0 ? kWM : 0; }

int64_t gemm_mtile_bound(int T, int E, int S, int k, int BM) {
  // sum_e ceil(n_e / BM) <= (sum_e n_e + E*(BM-1)) / BM, sum_e n_e <= T*k;
  // work items per GEMM <= row tiles * column tiles (a short-tile item covers
  // two column tiles)
  return ((int64_t)T * k + (int64_t)E * (BM - 1)) / BM + (int64_t)S * ((T + BM - 1) / BM);
}

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s) {
  if (dtype == 2) return launch_gateup_fp8(a, mtile_bound, s);
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (dtype != 1) {
    hipLaunchKernelGGL((expert_gemm_f32<true>), dim3((unsigned)grid), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL((expert_gemm_bf16<true, 2, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(const GemmArgs& a, int dtype, int64_t mtile_bound, hipStream_t s) {
  if (dtype == 2) return launch_down_fp8(a, mtile_bound, s);
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (dtype != 1) {
    hipLaunchKernelGGL((expert_gemm_f32<false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  } else if (a.stream_b) {
    hipLaunchKernelGGL((expert_gemm_bf16<false, 1, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  } else if (a.a3) {
    hipLaunchKernelGGL((expert_gemm_bf16<false, 0, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((expert_gemm_bf16<false, 0, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}
