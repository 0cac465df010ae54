// FP8 grouped expert GEMMs for gfx950: E4M3 operands with UE8M0 block scales
// ("15. DeepSeek：MLA、MoE 与 MTP", section "FP8 训练是训练配方，不是架构": E4M3
// inputs of the matrix products, one scale per 1 x 128 activation tile and
// per 128 x 128 weight block; UE8M0 scales as in V3.1), and the 1 x 128 tile
// quantisation of activations.
//
// The scales are applied inside the matrix cores: v_mfma_scale_f32_32x32x64
// multiplies each operand's 32-element K block by 2^(s - 127) of its own
// scale byte.  A 128-byte LDS tile row is one 128-wide K block, so every
// MFMA of a K step uses one A scale per row and one B scale per weight block.
// Scales come in groups of four K steps (one dword per A row, one per B
// block): A's in a row-space layout where a fragment's 32 rows are one
// 128-byte line, B's in rows padded to four bytes; a group is loaded once
// per four steps, a full step before the barrier that completes it.
//
// The tiling, LDS layout, XCD-aware work order and copy pipeline follow the
// bf16 kernel (gemm.hip): 256-row x 256-column items, 4 wavefronts of
// 128 x 128, two A stages and three B stages of 32 KB, XOR-swizzled rows.  A
// K step (128 bytes) is two 64-wide sub-steps of v_mfma_scale_f32_32x32x64
// (64 cycles each, the time of four bf16 sub-steps): the fragments of the
// next sub-step are read under the current one's MFMAs, the single barrier
// sits before the second sub-step, and the copies of step kt go out as B of
// step kt+2 in the first sub-step and A of step kt+2 in the second.  With
// only two sub-steps per barrier, a copy issued after the barrier's half of
// the step would have half a step to land; this order gives every copy at
// least a full step, which is what sets the pace when the weights stream
// from HBM with little MFMA work per step (small batches).
//
// The gate/up epilogue applies SwiGLU and quantises h per row and 128-wide
// column block (one item covers exactly one such block): h goes to an fp32
// tile in LDS, then each thread takes one row, finds its maximum, turns it
// into the UE8M0 exponent and writes the row's 128 codes.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "gemm_sched.hpp"
#include "kernels.hpp"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;         // one K step: 128 E4M3 values = one scale block
constexpr int kBNB = 256;              // B rows per block tile
constexpr int kWM = 128;               // rows per wavefront of a full tile
constexpr int kAStage = 2 * kWM * kRowBytes;
constexpr int kBStage = kBNB * kRowBytes;
constexpr int kAStages = 2, kBStages = 3;
constexpr int kLdsBytes = kAStages * kAStage + kBStages * kBStage;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup");
static_assert(4 * kWM * (128 * 2 + 16) <= kLdsBytes, "down epilogue staging fits in the stages");

// Exponent p of the UE8M0 scale of a tile whose largest magnitude is amax:
// the smallest p >= -127 with amax / 2^p <= 448 (= 1.75 * 2^8); a zero or
// subnormal maximum takes p = -127.
__device__ __forceinline__ int e8m0_exp_of_amax(float amax) {
  const uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (u < 0x00800000u) return -127;
  const int E = (int)(u >> 23) - 127;
  const int p = E - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return p < -127 ? -127 : p;
}

// E4M3 codes of two fp32 values (nearest-even, sign kept), in the low
// 16 bits.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Copies I0 .. I0+N-1 of a wave's group: copy i reads base + off[i] (bytes)
// and fills the 1 KB of LDS at dst + i*1024 (NT: non-temporal).
template <bool NT, int I0, int N, int M>
__device__ __forceinline__ void copy_rows8(const uint8_t* base, const uint32_t (&off)[M], char* dst) {
  static_assert(I0 + N <= M, "copy range");
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) {
    if constexpr (NT)
      copy16_nt(reinterpret_cast<const bf16*>(base + off[i]), dst + i * 1024);
    else
      copy16(reinterpret_cast<const bf16*>(base + off[i]), dst + i * 1024);
  }
}

// The same through a buffer resource: copy i reads byte voff[i] + soff
// (zeros for a row past the tile's end, whose offset is out of range).
template <int I0, int N, int M>
__device__ __forceinline__ void copy_rows8_buf(__amdgpu_buffer_rsrc_t r, const uint32_t (&voff)[M], uint32_t soff,
                                               char* dst) {
  static_assert(I0 + N <= M, "copy range");
#pragma unroll
  for (int i = I0; i < I0 + N; ++i) copy16_buf(r, voff[i], soff, dst + i * 1024);
}

// Fragments of one 64-wide sub-step: lane half hf of row r takes the 16-byte
// chunks 4s + hf and 4s + 2 + hf of the row (the MFMA's K order: bytes 0-15
// of the operand are K 32j + 16hf + i of the block's first 32, bytes 16-31
// the second 32).  slot0/slot1 are the swizzled byte offsets of the two chunks.
template <int MB>
__device__ __forceinline__ void load_frags8(const char* sa, const char* sb, int arow, const int (&brow)[4], int slot0,
                                            int slot1, i32x8 (&fa)[MB], i32x8 (&fb)[4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const char* p = sa + arow + m * 32 * kRowBytes;
    fa[m] = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(p + slot0),
                                    *reinterpret_cast<const i32x4*>(p + slot1), 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const char* p = sb + brow[n];
    fb[n] = __builtin_shufflevector(*reinterpret_cast<const i32x4*>(p + slot0),
                                    *reinterpret_cast<const i32x4*>(p + slot1), 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// One 64-wide sub-step of MFMAs with the current step's scales: sa[m] for
// the lane's A row of block m, sb[n] for B block n.
template <int MB>
__device__ __forceinline__ void mfma_step8(const i32x8 (&fa)[MB], const i32x8 (&fb)[4], const int (&sa)[MB],
                                           const int (&sb)[4], f32x16 (&acc)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
      acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[m], fb[n], acc[m][n], 0, 0, 0, sa[m], 0, sb[n]);
}

// Interleave one sub-step: NS scale loads first, two fragment reads after
// each of the first MB+4 MFMAs (a one-block tile has one fragment more than
// MFMAs: its last two reads follow), then the NC copies one per MFMA (reads
// are written before copies in program order, which the compiler keeps for
// LDS reads and LDS copies).
template <int MB, int NC, int NS = 0>
__device__ __forceinline__ void interleave8() {
  constexpr int NR = MB + 4, NP = NR < MB * 4 ? NR : MB * 4;
  constexpr int NM = MB * 4 - NP;
  if (NS > 0) __builtin_amdgcn_sched_group_barrier(0x020, NS, 0);  // scale loads
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
  }
  if (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, 2 * (NR - NP), 0);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 copy
  }
  if (NM > NC) __builtin_amdgcn_sched_group_barrier(0x008, NM - NC, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// An ordering point after which every accumulator has been produced.
template <int MB>
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) asm volatile("" ::"a"(acc[m][n]));
}

// Scales of the 4-step group g (steps 4g .. 4g+3, one per byte): one dword
// per A row of the lane (grouped layout, see GemmArgs) and one uniform dword
// per B block of the wave.
template <int MB, bool GATEUP>
__device__ __forceinline__ void load_scale_group(const GemmArgs& a, const int (&sidx)[MB], int64_t bw0, int64_t bw1,
                                                 int g, uint32_t (&sa)[MB], uint32_t& sb0, uint32_t& sb1) {
  const uint32_t* ag = reinterpret_cast<const uint32_t*>(a.sa) + (int64_t)g * a.n_rows;
#pragma unroll
  for (int m = 0; m < MB; ++m) sa[m] = ag[sidx[m]];
  sb0 = reinterpret_cast<const uint32_t*>(a.sb0)[bw0 + g];
  sb1 = GATEUP ? reinterpret_cast<const uint32_t*>(a.sb1)[bw1 + g] : sb0;
}

// Scale operands of one step: byte `sh/8` of the group's dwords (the
// instruction reads byte 0 of its scale operand).
template <int MB>
__device__ __forceinline__ void step_scales(const uint32_t (&ga)[MB], uint32_t gb0, uint32_t gb1, int sh, int (&sa)[MB],
                                            int (&sb)[4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m) sa[m] = (int)(ga[m] >> sh);
  sb[0] = sb[1] = (int)(gb0 >> sh);
  sb[2] = sb[3] = (int)(gb1 >> sh);
}

template <int WM, bool GATEUP, bool NTB>
__device__ __forceinline__ void gemm_tile_fp8(const GemmArgs& a, char* lds, int e, int nt, int row0, int rows) {
  constexpr int BM = 2 * WM;
  constexpr int MB = WM / 32;
  constexpr int A_PER_WAVE = BM / 8 / 4;
  constexpr int B_PER_WAVE = kBNB / 8 / 4;
  constexpr int NSL = MB + (GATEUP ? 2 : 1);  // vector loads of one scale group

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K = a.K;  // bytes per row = E4M3 values per row
  const int nk = K / kRowBytes;
  const int lrow = lane >> 3;
  const int wr = wave & 1, wc = wave >> 1;

  // A rows through a buffer resource: the rows of the tile past `rows` read
  // as zero codes (no memory traffic, zeros into the matrix cores)
  __amdgpu_buffer_rsrc_t arsrc;
  uint32_t aoff[A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int r = (wave * A_PER_WAVE + i) * 8 + lrow;
    const uint32_t chunk = (uint32_t)((lane & 7) ^ swz_of_row(r)) * 16u;
    if constexpr (GATEUP)
      aoff[i] = r < rows ? (uint32_t)a.row_token[row0 + r] * (uint32_t)K + chunk : kOutOfRange;
    else
      aoff[i] = r < rows ? (uint32_t)r * (uint32_t)K + chunk : kOutOfRange;
  }
  if constexpr (GATEUP)
    arsrc = raw_rsrc(a.a, a.a_bytes);
  else
    arsrc = raw_rsrc(static_cast<const uint8_t*>(a.a) + (int64_t)row0 * K, (uint32_t)rows * (uint32_t)K);

  const uint8_t* bbase;
  uint32_t boff[B_PER_WAVE];
  int64_t bw0, bw1;  // dword index of the wave's B block(s) in the padded scale rows
  const int nkb4 = ((K / 128) + 3) & ~3, nnb = a.N / 128;
  const int ng = (nk + 3) >> 2;  // 4-step scale groups
  if constexpr (GATEUP) {
    bbase = static_cast<const uint8_t*>(wave < 2 ? a.b0 : a.b1) + ((int64_t)e * a.N + nt * 128) * K;
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int rb = ((wave & 1) * B_PER_WAVE + i) * 8 + lrow;
      boff[i] = (uint32_t)rb * (uint32_t)K + ((lane & 7) ^ swz_of_row(rb)) * 16;
    }
    bw0 = bw1 = ((int64_t)e * nnb + nt) * nkb4 / 4;
  } else {
    bbase = static_cast<const uint8_t*>(a.b0) + ((int64_t)e * a.N + nt * kBNB) * K;
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i) {
      const int rb = (wave * B_PER_WAVE + i) * 8 + lrow;
      boff[i] = (uint32_t)rb * (uint32_t)K + ((lane & 7) ^ swz_of_row(rb)) * 16;
    }
    bw0 = bw1 = ((int64_t)e * nnb + nt * 2 + wc) * nkb4 / 4;
  }
  // A scale rows of the lane: fragment m holds row wr*WM + m*32 + lane%32
  int sidx[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) sidx[m] = row0 + min(wr * WM + m * 32 + (lane & 31), rows - 1);

  char* const b_lds = lds + kAStages * kAStage;
  char* const a_dst = lds + wave * A_PER_WAVE * 1024;
  char* const b_dst = b_lds + wave * B_PER_WAVE * 1024;

  f32x16 acc[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;

  const int arow = (wr * WM + (lane & 31)) * kRowBytes;
  int brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if constexpr (GATEUP)
      brow[n] = ((n < 2 ? wc * 64 + n * 32 : 128 + wc * 64 + (n - 2) * 32) + (lane & 31)) * kRowBytes;
    else
      brow[n] = (wc * 128 + n * 32 + (lane & 31)) * kRowBytes;
  }
  const int hf = lane >> 5, sw = swz_of_row(lane & 15);
  const int s00 = ((0 + hf) ^ sw) << 4, s01 = ((2 + hf) ^ sw) << 4;  // sub-step 0
  const int s10 = ((4 + hf) ^ sw) << 4, s11 = ((6 + hf) ^ sw) << 4;  // sub-step 1

  uint32_t ga[MB], gb0, gb1, na[MB], nb0, nb1;  // scales of the current and the next group
  load_scale_group<MB, GATEUP>(a, sidx, bw0, bw1, 0, ga, gb0, gb1);
  // prologue: A and B of steps 0 and 1 in the order of the main loop (B of a
  // step before its A), then wait for step 0
  copy_rows8_buf<0, A_PER_WAVE>(arsrc, aoff, 0, a_dst);
  copy_rows8<NTB, 0, B_PER_WAVE>(bbase, boff, b_dst);
  copy_rows8<NTB, 0, B_PER_WAVE>(bbase + min(1, nk - 1) * kRowBytes, boff, b_dst + kBStage);
  copy_rows8_buf<0, A_PER_WAVE>(arsrc, aoff, min(1, nk - 1) * kRowBytes, a_dst + kAStage);
  wait_vmem_upto<A_PER_WAVE + B_PER_WAVE>();
  __builtin_amdgcn_s_barrier();

  i32x8 fa0[MB], fb0[4], fa1[MB], fb1[4];
  int sbi = 0;
  load_frags8<MB>(lds, b_lds, arow, brow, s00, s01, fa0, fb0);
  // Scale groups: group g+1 is loaded at the start of sub-step 1 of step 4g
  // (after that step's barrier) and becomes current after step 4g+3.  The
  // steps of a group are written out (J = position in the group; the last
  // steps when nk % 4 != 0 take J = -1 and test at run time), so these
  // positions are fixed in the code: the loads are then forced complete by
  // the barrier of step 4g+1 (one step of latency to hide), and the compiler
  // sees them complete before their use instead of inserting a wait for every
  // outstanding copy.
  auto step = [&](int kt, auto J) {
    constexpr int j = decltype(J)::value;
    const bool first = j < 0 ? (kt & 3) == 0 : j == 0;
    const bool last = j < 0 ? (kt & 3) == 3 : j == 3;
    const char* sa = lds + (kt & 1) * kAStage;
    const char* sb = b_lds + sbi * kBStage;
    const int sbn = sbi == kBStages - 1 ? 0 : sbi + 1;
    const int sbf = sbn == kBStages - 1 ? 0 : sbn + 1;
    int sa_k[MB], sb_k[4];
    step_scales<MB>(ga, gb0, gb1, (kt & 3) * 8, sa_k, sb_k);
    // sub-step 0: B of step kt+2 into the stage freed at the last barrier
    load_frags8<MB>(sa, sb, arow, brow, s10, s11, fa1, fb1);
    copy_rows8<NTB, 0, B_PER_WAVE>(bbase + min(kt + 2, nk - 1) * kRowBytes, boff, b_dst + sbf * kBStage);
    mfma_step8<MB>(fa0, fb0, sa_k, sb_k, acc);
    interleave8<MB, B_PER_WAVE>();
    // the wave's reads of the current stages are done and A and B of step
    // kt+1 have landed (only B of step kt+2 was issued after them); after the
    // barrier every wave is past the current stages.  (The empty asm
    // statements consume the accumulators, so code placement cannot sink the
    // sub-step's MFMAs past the barrier, where the matrix cores would sit idle
    // while the wave waits.)
    pin_acc<MB>(acc);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    wait_vmem_upto<B_PER_WAVE>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1: the next scale group (first step of a group), step kt+1's
    // first fragments, and A of step kt+2 into the A stage just freed.  Every
    // copy thus has a full step or more before the barrier that needs it:
    // A from here to the next step's barrier, B from sub-step 0 to the
    // barrier of the step after next.
    if (first) load_scale_group<MB, GATEUP>(a, sidx, bw0, bw1, min((kt >> 2) + 1, ng - 1), na, nb0, nb1);
    load_frags8<MB>(lds + ((kt + 1) & 1) * kAStage, b_lds + sbn * kBStage, arow, brow, s00, s01, fa0, fb0);
    copy_rows8_buf<0, A_PER_WAVE>(arsrc, aoff, min(kt + 2, nk - 1) * kRowBytes, a_dst + (kt & 1) * kAStage);
    mfma_step8<MB>(fa1, fb1, sa_k, sb_k, acc);
    if constexpr (j == 0)
      interleave8<MB, A_PER_WAVE, NSL>();
    else
      interleave8<MB, A_PER_WAVE>();
    pin_acc<MB>(acc);
    if (last) {
#pragma unroll
      for (int m = 0; m < MB; ++m) ga[m] = na[m];
      gb0 = nb0;
      gb1 = nb1;
    }
    sbi = sbn;
  };
  const int nfull = nk & ~3;
  for (int kt = 0; kt < nfull; kt += 4) {
    step(kt, std::integral_constant<int, 0>());
    step(kt + 1, std::integral_constant<int, 1>());
    step(kt + 2, std::integral_constant<int, 2>());
    step(kt + 3, std::integral_constant<int, 3>());
  }
  for (int kt = nfull; kt < nk; ++kt) step(kt, std::integral_constant<int, -1>());
  wait_vmem_upto<0>();

  if constexpr (GATEUP) {
    // SwiGLU into an fp32 tile in LDS (rows padded to 132 floats: a row's 16
    // rows apart fall in distinct bank groups), then one thread per row: the
    // row's maximum over its 128 columns (this item's 128-wide block of h),
    // the UE8M0 scale, and the E4M3 codes written 16 bytes at a time
    constexpr int kTS = 132;
    float* tile = reinterpret_cast<float*>(lds);  // [BM][kTS]
    __syncthreads();                              // every wave is done with the stages
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * WM + m * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const float g = acc[m][n][r], u = acc[m][n + 2][r];
          tile[row * kTS + wc * 64 + n * 32 + (lane & 31)] = swiglu(g, u);
        }
      }
    __syncthreads();
    const int row = tid;
    if (row < BM && row < rows) {
      const f32x4* src = reinterpret_cast<const f32x4*>(tile + row * kTS);
      float mx = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const f32x4 v = src[c];
        mx = fmaxf(mx, fmaxf(fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                             fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]))));
      }
      const int p = e8m0_exp_of_amax(mx);
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.c) + (int64_t)(row0 + row) * a.N + nt * 128);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = src[c * 4 + i];
          w[i] = e4m3_pair(__builtin_amdgcn_ldexpf(v[0], -p), __builtin_amdgcn_ldexpf(v[1], -p)) |
                 (e4m3_pair(__builtin_amdgcn_ldexpf(v[2], -p), __builtin_amdgcn_ldexpf(v[3], -p)) << 16);
        }
        dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      a.sc[((int64_t)(nt >> 2) * a.n_rows + row0 + row) * 4 + (nt & 3)] = (uint8_t)(p + 127);
    }
  } else if (a.c16 == nullptr || e >= a.n_routed) {
    // fp32 expert rows (shared experts' rows at row - routed_rows when the
    // routed rows go to c16), written directly from the MFMA layout
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr * WM + m * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row >= rows) continue;
        const int64_t orow_i = (int64_t)(row0 + row) - (a.c16 ? a.routed_rows : 0);
        float* orow = static_cast<float*>(a.c) + orow_i * a.N;
#pragma unroll
        for (int n = 0; n < 4; ++n) orow[nt * kBNB + wc * 128 + n * 32 + (lane & 31)] = acc[m][n][r];
      }
    }
  } else {
    // bf16 routed rows through LDS: each wave stages its WM x 128 sub-tile in
    // a region of its own (rows padded by 16 bytes) and writes whole row
    // segments with 16-byte stores (an eighth of the store instructions of
    // writing the MFMA layout directly)
    constexpr int P = 128 * 2 + 16;
    __syncthreads();  // every wave is done with the stages
    char* const ep = lds + wave * (kWM * P);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          *reinterpret_cast<bf16*>(ep + (m * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)) * P + (n * 32 + (lane & 31)) * 2) =
              (bf16)acc[m][n][r];
    const int rows_w = rows - wr * WM;  // rows of this wave's sub-tile that exist (may be <= 0)
    bf16* const cw = static_cast<bf16*>(a.c16) + (int64_t)(row0 + wr * WM) * a.N + nt * kBNB + wc * 128;
#pragma unroll
    for (int i = 0; i < WM * 16 / 64; ++i) {
      const int idx = i * 64 + lane, row = idx >> 4, ch = idx & 15;
      const i32x4 v = *reinterpret_cast<const i32x4*>(ep + row * P + ch * 16);
      if (row < rows_w) *reinterpret_cast<i32x4*>(cw + (int64_t)row * a.N + ch * 8) = v;
    }
  }
}

// Weight cache policy as in the bf16 kernels: NT = 2 per item (non-temporal
// for an expert whose rows fit one row tile, gate/up), 1 every item, 0 none.
template <int WM, bool GATEUP, int NT>
__device__ __forceinline__ void gemm_tile_fp8_of(const GemmArgs& a, char* lds, const Work& w, int nt) {
  if (NT == 1 || (NT == 2 && w.single))
    gemm_tile_fp8<WM, GATEUP, true>(a, lds, w.e, nt, w.row0, w.rows);
  else
    gemm_tile_fp8<WM, GATEUP, false>(a, lds, w.e, nt, w.row0, w.rows);
}

template <bool GATEUP, int NT>
__global__ __launch_bounds__(256, 1) void expert_gemm_fp8(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  Work w;
  if (!work_of_block(a, 2 * kWM, w, reinterpret_cast<int*>(lds))) return;
  if (!w.pair) {
    // a last row tile of 129-192 rows: three 32-row blocks per wavefront
    if (w.rows > 3 * kWM / 2)
      gemm_tile_fp8_of<kWM, GATEUP, NT>(a, lds, w, w.nt);
    else
      gemm_tile_fp8_of<3 * kWM / 4, GATEUP, NT>(a, lds, w, w.nt);
  } else if (w.rows > kWM / 2) {
    gemm_tile_fp8_of<kWM / 2, GATEUP, NT>(a, lds, w, w.nt);
    if (w.nt + 1 < a.n_tiles) {
      __syncthreads();
      gemm_tile_fp8_of<kWM / 2, GATEUP, NT>(a, lds, w, w.nt + 1);
    }
  } else {
    // a short tile of at most 64 rows: one 32-row block per wavefront
    gemm_tile_fp8_of<kWM / 4, GATEUP, NT>(a, lds, w, w.nt);
    if (w.nt + 1 < a.n_tiles) {
      __syncthreads();
      gemm_tile_fp8_of<kWM / 4, GATEUP, NT>(a, lds, w, w.nt + 1);
    }
  }
}

// 1 x 128 tile quantisation: 16 lanes per tile, 8 values per lane.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(QuantArgs a) {
  const int tiles_per_row = a.K / 128;
  const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (tile >= a.rows * tiles_per_row) return;
  const int64_t row = tile / tiles_per_row;
  const int tb = (int)(tile - row * tiles_per_row);
  const int sub = threadIdx.x & 15;
  const int64_t off = row * a.K + tb * 128 + sub * 8;
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.in) + off);
  float f[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = (float)v[i];
    m = fmaxf(m, __builtin_fabsf(f[i]));
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  const int p = e8m0_exp_of_amax(m);
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t lo = e4m3_pair(__builtin_amdgcn_ldexpf(f[4 * i], -p), __builtin_amdgcn_ldexpf(f[4 * i + 1], -p));
    const uint32_t hi =
        e4m3_pair(__builtin_amdgcn_ldexpf(f[4 * i + 2], -p), __builtin_amdgcn_ldexpf(f[4 * i + 3], -p));
    w[i] = lo | (hi << 16);
  }
  *reinterpret_cast<uint2*>(a.codes + off) = make_uint2(w[0], w[1]);
  if (sub == 0) a.scales[row * a.sstride + tb] = (uint8_t)(p + 127);
}

// Row-space copies of the tokens' x scales in the grouped layout:
// out[((kb/4) * n_rows + r) * 4 + kb%4] = sx[row_token[r], kb] (unused rows
// are skipped).
__global__ __launch_bounds__(256) void row_scales_kernel(RowScaleArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.n_rows * a.nkb) return;
  const int kb = (int)(i / a.n_rows), r = (int)(i - (int64_t)kb * a.n_rows);
  const int t = a.row_token[r];
  if (t >= 0) a.out[((int64_t)(kb >> 2) * a.n_rows + r) * 4 + (kb & 3)] = a.sx[(int64_t)t * a.nkb + kb];
}

// Weight block scales with rows padded to a multiple of 4 bytes (one
// matrix per blockIdx.y): dst[row, kb] = src[row, kb], pad bytes 127.
__global__ __launch_bounds__(256) void pack_scales_kernel(ScalePackArgs a) {
  const ScalePackArgs::Mat& m = a.m[blockIdx.y];
  const int nkb4 = (m.nkb + 3) & ~3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)m.rows * nkb4) return;
  const int64_t r = i / nkb4;
  const int kb = (int)(i - r * nkb4);
  m.dst[i] = kb < m.nkb ? m.src[r * m.nkb + kb] : (uint8_t)127;
}

}  // namespace

hipError_t launch_pack_scales(const ScalePackArgs& a, hipStream_t s) {
  int64_t n = 0;
  for (int j = 0; j < 3; ++j) n = std::max<int64_t>(n, (int64_t)a.m[j].rows * ((a.m[j].nkb + 3) & ~3));
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((n + 255) / 256), 3), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row_scales(const RowScaleArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_rows * a.nkb;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup_fp8(const GemmArgs& a, int64_t mtile_bound, hipStream_t s) {
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((expert_gemm_fp8<true, 2>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const GemmArgs& a, int64_t mtile_bound, hipStream_t s) {
  const int64_t grid = mtile_bound * a.n_tiles;
  if (grid <= 0) return hipSuccess;
  if (a.stream_b)
    hipLaunchKernelGGL((expert_gemm_fp8<false, 1>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((expert_gemm_fp8<false, 0>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t s) {
  const int64_t tiles = a.rows * (a.K / 128);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)((tiles + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}
