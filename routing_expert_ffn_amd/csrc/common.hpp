// Internal types and helpers of the gfx950 MoE kernels (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

// Largest routed expert count the router kernels hold in registers (8 per lane).
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_GROUPS 32
#define MOE_MAX_TOPK 32

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) {
  return (float)v;
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return (bf16)v;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Lane exchanges inside each row of 16 lanes through DPP, for reductions of
// the whole (fully active) wavefront: lane ^ 1 and lane ^ 2 (quad
// permutations [1,0,3,2] and [2,3,0,1]), then the mirror of each half row
// (lane i <-> 7 - i) and of each row (i <-> 15 - i).  Once every lane of a
// quad (of a half row) holds that quad's (half row's) reduction, the mirror
// pairs it with the other quad (half row), so four exchanges reduce a row.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of a 64-bit key over the wavefront (every lane gets it): rows
// reduced through DPP, then the four row maxima read out.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppQuadXor1>(v));
  v = max_u64(v, dpp_u64<kDppQuadXor2>(v));
  v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppMirror>(v));
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)), max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 1; off < MOE_WAVE; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger int).
// -0 is first turned into +0 so that the two zeros tie.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rank key: higher score first, lower expert index on equal scores.  Key 0 is
// "nothing" (never produced for a real expert: ordered_bits of a finite
// float is never 0 in the high word together with index slot 0xFFFFFFFF).
__device__ __forceinline__ uint64_t rank_key(float score, int e) {
  return ((uint64_t)ordered_bits(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu)); }

// SwiGLU of one gate/up pair: silu(g) * u = g * u / (1 + e^-g), the
// reciprocal from v_rcp_f32 (about 1 ulp) instead of a correctly rounded
// division: the result is rounded to bf16 or E4M3 next, and the division's
// refinement steps cost ~15 VALU instructions for each of the 128 values a
// lane produces per tile.  Large negative g gives e^-g = inf, rcp = 0: -0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---- global->LDS staging of 128-byte tile rows (grouped GEMMs, router GEMM)

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
// (A plain function: the builtin must not sit in a template or lambda, whose
// host-side instantiation would drop the kernel's launch stub.)
__device__ __forceinline__ void copy16(const bf16* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}

// copy16 with the non-temporal cache policy, for data read exactly once (the
// expert weights when every expert has at most one row tile).
__device__ __forceinline__ void copy16_nt(const bf16* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 2);
}

// Raw buffer resource over [base, base + bytes), bytes < 2^31: a buffer load
// whose offset lies past the end returns zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Lane offset that is past the end of every resource made by raw_rsrc.
constexpr uint32_t kOutOfRange = 0x80000000u;

// The buffer form of copy16: lane L reads 16 bytes at voff + soff of the
// resource (zeros when voff is out of range) into LDS bytes [dst + 16*L, +16).
__device__ __forceinline__ void copy16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, soff, 0, 0);
}
