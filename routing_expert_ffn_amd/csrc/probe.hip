// Attainable-rate probes of the part the layer runs on: the sustained dense
// bf16 matrix-core rate and the HBM streaming read rate, measured with this
// library's own kernels so the layer's timings can be set against what the
// chip delivers under the same power limit, not only against its nominal
// peaks.
//
// mfma_probe_kernel: every wavefront issues independent chains of
//   v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic inside
//   the loop), eight accumulators so no MFMA waits for the previous one of its
//   chain.  The operands are pseudo-random bf16 values: four A and four B
//   fragments taken in turn (the realistic case: the multiplier inputs
//   change between instructions, as in a GEMM), or one fixed pair (far fewer
//   toggling bits, less power, a higher clock under the power limit).
// mfma_fp8_probe_kernel: the same with v_mfma_scale_f32_32x32x64_f8f6f4 on
//   E4M3 operands and unit block scales, the instruction of the FP8 expert
//   GEMMs.
// read_probe_kernel: a grid-stride read of a device buffer in 16-byte pieces,
//   eight loads in flight per lane, into registers with the default or the
//   non-temporal cache policy, or as global->LDS copies with either policy
//   (the form the expert GEMMs stream their operands in); a per-lane XOR of
//   what was read is written out.
#include "common.hpp"
#include "kernels.hpp"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 256;
constexpr int kMfmaChains = 8;
constexpr int kReadUnroll = 8;

// Pseudo-random bf16 in [-2, 2] from a lane and an index (a few multiply /
// xor-shift rounds; any bits will do, what matters is that they vary).
__device__ __forceinline__ bf16 probe_value(uint32_t a, uint32_t b) {
  uint32_t h = a * 0x9E3779B1u ^ (b + 0x7F4A7C15u) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0xC2B2AE3Du;
  h ^= h >> 13;
  return (bf16)((float)(h & 0xFFFFu) * (4.0f / 65536.0f) - 2.0f);
}

// VARY: every MFMA of a round takes a different A or B fragment (four of
// each, as the fragments of a 4 x 4 block of a GEMM tile), so the multiplier
// inputs change from one instruction to the next; otherwise one fixed pair.
template <bool VARY>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int64_t iters, float* sink) {
  const int tid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[f][i] = probe_value((uint32_t)tid, (uint32_t)(f * 8 + i));
      b[f][i] = probe_value((uint32_t)tid + 0x10000u, (uint32_t)(f * 8 + i));
    }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) {
      const int fa = VARY ? (c & 3) : 0, fb = VARY ? ((c + (c >> 2)) & 3) : 0;
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fa], b[fb], acc[c], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[tid] = s;
}

// Four pseudo-random E4M3 codes in a dword; bit 3 of each byte cleared, so
// no code is the NaN pattern (0x7F / 0xFF).
__device__ __forceinline__ int probe_fp8x4(uint32_t a, uint32_t b) {
  uint32_t h = a * 0x9E3779B1u ^ (b + 0x7F4A7C15u) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0xC2B2AE3Du;
  h ^= h >> 13;
  return (int)(h & 0xF7F7F7F7u);
}

template <bool VARY>
__global__ __launch_bounds__(kProbeThreads) void mfma_fp8_probe_kernel(int64_t iters, float* sink) {
  const int tid = blockIdx.x * kProbeThreads + threadIdx.x;
  i32x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[f][i] = probe_fp8x4((uint32_t)tid, (uint32_t)(f * 8 + i));
      b[f][i] = probe_fp8x4((uint32_t)tid + 0x10000u, (uint32_t)(f * 8 + i));
    }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) {
      const int fa = VARY ? (c & 3) : 0, fb = VARY ? ((c + (c >> 2)) & 3) : 0;
      // formats 0/0 (E4M3 both), scale exponent bytes 127 (x 1)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fa], b[fb], acc[c], 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[tid] = s;
}

// One 16-byte piece per lane at index j: into registers (MODE 0 plain, 1
// non-temporal) or copied to the wave's LDS slot u (MODE 2 default policy,
// 3 non-temporal).
template <int MODE>
__device__ __forceinline__ void read_piece(const u32x4* p, int64_t j, char* slot, u32x4& acc) {
  if constexpr (MODE == 0) {
    acc ^= p[j];
  } else if constexpr (MODE == 1) {
    acc ^= __builtin_nontemporal_load(p + j);
  } else if constexpr (MODE == 2) {
    copy16(reinterpret_cast<const bf16*>(p + j), slot);
  } else {
    copy16_nt(reinterpret_cast<const bf16*>(p + j), slot);
  }
}

template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* p, int64_t n16, float* sink) {
  __shared__ __attribute__((aligned(1024))) char lds[kReadUnroll * 4 * 1024];
  const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  // wave w's slot for the u-th piece of a round: 1 KB at u * 4 KB + w * 1 KB
  char* const wslot = lds + (threadIdx.x >> 6) * 1024;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t full = n16 / (kReadUnroll * stride) * (kReadUnroll * stride);
  int64_t i = tid;
  for (; i < full; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
    if constexpr (MODE <= 1) {
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) {
        v[u] = u32x4{0u, 0u, 0u, 0u};
        read_piece<MODE>(p, i + u * stride, nullptr, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    } else {
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) read_piece<MODE>(p, i + u * stride, wslot + u * 4096, acc);
    }
  }
  for (; i < n16; i += stride) read_piece<MODE>(p, i, wslot, acc);
  if constexpr (MODE >= 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    acc = *reinterpret_cast<const u32x4*>(lds + threadIdx.x * 16);
  }
  sink[tid] = __uint_as_float((acc.x ^ acc.y ^ acc.z ^ acc.w) & 0x007FFFFFu);
}

}  // namespace

int probe_threads() { return kProbeThreads; }

double probe_mfma_flops_per_iter_block(int fp8) {
  return (double)(kProbeThreads / 64) * kMfmaChains * 32.0 * 32.0 * (fp8 ? 64.0 : 16.0) * 2.0;
}

hipError_t launch_probe_mfma(int fp8, int vary, int blocks, int64_t iters, float* sink, hipStream_t s) {
  if (fp8 && vary)
    hipLaunchKernelGGL((mfma_fp8_probe_kernel<true>), dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
  else if (fp8)
    hipLaunchKernelGGL((mfma_fp8_probe_kernel<false>), dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
  else if (vary)
    hipLaunchKernelGGL((mfma_probe_kernel<true>), dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<false>), dim3(blocks), dim3(kProbeThreads), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_read(int mode, int blocks, const void* buf, int64_t n16, float* sink, hipStream_t s) {
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (mode == 0)
    hipLaunchKernelGGL((read_probe_kernel<0>), dim3(blocks), dim3(kProbeThreads), 0, s, p, n16, sink);
  else if (mode == 1)
    hipLaunchKernelGGL((read_probe_kernel<1>), dim3(blocks), dim3(kProbeThreads), 0, s, p, n16, sink);
  else if (mode == 2)
    hipLaunchKernelGGL((read_probe_kernel<2>), dim3(blocks), dim3(kProbeThreads), 0, s, p, n16, sink);
  else
    hipLaunchKernelGGL((read_probe_kernel<3>), dim3(blocks), dim3(kProbeThreads), 0, s, p, n16, sink);
  return hipGetLastError();
}
