// Gate-weighted combine of the MoE layer for gfx950:
//   out[t] = sum_j w[t,j] * y_routed[slot_row[t,j]] + sum_s y_shared[s*T + t]
// ("15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个", the
// router sketch's last line: weighted routed experts plus the shared expert).
// One workgroup per token (one thread per 8 values of the row); 16-byte
// non-temporal loads of the expert rows (each is read exactly once; routed
// rows fp32 or bf16, shared rows fp32) and non-temporal stores of the output
// (hundreds of MB at prefill sizes, more than the caches hold), fp32
// accumulation in a fixed order (slots, then shared experts), so the result
// is deterministic.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace {

constexpr int kSlotBatch = 8;  // routed rows loaded together per thread

template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  struct Raw {
    bf16x8 x;
  };
  static __device__ __forceinline__ Raw load_raw(const bf16* p) {
    return Raw{__builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p))};
  }
  static __device__ __forceinline__ float at(const Raw& r, int i) { return (float)r.x[i]; }
  static __device__ __forceinline__ void load(const bf16* p, float (&v)[8]) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  }
  static __device__ __forceinline__ void store(bf16* p, const float (&v)[8]) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (bf16)v[i];
    __builtin_nontemporal_store(x, reinterpret_cast<bf16x8*>(p));
  }
};
template <>
struct Vec8<float> {
  struct Raw {
    f32x4 a, b;
  };
  static __device__ __forceinline__ Raw load_raw(const float* p) {
    return Raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
               __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4))};
  }
  static __device__ __forceinline__ float at(const Raw& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[i + 4] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = v[i];
      b[i] = v[i + 4];
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
  }
};

template <typename TR, typename TO>
__global__ __launch_bounds__(1024) void combine_kernel(CombineArgs a) {
  __shared__ int32_t srow[MOE_MAX_TOPK];
  __shared__ float sw[MOE_MAX_TOPK];
  const int t = blockIdx.x;
  if (threadIdx.x < a.k) {
    srow[threadIdx.x] = a.slot_row[(int64_t)t * a.k + threadIdx.x];
    sw[threadIdx.x] = a.topk_w[(int64_t)t * a.k + threadIdx.x];
  }
  __syncthreads();
  const TR* y = static_cast<const TR*>(a.y_routed);
  TO* out = static_cast<TO*>(a.out) + (int64_t)t * a.H;
  for (int c = threadIdx.x * 8; c < a.H; c += blockDim.x * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // the first shared expert's row is loaded with the first batch and
    // added after the slots
    typename Vec8<float>::Raw sh;
    if (a.S > 0) sh = Vec8<float>::load_raw(a.y_shared + (int64_t)t * a.H + c);
    // slots in batches of kSlotBatch: every slot of a batch loads (raw, no
    // conversion, so no load waits for another) before any is added; an
    // empty slot reads row 0 and discards it
    for (int j0 = 0; j0 < a.k; j0 += kSlotBatch) {
      typename Vec8<TR>::Raw v[kSlotBatch];
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        const int j = j0 + jj;
        if (j < a.k) {
          const int r = srow[j];
          v[jj] = Vec8<TR>::load_raw(y + (int64_t)(r >= 0 ? r : 0) * a.H + c);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        const int j = j0 + jj;
        if (j < a.k) {
          const bool live = srow[j] >= 0;
          const float w = sw[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = live ? acc[i] + w * Vec8<TR>::at(v[jj], i) : acc[i];
        }
      }
    }
    if (a.S > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += Vec8<float>::at(sh, i);
    }
    for (int s = 1; s < a.S; ++s) {
      float v[8];
      Vec8<float>::load(a.y_shared + ((int64_t)s * a.T + t) * a.H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    Vec8<TO>::store(out + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, int out_dtype, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  (void)dtype;  // expert rows are fp32 for every input dtype
  // one pass over the row: H/8 threads (a multiple of 64), at most 1024
  const int threads = std::min(1024, std::max(64, ((a.H / 8 + 63) / 64) * 64));
  dim3 grid(a.T), block(threads);
  if (a.routed_bf16 && out_dtype == 1)
    hipLaunchKernelGGL((combine_kernel<bf16, bf16>), grid, block, 0, s, a);
  else if (a.routed_bf16)
    hipLaunchKernelGGL((combine_kernel<bf16, float>), grid, block, 0, s, a);
  else if (out_dtype == 1)
    hipLaunchKernelGGL((combine_kernel<float, bf16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<float, float>), grid, block, 0, s, a);
  return hipGetLastError();
}
