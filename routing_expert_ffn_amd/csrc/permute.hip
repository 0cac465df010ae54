// Token permutation (dispatch by expert) for gfx950.
//
// The pages ask for tokens to be regrouped by expert with scatter/gather
// instead of per-expert masks ("MoE架构揭秘", section 4.1) and describe a
// router output packed with token ids and dispatched in one kernel ("GPT-4
// Has 1.8 Trillion Parameters. It Uses 2% of Them Per Token", section 4.2).
// Rows are ordered by (expert asc, token asc) so the result is unique:
//   count   one wavefront per 64-token chunk: LDS bit masks mask[e] (bit =
//           token of the chunk routed to e, set with LDS atomics), chunk
//           count = popcount;
//   scan    per expert, exclusive prefix over chunks (chunk base) and the
//           total; exclusive prefix over experts (offsets);
//   scatter row = offsets[e] + base[chunk][e] + popcount(mask[e] below the
//           token's bit), no float atomics and no order dependence.
#include "common.hpp"
#include "kernels.hpp"

namespace {

constexpr int kChunk = 64;

__device__ __forceinline__ void build_masks(const PermuteArgs& a, int chunk, uint64_t* mask) {
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += MOE_WAVE) mask[e] = 0;
  __syncthreads();
  const int t = chunk * kChunk + lane;
  if (t < a.T) {
    for (int j = 0; j < a.k; ++j) {
      const int e = a.topk_idx[(int64_t)t * a.k + j];
      if (e >= 0 && e < a.E) atomicOr((unsigned long long*)&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(64) void perm_count_kernel(PermuteArgs a) {
  extern __shared__ uint64_t lds_mask[];
  const int chunk = blockIdx.x;
  build_masks(a, chunk, lds_mask);
  for (int e = threadIdx.x; e < a.E; e += MOE_WAVE)
    a.chunk_cnt[(int64_t)chunk * a.E + e] = __popcll(lds_mask[e]);
}

// One workgroup of 1024 threads: `tpe` threads per expert split the chunks,
// then the experts are scanned.
__global__ __launch_bounds__(1024) void perm_scan_kernel(PermuteArgs a) {
  extern __shared__ int32_t lds_scan[];  // [1024] partial sums, then [E] totals
  const int tid = threadIdx.x;
  const int tpe = max(1, 1024 / a.E);                // threads per expert
  const int per = (a.nchunks + tpe - 1) / tpe;       // chunks per thread
  int32_t* part = lds_scan;
  int32_t* tot = lds_scan + 1024;
  for (int e0 = 0; e0 < a.E; e0 += 1024 / tpe) {
    const int e = e0 + tid / tpe;
    const int q = tid % tpe;
    const bool act = e < a.E && tid / tpe < 1024 / tpe;
    int sum = 0;
    if (act) {
      const int c1 = min(a.nchunks, (q + 1) * per);
      for (int c = q * per; c < c1; ++c) sum += a.chunk_cnt[(int64_t)c * a.E + e];
    }
    part[tid] = sum;
    __syncthreads();
    int before = 0;
    if (act) {
      for (int r = 0; r < q; ++r) before += part[tid - q + r];
      int run = before;
      const int c1 = min(a.nchunks, (q + 1) * per);
      for (int c = q * per; c < c1; ++c) {
        const int v = a.chunk_cnt[(int64_t)c * a.E + e];
        a.chunk_base[(int64_t)c * a.E + e] = run;
        run += v;
      }
      if (q == tpe - 1) tot[e] = run;
    }
    __syncthreads();
  }
  // exclusive scan of the totals over experts (single thread per 1024 is
  // enough: E <= 1024 and this runs once per layer call)
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < a.E; ++e) {
      a.counts[e] = tot[e];
      a.offsets[e] = run;
      run += tot[e];
    }
    a.offsets[a.E] = run;
    tot[0] = run;  // reuse: number of assigned rows
  }
  __syncthreads();
  const int assigned = tot[0];
  const int64_t routed_rows = (int64_t)a.T * a.k;
  for (int64_t r = assigned + tid; r < routed_rows; r += 1024) a.row_token[r] = -1;
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(PermuteArgs a) {
  extern __shared__ uint64_t lds_mask[];
  const int chunk = blockIdx.x;
  build_masks(a, chunk, lds_mask);
  const int lane = threadIdx.x;
  const int t = chunk * kChunk + lane;
  if (t >= a.T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < a.k; ++j) {
    const int e = a.topk_idx[(int64_t)t * a.k + j];
    int row = -1;
    if (e >= 0 && e < a.E) {
      row = a.offsets[e] + a.chunk_base[(int64_t)chunk * a.E + e] + __popcll(lds_mask[e] & below);
      a.row_token[row] = t;
    }
    a.slot_row[(int64_t)t * a.k + j] = row;
  }
  const int64_t base = (int64_t)a.T * a.k;
  for (int s = 0; s < a.S; ++s) a.row_token[base + (int64_t)s * a.T + t] = t;
}

}  // namespace

hipError_t launch_perm_count(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(perm_count_kernel, dim3(a.nchunks), dim3(64), sizeof(uint64_t) * a.E, s, a);
  return hipGetLastError();
}

hipError_t launch_perm_scan(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), sizeof(int32_t) * (1024 + a.E), s, a);
  return hipGetLastError();
}

hipError_t launch_perm_scatter(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(a.nchunks), dim3(64), sizeof(uint64_t) * a.E, s, a);
  return hipGetLastError();
}
