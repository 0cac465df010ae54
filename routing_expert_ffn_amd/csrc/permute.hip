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
//   scan    one workgroup per expert: exclusive prefix over chunks (chunk
//           base) and the total (count);
//   scatter each chunk's workgroup scans the counts over experts (offsets;
//           chunk 0 stores them), row = offsets[e] + base[chunk][e] +
//           popcount(mask[e] below the token's bit); no float atomics and
//           no order dependence.
#include <algorithm>

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

// Exclusive prefix sum over the 256 threads of a workgroup (sh: 4 ints of
// LDS); *total receives the sum of all values.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < MOE_WAVE; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == MOE_WAVE - 1) sh[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sh[w];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  return before + incl - v;
}

// One workgroup per expert: thread i owns a contiguous range of chunks.
__global__ __launch_bounds__(256) void perm_scan_kernel(PermuteArgs a) {
  __shared__ int sh[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int per = (a.nchunks + 255) / 256;
  const int c0 = min(a.nchunks, tid * per), c1 = min(a.nchunks, c0 + per);
  int sum = 0;
  int c = c0;
  for (; c + 8 <= c1; c += 8) {
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = a.chunk_cnt[(int64_t)(c + i) * a.E + e];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += q[i];
  }
  for (; c < c1; ++c) sum += a.chunk_cnt[(int64_t)c * a.E + e];
  int total;
  int run = block_exclusive_scan_256(sum, sh, &total);
  for (c = c0; c < c1; ++c) {
    const int v = a.chunk_cnt[(int64_t)c * a.E + e];
    a.chunk_base[(int64_t)c * a.E + e] = run;
    run += v;
  }
  if (tid == 0) a.counts[e] = total;
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(PermuteArgs a) {
  extern __shared__ uint64_t lds_mask[];  // [E] masks, then [E+1] offsets
  int32_t* off = reinterpret_cast<int32_t*>(lds_mask + a.E);
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x;
  // offsets: exclusive prefix of the counts over experts, lane l summing the
  // experts [l*per, (l+1)*per) (E <= 512)
  {
    const int per = (a.E + MOE_WAVE - 1) / MOE_WAVE;
    const int e0 = min(a.E, lane * per), e1 = min(a.E, e0 + per);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += a.counts[e];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
    for (int e = e0; e < e1; ++e) {
      off[e] = run;
      run += a.counts[e];
    }
    if (lane == MOE_WAVE - 1) off[a.E] = incl;
  }
  build_masks(a, chunk, lds_mask);  // its barriers also publish off[]
  if (chunk == 0)
    for (int e = lane; e <= a.E; e += MOE_WAVE) a.offsets[e] = off[e];
  // routed rows past the assigned ones (dropped slots) hold no token
  const int64_t routed_rows = (int64_t)a.T * a.k;
  for (int64_t r = off[a.E] + (int64_t)chunk * kChunk + lane; r < routed_rows; r += (int64_t)a.nchunks * kChunk)
    a.row_token[r] = -1;
  const int t = chunk * kChunk + lane;
  if (t >= a.T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < a.k; ++j) {
    const int e = a.topk_idx[(int64_t)t * a.k + j];
    int row = -1;
    if (e >= 0 && e < a.E) {
      row = off[e] + a.chunk_base[(int64_t)chunk * a.E + e] + __popcll(lds_mask[e] & below);
      a.row_token[row] = t;
    }
    a.slot_row[(int64_t)t * a.k + j] = row;
  }
  const int64_t base = (int64_t)a.T * a.k;
  for (int s = 0; s < a.S; ++s) a.row_token[base + (int64_t)s * a.T + t] = t;
}

// Drop mode: an assignment whose rank in its expert's token-ordered rows is
// at or beyond the capacity is dropped (first come, first served is then
// exactly "keep while the expert holds fewer than C tokens").
__global__ __launch_bounds__(256) void drop_kernel(DropArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)a.T * a.k) {
    const int e = a.topk_idx[i];
    if (e >= 0 && e < a.E && a.slot_row[i] - a.offsets[e] >= a.capacity) {
      a.topk_idx[i] = -1;
      a.topk_w[i] = 0.0f;
    }
  }
  if (a.counts && i < a.E) a.counts[i] = min(a.full_counts[i], a.capacity);
}

}  // namespace

hipError_t launch_perm_count(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(perm_count_kernel, dim3(a.nchunks), dim3(64), sizeof(uint64_t) * a.E, s, a);
  return hipGetLastError();
}

hipError_t launch_perm_scan(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(a.E), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_perm_scatter(const PermuteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const size_t lds = sizeof(uint64_t) * a.E + sizeof(int32_t) * (a.E + 1);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(a.nchunks), dim3(64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_drop(const DropArgs& a, hipStream_t s) {
  const int64_t n = std::max<int64_t>((int64_t)a.T * a.k, a.E);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(drop_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}
