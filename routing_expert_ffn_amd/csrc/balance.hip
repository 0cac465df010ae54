// Auxiliary-loss-free load balancing step and load telemetry for gfx950.
//
// "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选 8 个", the
// paragraph on the bias: after each step, an expert that received more tokens
// than the mean has its selection-only bias lowered by gamma and one that
// received fewer has it raised (an expert exactly at the mean keeps it); the
// monitoring paragraph of the same section and the expert-call entropy of
// "GPT-4稀疏激活原理：2%参数调用背后的MoE工程实践", section 4.4, are the
// telemetry.  One workgroup, one thread per expert; the
// mean test is exact integer arithmetic and the reductions run in a fixed
// order, so the result is deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace {

constexpr int kBalanceThreads = 512;  // >= MOE_MAX_EXPERTS

// Sum over the workgroup in a fixed tree order (buf: kBalanceThreads values).
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int half = kBalanceThreads / 2; half > 0; half >>= 1) {
    if (tid < half) buf[tid] = buf[tid] + buf[tid + half];
    __syncthreads();
  }
  const T r = buf[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kBalanceThreads) void balance_kernel(BalanceArgs a) {
  __shared__ long long ibuf[kBalanceThreads];
  __shared__ double dbuf[kBalanceThreads];
  const int e = threadIdx.x;
  const bool mine = e < a.E;
  const long long n = mine ? (long long)a.counts[e] : 0;
  const long long N = block_sum<long long>(n, ibuf);
  int over = 0, under = 0;
  if (mine && N > 0 && a.bias) {
    const long long scaled = n * (long long)a.E;
    if (scaled > N) {
      a.bias[e] = a.bias[e] - a.gamma;
      over = 1;
    } else if (scaled < N) {
      a.bias[e] = a.bias[e] + a.gamma;
      under = 1;
    }
  } else if (mine && N > 0) {
    const long long scaled = n * (long long)a.E;
    over = scaled > N;
    under = scaled < N;
  }
  const double p = (mine && N > 0) ? (double)n / (double)N : 0.0;
  if (mine && a.share) a.share[e] = (float)p;
  const double ent = block_sum<double>(p > 0.0 ? -p * log(p) : 0.0, dbuf);
  // the largest share: a max over the same tree
  dbuf[e] = p;
  __syncthreads();
  for (int half = kBalanceThreads / 2; half > 0; half >>= 1) {
    if (e < half) dbuf[e] = fmax(dbuf[e], dbuf[e + half]);
    __syncthreads();
  }
  const double mx = dbuf[0];
  __syncthreads();
  const long long n_over = block_sum<long long>(over, ibuf);
  const long long n_under = block_sum<long long>(under, ibuf);
  if (e == 0 && a.stats) {
    a.stats[0] = (float)ent;
    a.stats[1] = (float)mx;
    a.stats[2] = (float)n_over;
    a.stats[3] = (float)n_under;
  }
}

}  // namespace

hipError_t launch_balance(const BalanceArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(kBalanceThreads), 0, s, a);
  return hipGetLastError();
}
