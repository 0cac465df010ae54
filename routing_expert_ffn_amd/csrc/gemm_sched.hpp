// Work items of the grouped expert GEMMs (shared by the bf16 and FP8 kernels):
// the flat list of (expert, column tile, row tile) items built from the
// device-side schedule, and its XCD-aware order.
#pragma once

#include "kernels.hpp"

namespace {

constexpr int kGroup = 4;             // full row tiles of an expert walked together

// Work item of one workgroup.  The items of an expert are ordered as: groups
// of up to kGroup full row tiles; inside a group, column-tile pairs (2p, 2p+1),
// first every full row tile of the group at column 2p, then at 2p+1, then --
// in the expert's last group only -- one item that runs the expert's short
// last row tile (at most half_rows rows: half the MFMA work, a quarter when it
// has at most half_rows/2 rows and the kernel runs quarter-height tiles) at
// both columns.
// Every item then takes about one full tile's time, items that share a weight
// tile or a row tile of the input are close together, and each XCD (one L2)
// walks a contiguous range of items, so neighbours run at the same time and
// re-read shared operands from L2.
struct Work {
  int e, nt, row0, rows;
  bool pair;    // short row tile at columns nt and nt + 1 (when nt + 1 exists)
  bool single;  // the expert's rows fit one row tile: its weight tiles are read by this item only
};

__device__ __forceinline__ int items_before(const GemmArgs& a, int e, int np) {
  return a.f_prefix[e] * a.n_tiles + a.h_prefix[e] * np;
}

// Item of the workgroup.  XCD x (blocks x, x+8, ...: the hardware hands
// blocks to the eight XCDs in turn) owns the contiguous range of n_x items
// starting at start_x, and its blocks take them in order.  With a pool, the
// last ceil(n_x/16) items of every range are shared instead: blocks past
// their XCD's own part take pool items through one atomic counter, so an XCD
// that runs ahead finishes the others' last items (the XCDs progress at
// different rates, and the kernel ends with the slowest).  `slot` is one int
// of LDS that broadcasts the counter value to the workgroup (the stages are
// not in use yet).  Every item is taken exactly once: the counter hands out
// each pool index once, and every XCD has at least its own share of takers
// (its last blocks) because the grid is at least the item count.
__device__ __forceinline__ bool work_of_block(const GemmArgs& a, int BM, Work& w, int* slot = nullptr) {
  const int ntn = a.n_tiles;
  const int np = (ntn + 1) >> 1;
  const int total = items_before(a, a.n_exp, np);
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q = total >> 3, r = total & 7, local = bid >> 3;
  const int nx = q + (xcd < r ? 1 : 0);
  int L;
  if (a.pool == nullptr) {
    if (local >= nx) return false;  // the same as bid >= total
    L = xcd * q + min(xcd, r) + local;
  } else {
    const int tx = (nx + 15) >> 4;
    if (local < nx - tx) {
      L = xcd * q + min(xcd, r) + local;
    } else {
      // at most twice its own share of takers per XCD (its own last blocks
      // and as many surplus blocks): enough for an XCD that runs ahead to take
      // a second share, while the surplus blocks beyond them leave without
      // touching the contended counter
      if (local >= nx + tx) return false;
      // pool size: the shares of the eight ranges (q or q + 1 items each)
      const int tq = (q + 15) >> 4, tq1 = (q + 16) >> 4;
      const int pool_total = r * tq1 + (8 - r) * tq;
      if (threadIdx.x == 0) *slot = atomicAdd(a.pool, 1);
      __syncthreads();
      const int i = __builtin_amdgcn_readfirstlane(*slot);
      __syncthreads();  // every thread has the value before the stages are written
      if (i >= pool_total) return false;
      // pool index i: the shares of XCDs 0..7 in order
      L = -1;
      int base = 0;
      for (int x = 0; x < 8; ++x) {
        const int n = q + (x < r ? 1 : 0), t = (n + 15) >> 4;
        if (i < base + t) {
          L = x * q + min(x, r) + (n - t) + (i - base);
          break;
        }
        base += t;
      }
      if (L < 0) return false;
    }
  }
  // largest e with items_before(e) <= L (experts without items are skipped)
  int lo = 0, hi = a.n_exp;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (items_before(a, mid, np) <= L)
      lo = mid;
    else
      hi = mid;
  }
  const int e = lo;
  int i = L - items_before(a, e, np);
  const int F = a.f_prefix[e + 1] - a.f_prefix[e];
  const int Hs = a.h_prefix[e + 1] - a.h_prefix[e];
  const int nfg = max(1, (F + kGroup - 1) / kGroup);
  const int g = min(i / (kGroup * ntn), nfg - 1);
  i -= g * kGroup * ntn;
  const int f = min(kGroup, F - g * kGroup);  // >= 1, or 0 when F == 0 (then Hs == 1)
  const int h = g == nfg - 1 ? Hs : 0;
  const int bs = 2 * f + h;                   // items per column pair
  const int p = min(i / bs, np - 1);
  const int j = i - p * bs;
  const int ncols = 2 * p + 1 < ntn ? 2 : 1;
  const int len = a.seg_len[e];
  w.e = e;
  w.single = __builtin_amdgcn_readfirstlane(F + Hs == 1 ? 1 : 0) != 0;
  if (j < f * ncols) {
    const int mt = g * kGroup + j % f;
    w.nt = 2 * p + j / f;
    w.row0 = a.seg_start[e] + mt * BM;
    w.rows = min(BM, len - mt * BM);
    w.pair = false;
  } else {
    w.nt = 2 * p;
    w.row0 = a.seg_start[e] + F * BM;
    w.rows = len - F * BM;
    w.pair = true;
  }
  // the same in every lane: keep the item (and the addresses and buffer
  // resources derived from it) in scalar registers; a resource the compiler
  // takes for divergent costs a waterfall loop around every copy
  w.e = __builtin_amdgcn_readfirstlane(w.e);
  w.nt = __builtin_amdgcn_readfirstlane(w.nt);
  w.row0 = __builtin_amdgcn_readfirstlane(w.row0);
  w.rows = __builtin_amdgcn_readfirstlane(w.rows);
  return true;
}

}  // namespace
