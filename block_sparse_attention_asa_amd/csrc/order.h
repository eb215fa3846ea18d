// Work schedules for the attention kernels (device code shared by the mask builders and
// the backward).  Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asa_internal.h"

namespace asa {

constexpr int kOrderThreads = 1024;   // workgroup size of a launch that calls order_range

// Processing order of the work items (CSR rows, or key blocks of the transposed mask):
// inside each XCD's contiguous range, items by descending length class, stable in index,
// so long items (text rows, full heads, popular key blocks) start first and do not form
// the tail.  Class of an item of length c: 0 for c = 0, else 1 + floor(log2 c).  One
// workgroup of kOrderThreads per range: every thread owns a run of consecutive items and
// counts them per class, a workgroup scan per class gives each thread its output slots,
// and the items are written in order (deterministic).  len(i) returns item i's length.
constexpr int kOrderClasses = 12;   // lengths <= kMaxMaskBlocks = 2^10 -> classes 0..11

__device__ inline int length_class(int c) { return c <= 0 ? 0 : 32 - __clz(c); }

struct OrderScratch {
  int wsum[kOrderThreads / 64][kOrderClasses];
  int base[kOrderClasses];
};

template <typename Len>
__device__ void order_range(Len len, int32_t* __restrict__ order, int total, int x, OrderScratch& sh) {
  int lo, hi;
  xcd_range(x, total, lo, hi);
  const int n = hi - lo;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (n + kOrderThreads - 1) / kOrderThreads;
  const int t0 = lo + threadIdx.x * per, t1 = min(t0 + per, hi);
  int cnt[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) cnt[k] = 0;
  for (int i = t0; i < t1; ++i) {
    const int cl = length_class(len(i));
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) cnt[k] += cl == k ? 1 : 0;
  }
  // inclusive scan of each class count over the threads of a wavefront, then over waves
  int incl[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) {
    int v = cnt[k];
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    incl[k] = v;
    if (lane == 63) sh.wsum[wv][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < kOrderClasses) {   // exclusive wave offsets and class totals
    const int k = threadIdx.x;
    int run = 0;
    for (int w = 0; w < kOrderThreads / 64; ++w) {
      const int v = sh.wsum[w][k];
      sh.wsum[w][k] = run;
      run += v;
    }
    sh.base[k] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {   // class starts, longest class first
    int start = 0;
    for (int k = kOrderClasses - 1; k >= 0; --k) {
      const int tot = sh.base[k];
      sh.base[k] = start;
      start += tot;
    }
  }
  __syncthreads();
  int slot[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) slot[k] = lo + sh.base[k] + sh.wsum[wv][k] + incl[k] - cnt[k];
  for (int i = t0; i < t1; ++i) {
    const int cl = length_class(len(i));
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) {
      if (cl == k) order[slot[k]++] = i;
    }
  }
}

}  // namespace asa
