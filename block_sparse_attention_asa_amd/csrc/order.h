// Work schedules for the attention kernels (device code shared by the mask builders and
// the backward).  Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asa_internal.h"

namespace asa {

constexpr int kOrderThreads = 1024;   // workgroup size of a launch that calls order_balanced

// Processing order of the work items (CSR rows, or key blocks of the transposed mask).
// Positions split into 8 contiguous ranges, one per XCD (xcd_range); the kernels give XCD x
// the items at the positions of range x.  Items are grouped by length class (0 for an empty
// item, else 1 + floor(log2 length)).  Every class is cut, in item order, into 8
// consecutive slices of near-equal size, and XCD x takes slice x of every class, so each XCD
// gets an equal share of the long items (the work is balanced even when heads differ in
// density) and each slice is a run of neighbouring items (rows of one head share K/V
// blocks in the XCD's L2).  The slices of class c have size floor(s_c / 8) or one more; the
// s_c mod 8 larger ones go to the XCDs that follow those that took the previous class's
// larger slices (a cursor over the XCDs, carried from class to class, longest class first),
// which makes range x hold exactly as many items as xcd_range gives it.  Inside a range
// the slices come longest class first.  One workgroup of kOrderThreads per range: every
// thread owns a run of consecutive items and counts them per class, a workgroup scan per
// class ranks the items inside their class, and each thread writes the items of its run
// that fall in this range's slices (deterministic).  len(i) returns item i's length.
constexpr int kOrderClasses = 12;   // lengths <= kMaxMaskBlocks = 2^10 -> classes 0..11

__device__ inline int length_class(int c) { return c <= 0 ? 0 : 32 - __clz(c); }

struct OrderScratch {
  int wsum[kOrderThreads / 64][kOrderClasses];
  int total[kOrderClasses];
  int slice_lo[kOrderClasses];    // this range's slice of each class, in class ranks
  int slice_hi[kOrderClasses];
  int out[kOrderClasses];         // position of the slice's first item
};

template <typename Len>
__device__ void order_balanced(Len len, int32_t* __restrict__ order, int total, int x, OrderScratch& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (total + kOrderThreads - 1) / kOrderThreads;
  const int t0 = min((int)threadIdx.x * per, total), t1 = min(t0 + per, total);
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
    sh.total[k] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {   // this range's slice of every class, longest class first
    int lo, hi;
    xcd_range(x, total, lo, hi);
    int cursor = 0, out = lo;
    for (int k = kOrderClasses - 1; k >= 0; --k) {
      const int s = sh.total[k], b = s / kXcds, e = s % kXcds;
      int start = x * b;
      for (int j = 0; j < x; ++j) start += ((j - cursor + kXcds) % kXcds) < e ? 1 : 0;
      const int size = b + (((x - cursor + kXcds) % kXcds) < e ? 1 : 0);
      sh.slice_lo[k] = start;
      sh.slice_hi[k] = start + size;
      sh.out[k] = out;
      out += size;
      cursor = (cursor + e) % kXcds;
    }
  }
  __syncthreads();
  int rank[kOrderClasses];   // class rank of this thread's next item of each class
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) rank[k] = sh.wsum[wv][k] + incl[k] - cnt[k];
  for (int i = t0; i < t1; ++i) {
    const int cl = length_class(len(i));
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) {
      if (cl == k) {
        const int q = rank[k]++;
        if (q >= sh.slice_lo[k] && q < sh.slice_hi[k]) order[sh.out[k] + q - sh.slice_lo[k]] = i;
      }
    }
  }
}

}  // namespace asa
