// Work schedules for the attention kernels, and the wavefront exchanges and scans they and
// the mask kernels use (device code shared by the mask builders and the backward).
// Nothing here is exported from the shared library.
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

// Inclusive sum over the lanes of a wavefront (lane i gets lanes 0..i) by DPP lane moves:
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then row 0's total broadcast into
// rows 1 and 3 and rows 0-1's total into rows 2 and 3.  It stays in the vector ALU; a
// scan by shuffles goes through the LDS crossbar once per step.
// The value held by lane (lane ^ LJ) of the wavefront, without the LDS crossbar: DPP quad
// permutations (LJ = 1, 2), row shifts up and down with a select on the lane's bit (4, 8),
// and the gfx950 row-swap instructions (16: rows 0<->1 and 2<->3, 32: halves).
template <int LJ>
__device__ inline uint32_t lane_xor(uint32_t v) {
  static_assert(LJ == 1 || LJ == 2 || LJ == 4 || LJ == 8 || LJ == 16 || LJ == 32, "lane distance");
  const int x = (int)v;
  if constexpr (LJ == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
  } else if constexpr (LJ == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
  } else if constexpr (LJ == 4 || LJ == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x100 + LJ, 0xf, 0xf, false);   // row_shl: lane + LJ
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x110 + LJ, 0xf, 0xf, false);   // row_shr: lane - LJ
    return (uint32_t)((__lane_id() & LJ) ? dn : up);
  } else if constexpr (LJ == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? p[0] : p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? p[0] : p[1];
  }
}
template <int LJ>
__device__ inline uint64_t lane_xor64(uint64_t v) {
  return ((uint64_t)lane_xor<LJ>((uint32_t)(v >> 32)) << 32) | lane_xor<LJ>((uint32_t)v);
}

__device__ inline int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return v;
}

struct OrderScratch {
  int wsum[kOrderThreads / 64][kOrderClasses];
  int total[kOrderClasses];
  int slice_lo[kOrderClasses];    // this range's slice of each class, in class ranks
  int slice_hi[kOrderClasses];
  int out[kOrderClasses];         // position of the slice's first item
  int4 slice[kOrderClasses];      // (slice_lo, slice_hi, out - slice_lo) of each class
  int rank0[kOrderClasses][kOrderThreads];   // each thread's first class rank, per class
};

template <typename Len>
__device__ void order_balanced(Len len, int32_t* __restrict__ order, int total, int x, OrderScratch& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (total + kOrderThreads - 1) / kOrderThreads;
  const int t0 = min((int)threadIdx.x * per, total), t1 = min(t0 + per, total);
  // per-class counts of this thread's run: packed 10 bits each (classes 0-5 in h[0],
  // 6-11 in h[1]) for runs shorter than 1024 items, one counter each otherwise
  static_assert(kOrderClasses <= 12, "two words of six 10-bit counters");
  int cnt[kOrderClasses];
  if (per < 1024) {
    uint64_t h[2] = {0ull, 0ull};
    // four lengths per round, loaded together (the last round re-reads item t1-1)
    for (int i0 = t0; i0 < t1; i0 += 4) {
      int ln[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ln[j] = len(min(i0 + j, t1 - 1));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cl = length_class(ln[j]);
        const uint64_t one = i0 + j < t1 ? 1ull << (10 * (cl % 6)) : 0ull;
        h[0] += cl < 6 ? one : 0ull;
        h[1] += cl < 6 ? 0ull : one;
      }
    }
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) cnt[k] = (int)((h[k / 6] >> (10 * (k % 6))) & 1023ull);
  } else {
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) cnt[k] = 0;
    for (int i = t0; i < t1; ++i) {
      const int cl = length_class(len(i));
#pragma unroll
      for (int k = 0; k < kOrderClasses; ++k) cnt[k] += cl == k ? 1 : 0;
    }
  }
  // inclusive scan of each class count over the threads of a wavefront, then over waves
  int incl[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) {
    const int v = wave_incl_sum(cnt[k]);
    incl[k] = v;
    if (lane == 63) sh.wsum[wv][k] = v;
  }
  __syncthreads();
  static_assert((kXcds & (kXcds - 1)) == 0, "XCD count is a power of two");
  static_assert(kOrderClasses <= 64, "one lane per class");
  if (wv == 0) {
    // lane k < kOrderClasses: exclusive wave offsets and the total of class k
    int tot = 0;
    if (lane < kOrderClasses) {
      int run = 0;
      for (int w = 0; w < kOrderThreads / 64; ++w) {
        const int v = sh.wsum[w][lane];
        sh.wsum[w][lane] = run;
        run += v;
      }
      tot = run;
    }
    // this range's slice of class k: the cursor (the XCD that takes class k's first larger
    // slice) is the sum of total mod 8 over the longer classes, i.e. over the lanes above
    const int e = tot & (kXcds - 1), b = tot / kXcds;
    const int incl_e = wave_incl_sum(e);
    const int cursor = (__builtin_amdgcn_readlane(incl_e, 63) - incl_e) & (kXcds - 1);
    int start = x * b;
    for (int j = 0; j < x; ++j) start += ((j - cursor) & (kXcds - 1)) < e ? 1 : 0;
    const int size = lane < kOrderClasses ? b + (((x - cursor) & (kXcds - 1)) < e ? 1 : 0) : 0;
    // slices come longest class first inside the range: class k starts after the slices of
    // the classes above it
    const int incl_s = wave_incl_sum(size);
    int lo, hi;
    xcd_range(x, total, lo, hi);
    const int out = lo + __builtin_amdgcn_readlane(incl_s, 63) - incl_s;
    if (lane < kOrderClasses) {
      sh.total[lane] = tot;
      sh.slice_lo[lane] = start;
      sh.slice_hi[lane] = start + size;
      sh.out[lane] = out;
      sh.slice[lane] = make_int4(start, start + size, out - start, 0);
    }
  }
  __syncthreads();
  // per class: the rank of this thread's next item, and the offset from a rank in this
  // range's slice to its position (rank + off), selected without branches
  int rank[kOrderClasses], slo[kOrderClasses], shi[kOrderClasses], off[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) {
    rank[k] = sh.wsum[wv][k] + incl[k] - cnt[k];
    slo[k] = sh.slice_lo[k];
    shi[k] = sh.slice_hi[k];
    off[k] = sh.out[k] - slo[k];
  }
  // a run that holds no rank of this range's slices writes nothing: skip it
  bool hit = false;
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) hit |= cnt[k] > 0 && rank[k] < shi[k] && rank[k] + cnt[k] > slo[k];
  if (per < 1024) {
    // an item's rank is its thread's first rank of the class (from LDS, this thread's own
    // column) plus the items of the class before it in the run (packed counters, as above)
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) sh.rank0[k][threadIdx.x] = rank[k];
    uint64_t pk[2] = {0ull, 0ull};
    for (int i = t0; hit && i < t1; ++i) {
      const int cl = length_class(len(i));
      const int sub = 10 * (cl % 6);
      const bool hi6 = cl >= 6;
      const uint64_t word = hi6 ? pk[1] : pk[0];
      const int q = sh.rank0[cl][threadIdx.x] + (int)((word >> sub) & 1023ull);
      pk[0] += hi6 ? 0ull : 1ull << sub;
      pk[1] += hi6 ? 1ull << sub : 0ull;
      const int4 si = sh.slice[cl];
      if (q >= si.x && q < si.y) order[si.z + q] = i;
    }
    return;
  }
  for (int i = t0; hit && i < t1; ++i) {
    const int cl = length_class(len(i));
    int q = 0, lo_k = 0, hi_k = 0, off_k = 0;
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) {
      const bool m = cl == k;
      q = m ? rank[k] : q;
      lo_k = m ? slo[k] : lo_k;
      hi_k = m ? shi[k] : hi_k;
      off_k = m ? off[k] : off_k;
      rank[k] += m ? 1 : 0;
    }
    if (q >= lo_k && q < hi_k) order[off_k + q] = i;
  }
}

}  // namespace asa
