// Block-mask construction for content-aware block-sparse attention (gfx950).
//
// Adaptive source: BLADE ("BLADE: Block-Sparse Attention Meets Step Distillation for
// Efficient Video Generation", abstract) generates a content-aware block mask per
// input; its rule is not on the pages, so the rule here is the one stated in asa.h:
// mean-pooled Q and K per block, float64 block scores / sqrt(d), row softmax, rank by
// probability (ties to the smaller block), keep top-k or the shortest prefix reaching
// the mass tau (capped), plus the diagonal and text blocks.
// Static sources: Sparse-vDiT ("Sparse-vDiT: Sparse Attention Acceleration for Video
// Diffusion Transformers"), "四种注意力模式" table (full, skip, diagonal,
// multi-diagonal, vertical stripe).
//
// Pipeline (all on the caller's stream):
//   pool_kernel      Q, K -> Qp [B,H,Nb,d], KpT [B,H,d,Nb] (float64 means); HBM-bound.
//   score_kernel     S = Qp KpT / sqrt(d) on the fp64 matrix cores, 32 x 32 tiles.
//   select_kernel    one workgroup per row: softmax, bitonic sort of (P, c) held in
//                    registers (cross-lane, LDS or in-register exchanges), prefix
//                    selection, union with forced / static blocks -> bitmask.
//   static_kernel    one wavefront per row: static pattern bitmask only.
//   csr_scan_kernel  exclusive scan of per-row counts -> row_ptr; optionally the
//                    processing order (long rows first inside each XCD range).
//   csr_fill_kernel  one wavefront per row: bitmask -> ascending col_idx.
#include <hip/hip_runtime.h>

#include "asa_internal.h"

namespace asa {
namespace {

constexpr int kThreads = 256;

__device__ inline double bf16_to_f64(uint16_t x) {
  return (double)__uint_as_float(((uint32_t)x) << 16);
}

// ------------------------------------------------------------------ static patterns
__device__ inline long long floor_div(long long a, long long b) {  // b > 0
  long long q = a / b;
  if ((a % b != 0) && (a < 0)) --q;
  return q;
}

// Is key block c kept in query-block row r by static pattern (id, param)?
__device__ inline bool static_keep(int id, int param, int r, int c, int N, int blk, int Nb) {
  switch (id) {
    case 1:  // full
      return true;
    case 3:  // diagonal
      return c == r;
    case 5:  // vertical stripe: leading `param` key blocks
      return c < param;
    case 4: {  // multi-diagonal, stride `param` tokens
      const long long qlo = (long long)r * blk;
      const long long qhi = min(qlo + blk, (long long)N) - 1;
      const long long klo = (long long)c * blk;
      const long long khi = min(klo + blk, (long long)N) - 1;
      const long long lo = klo - qhi, hi = khi - qlo;   // range of j - i over the tile
      const long long S = param;
      return floor_div(hi, S) * S >= lo;                // a multiple of S lies in [lo, hi]
    }
    case 6: {  // frame tiles of `param` tokens: the query's own frames and frame 0
      const long long F = param;
      const long long qlo = (long long)r * blk;
      const long long qhi = min(qlo + blk, (long long)N) - 1;
      const long long klo = (long long)c * blk;
      const long long khi = min(klo + blk, (long long)N) - 1;
      if (klo < F) return true;                         // the block holds frame-0 keys
      return klo / F <= qhi / F && qlo / F <= khi / F;  // frame ranges overlap
    }
    default:  // skip, adaptive
      return false;
  }
}

// ------------------------------------------------------------------ pooling
// grid = (B*H*Nb, 2): y = 0 pools Q into Qp (row-major), y = 1 pools K into KpT.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const void* __restrict__ q,
                                                        const void* __restrict__ k,
                                                        double* __restrict__ qp,
                                                        double* __restrict__ kpt, int N,
                                                        int blk, int Nb) {
  constexpr int VEC = 8;
  constexpr int TPR = D / VEC;          // threads per token row
  constexpr int RPP = kThreads / TPR;   // token rows per pass
  __shared__ double red[RPP][D];        // per-thread partial sums, one row per row group

  const int row = blockIdx.x;
  const int bh = row / Nb, r = row - bh * Nb;
  const int lo = r * blk, n = min(blk, N - lo);
  const int t = threadIdx.x, col = (t % TPR) * VEC, sub = t / TPR;
  const size_t head_off = (size_t)bh * N * D;

  double acc[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = 0.0;

  if (BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(blockIdx.y == 0 ? q : k) + head_off;
    auto add_row = [&](const uint4& v) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16_to_f64((uint16_t)(w[j] & 0xffffu));
        acc[2 * j + 1] += bf16_to_f64((uint16_t)(w[j] >> 16));
      }
    };
    // rows in the same order as one at a time, but all of a thread's loads for a full
    // 128-token block in flight at once
    constexpr int kBatch = 128 / RPP;
    int i = sub;
    for (; i + (kBatch - 1) * RPP < n; i += kBatch * RPP) {
      uint4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        v[b] = *reinterpret_cast<const uint4*>(x + (size_t)(lo + i + b * RPP) * D + col);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) add_row(v[b]);
    }
    for (; i < n; i += RPP) add_row(*reinterpret_cast<const uint4*>(x + (size_t)(lo + i) * D + col));
  } else {
    const float* x = static_cast<const float*>(blockIdx.y == 0 ? q : k) + head_off;
    for (int i = sub; i < n; i += RPP) {
      const float4 a = *reinterpret_cast<const float4*>(x + (size_t)(lo + i) * D + col);
      const float4 b = *reinterpret_cast<const float4*>(x + (size_t)(lo + i) * D + col + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) red[sub][col + j] = acc[j];
  __syncthreads();
  if (t < D) {   // one thread per column sums the row groups in a fixed order
    double v = 0.0;
#pragma unroll
    for (int s = 0; s < RPP; ++s) v += red[s][t];
    const double nn = (double)n;
    if (blockIdx.y == 0) qp[(size_t)row * D + t] = v / nn;
    else kpt[((size_t)bh * D + t) * Nb + r] = v / nn;
  }
}

// ------------------------------------------------------------------ block scores
// S = Qp KpT / sqrt(d) for one head, a dense float64 contraction, on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64).  One workgroup computes a 32 x 32 tile of S (query blocks r0..,
// key blocks c0..); each of its four wavefronts owns a 16 x 16 quarter.  Operand layout of
// the instruction, per lane l: A holds row l%16, k = l/16; B holds k = l/16, column l%16;
// result component e holds row 4e + l/16, column l%16.  Two accumulators take alternate
// k-steps.  grid = B*H * ceil(Nb/32)^2.
constexpr int kST = 32;          // score tile edge
typedef double f64x4_t __attribute__((ext_vector_type(4)));
template <int D>
__global__ __launch_bounds__(kThreads) void score_kernel(const double* __restrict__ qp,
                                                         const double* __restrict__ kpt,
                                                         double* __restrict__ score, int Nb) {
  const int tiles = (Nb + kST - 1) / kST;
  int id = blockIdx.x;
  const int tcol = id % tiles;
  id /= tiles;
  const int trow = id % tiles, bh = id / tiles;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r0 = trow * kST + 16 * (w >> 1), c0 = tcol * kST + 16 * (w & 1);
  const int ra = r0 + (l & 15), kl = l >> 4, cb = c0 + (l & 15);
  const double* q = qp + (size_t)bh * Nb * D;
  const double* kt = kpt + (size_t)bh * D * Nb;
  const bool a_ok = ra < Nb, b_ok = cb < Nb;
  f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int k0 = 0; k0 < D; k0 += 8) {
    const double a0 = a_ok ? q[(size_t)ra * D + k0 + kl] : 0.0;
    const double b0 = b_ok ? kt[(size_t)(k0 + kl) * Nb + cb] : 0.0;
    const double a1 = a_ok ? q[(size_t)ra * D + k0 + 4 + kl] : 0.0;
    const double b1 = b_ok ? kt[(size_t)(k0 + 4 + kl) * Nb + cb] : 0.0;
    acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc1, 0, 0, 0);
  }
  const double sqrt_d = sqrt((double)D);
  const int c = c0 + (l & 15);
  if (c < Nb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 4 * e + (l >> 4);
      if (r < Nb) score[((size_t)bh * Nb + r) * Nb + c] = (acc0[e] + acc1[e]) / sqrt_d;
    }
  }
}

// Rank keys.  Rank order is value descending, then block index ascending.  A key packs
// both into one uint64: the value's bits made order-preserving as an unsigned integer,
// its lowest 10 bits replaced by 1023 - c.  Dropping those bits merges values closer than
// 2^-42 relative (far inside the near-tie gap, where rows are ambiguous anyway); every
// other pair of blocks keeps its order, and keys of distinct blocks never tie.  Padding
// slots get key 0, after every real block.
__device__ inline uint64_t rank_key(double v, int c) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  b = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (b & ~(uint64_t)0x3FF) | (uint64_t)(1023 - c);
}
__device__ inline int key_block(uint64_t k) { return 1023 - (int)(k & 0x3FF); }

// Bitonic sort, keys descending, over NP2 slots: slot i = e*kThreads + tid lives in
// register e of thread tid.  A compare-exchange at distance j runs inside a thread's
// registers (j >= kThreads), through LDS (64 <= j < kThreads, two barriers) or across the
// lanes of one wavefront (j < 64, no barrier).  Every stage is unrolled, so each branch
// below is resolved at compile time.
template <int NP2, int KK, int J>
__device__ inline void bitonic_stage(uint64_t* kv, uint64_t* lds) {
  constexpr int PER = (NP2 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  if constexpr (J >= kThreads) {
    constexpr int je = J / kThreads;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int e2 = e ^ je;
      if (e2 > e) {
        const int i = e * kThreads + tid;
        const bool desc = (i & KK) == 0;   // this pair's run sorts descending
        const uint64_t a = kv[e], b = kv[e2];
        if ((a > b) != desc) { kv[e] = b; kv[e2] = a; }
      }
    }
  } else if constexpr (J >= 64) {
#pragma unroll
    for (int e = 0; e < PER; ++e) lds[e * kThreads + tid] = kv[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = e * kThreads + tid;
      const uint64_t b = lds[i ^ J];
      const bool first = ((i & KK) == 0) == ((i & J) == 0);   // keep the higher-ranked one
      kv[e] = first ? (kv[e] > b ? kv[e] : b) : (kv[e] > b ? b : kv[e]);
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = e * kThreads + tid;
      const uint64_t b = (uint64_t)__shfl_xor((long long)kv[e], J, 64);
      const bool first = ((i & KK) == 0) == ((i & J) == 0);
      kv[e] = first ? (kv[e] > b ? kv[e] : b) : (kv[e] > b ? b : kv[e]);
    }
  }
  if constexpr (J > 1) bitonic_stage<NP2, KK, J / 2>(kv, lds);
}
template <int NP2, int KK>
__device__ inline void bitonic_pass(uint64_t* kv, uint64_t* lds) {
  bitonic_stage<NP2, KK, KK / 2>(kv, lds);
  if constexpr (KK < NP2) bitonic_pass<NP2, KK * 2>(kv, lds);
}
template <int NP2>
__device__ inline void bitonic_sort_desc(uint64_t* kv, uint64_t* lds) {
  if constexpr (NP2 >= 2) bitonic_pass<NP2, 2>(kv, lds);
}

// ------------------------------------------------------------------ block reductions
// Workgroup reductions: butterfly within each wavefront, then the 4 wave results in a fixed
// order (deterministic).  scratch holds at least 4 doubles.
__device__ inline double block_reduce_max(double v, double* scratch) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = fmax(fmax(scratch[0], scratch[1]), fmax(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}

__device__ inline double block_reduce_sum(double v, double* scratch) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ selection
// grid = B*H*Nb rows; one workgroup per row.
__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ score,
                                                          uint32_t* __restrict__ bits,
                                                          int32_t* __restrict__ count,
                                                          MaskGeom g, AdaptiveParams p,
                                                          HeadTable heads) {
  __shared__ double wgt[kMaxMaskBlocks];     // scores (top-k) or softmax numerators (mass)
  __shared__ uint64_t xch[kMaxMaskBlocks];   // sort exchange space, then the ranked blocks
  __shared__ double scratch[kThreads];
  __shared__ uint32_t word[kMaxMaskBlocks / 32];
  __shared__ int kept_prefix;

  const int row = blockIdx.x;
  const int bh = row / g.Nb, r = row - bh * g.Nb, h = bh % g.H;
  const int tid = threadIdx.x;
  const int pid = heads.id[h], prm = heads.param[h];
  const int Nb = g.Nb;

  if (tid < g.words) word[tid] = 0u;
  __syncthreads();

  if (pid == 2) {   // skip head: empty row
    if (tid < g.words) bits[(size_t)row * g.words + tid] = 0u;
    if (tid == 0) count[row] = 0;
    return;
  }
  if (r < p.n_text_blocks) {   // query block holding text tokens: full row
    for (int c = tid; c < Nb; c += kThreads) atomicOr(&word[c >> 5], 1u << (c & 31));
  } else if (p.mode == 0 && p.k >= Nb) {   // top-k keeping every block: nothing to rank
    for (int c = tid; c < Nb; c += kThreads) atomicOr(&word[c >> 5], 1u << (c & 31));
  } else {
    const double* srow = score + (size_t)row * Nb;
    // Rank keys.  Top-k ranks by the score itself: exp is increasing, so the order by P
    // equals the order by S wherever the S values differ by more than float64 rounding of
    // P can hide (a top-k boundary closer than that is a near-tie, see ambiguous rows).
    // The mass prefix needs P itself: softmax over all key blocks of this row.
    double z = 1.0;
    if (p.mode == 0) {
      for (int c = tid; c < Nb; c += kThreads) wgt[c] = srow[c];
      __syncthreads();
    } else {
      double mx = -INFINITY;
      for (int c = tid; c < Nb; c += kThreads) mx = fmax(mx, srow[c]);
      mx = block_reduce_max(mx, scratch);
      double part = 0.0;
      for (int c = tid; c < Nb; c += kThreads) {
        const double e = exp(srow[c] - mx);
        wgt[c] = e;
        part += e;
      }
      z = block_reduce_sum(part, scratch);   // also a barrier for wgt[]
    }
    int np2 = 1;
    while (np2 < Nb) np2 <<= 1;
    constexpr int kPer = kMaxMaskBlocks / kThreads;
    uint64_t kv[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = e * kThreads + tid;
      kv[e] = i < Nb ? rank_key(p.mode == 0 ? wgt[i] : wgt[i] / z, i) : 0ull;
    }
    switch (np2) {
      case 1: break;
      case 2: bitonic_sort_desc<2>(kv, xch); break;
      case 4: bitonic_sort_desc<4>(kv, xch); break;
      case 8: bitonic_sort_desc<8>(kv, xch); break;
      case 16: bitonic_sort_desc<16>(kv, xch); break;
      case 32: bitonic_sort_desc<32>(kv, xch); break;
      case 64: bitonic_sort_desc<64>(kv, xch); break;
      case 128: bitonic_sort_desc<128>(kv, xch); break;
      case 256: bitonic_sort_desc<256>(kv, xch); break;
      case 512: bitonic_sort_desc<512>(kv, xch); break;
      default: bitonic_sort_desc<1024>(kv, xch); break;
    }
    // length of the adaptive prefix
    if (p.mode == 0) {
      if (tid == 0) kept_prefix = min(max(p.k, 0), Nb);
    } else {
      // running mass in rank order, summed sequentially from the exact weights (the order
      // fixes the float64 bits): the ranked block indices go through LDS
      int* order_lds = reinterpret_cast<int*>(xch);   // free again after the sort
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (e * kThreads < np2) order_lds[e * kThreads + tid] = key_block(kv[e]);
      __syncthreads();
      if (tid == 0) {
        int m = Nb;
        double mass = 0.0;
        for (int t = 0; t < Nb; ++t) {
          mass += wgt[order_lds[t]] / z;
          if (mass >= p.tau) { m = t + 1; break; }
        }
        if (p.k_cap > 0) m = min(m, p.k_cap);
        kept_prefix = m;
      }
    }
    __syncthreads();
    const int m = kept_prefix;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = e * kThreads + tid;
      if (i < m) {
        const int c = key_block(kv[e]);
        atomicOr(&word[c >> 5], 1u << (c & 31));
      }
    }
    for (int c = tid; c < Nb; c += kThreads) {
      const bool forced = (p.keep_diag && c == r) || (c < p.n_text_blocks) ||
                          static_keep(pid, prm, r, c, g.N, g.blk, Nb);
      if (forced) atomicOr(&word[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();
  if (tid < g.words) bits[(size_t)row * g.words + tid] = word[tid];
  if (tid < 64) {
    int pc = tid < g.words ? __popc(word[tid]) : 0;
    for (int off = 32; off > 0; off >>= 1) pc += __shfl_xor(pc, off, 64);
    if (tid == 0) count[row] = pc;
  }
}

// ------------------------------------------------------------------ static-only rows
// One wavefront per row, 4 rows per workgroup.
__global__ __launch_bounds__(kThreads) void static_kernel(uint32_t* __restrict__ bits,
                                                          int32_t* __restrict__ count,
                                                          MaskGeom g, HeadTable heads, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bh = row / g.Nb, r = row - bh * g.Nb, h = bh % g.H;
  const int pid = heads.id[h], prm = heads.param[h];
  uint32_t w = 0u;
  if (lane < g.words) {
    for (int b = 0; b < 32; ++b) {
      const int c = lane * 32 + b;
      if (c < g.Nb && static_keep(pid, prm, r, c, g.N, g.blk, g.Nb)) w |= 1u << b;
    }
    bits[(size_t)row * g.words + lane] = w;
  }
  int pc = __popc(w);
  for (int off = 32; off > 0; off >>= 1) pc += __shfl_xor(pc, off, 64);
  if (lane == 0) count[row] = pc;
}

// ------------------------------------------------------------------ CSR
constexpr int kScanThreads = 1024;

// Processing order for the attention kernel: inside each XCD's contiguous row range, rows
// by descending length class, stable in row index, so long rows (text rows, full heads)
// start first and do not form the tail.  Class of a row with c kept blocks: 0 for c = 0,
// else 1 + floor(log2 c).  One workgroup of the scan launch per range, beside the one that
// scans: every thread owns a run of consecutive rows and counts them per class, a
// workgroup scan per class gives each thread its output slots, and the rows are written
// in order (deterministic).
constexpr int kOrderClasses = 12;   // c <= kMaxMaskBlocks = 2^10 -> classes 0..11

__device__ inline int length_class(int c) { return c <= 0 ? 0 : 32 - __clz(c); }

struct OrderScratch {
  int wsum[kScanThreads / 64][kOrderClasses];
  int base[kOrderClasses];
};

__device__ void order_range(const int32_t* __restrict__ count, int32_t* __restrict__ order, int rows,
                            int x, OrderScratch& sh) {
  int lo, hi;
  xcd_range(x, rows, lo, hi);
  const int n = hi - lo;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int t0 = lo + threadIdx.x * per, t1 = min(t0 + per, hi);
  int cnt[kOrderClasses];
#pragma unroll
  for (int k = 0; k < kOrderClasses; ++k) cnt[k] = 0;
  for (int i = t0; i < t1; ++i) {
    const int cl = length_class(count[i]);
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
    for (int w = 0; w < kScanThreads / 64; ++w) {
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
    const int cl = length_class(count[i]);
#pragma unroll
    for (int k = 0; k < kOrderClasses; ++k) {
      if (cl == k) order[slot[k]++] = i;
    }
  }
}

// Workgroup 0: row_ptr[0] = 0, row_ptr[i+1] = sum of count[0..i].  Each thread owns a
// run of consecutive rows; one wave-level scan of the per-thread totals.
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(const int32_t* __restrict__ count,
                                                                int32_t* __restrict__ row_ptr,
                                                                int32_t* __restrict__ order,
                                                                int rows) {
  __shared__ int wsum[kScanThreads / 64];
  __shared__ OrderScratch osh;
  if (blockIdx.x > 0) {   // workgroups 1..8: the processing order of one XCD range each
    order_range(count, order, rows, blockIdx.x - 1, osh);
    return;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int t0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (t0 + i < rows) local += count[t0 + i];
  int incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const int v0 = lane < kScanThreads / 64 ? wsum[lane] : 0;
    int x = v0;
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(x, off, 64);
      if (lane >= off) x += v;
    }
    if (lane < kScanThreads / 64) wsum[lane] = x - v0;   // exclusive
  }
  __syncthreads();
  int run = wsum[wv] + incl - local;
  if (threadIdx.x == 0) row_ptr[0] = 0;
  for (int i = 0; i < per; ++i) {
    if (t0 + i < rows) {
      run += count[t0 + i];
      row_ptr[t0 + i + 1] = run;
    }
  }
}

// One wavefront per row: kept bits -> ascending block indices.
__global__ __launch_bounds__(kThreads) void csr_fill_kernel(const uint32_t* __restrict__ bits,
                                                            const int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ col_idx,
                                                            int words, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint32_t w = lane < words ? bits[(size_t)row * words + lane] : 0u;
  const int pc = __popc(w);
  int incl = pc;   // inclusive prefix over lanes
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int out = row_ptr[row] + incl - pc;
  while (w) {
    const int b = __ffs(w) - 1;
    col_idx[out++] = lane * 32 + b;
    w &= w - 1u;
  }
}

}  // namespace

// ------------------------------------------------------------------ host launchers
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t mask_workspace_layout(const MaskGeom& g, bool adaptive, MaskWorkspace* ws, void* base) {
  const size_t rows = (size_t)g.B * g.H * g.Nb;
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  MaskWorkspace w{};
  if (adaptive) {
    w.qp = static_cast<double*>(take(rows * g.d * sizeof(double)));
    w.kpt = static_cast<double*>(take(rows * g.d * sizeof(double)));
    w.score = static_cast<double*>(take(rows * g.Nb * sizeof(double)));
  }
  w.bits = static_cast<uint32_t*>(take(rows * g.words * sizeof(uint32_t)));
  w.count = static_cast<int32_t*>(take(rows * sizeof(int32_t)));
  if (ws) *ws = w;
  return off;
}

hipError_t launch_pool(const void* q, const void* k, bool bf16, const MaskGeom& g,
                       const MaskWorkspace& ws, hipStream_t s) {
  const dim3 grid((unsigned)(g.B * g.H * g.Nb), 2);
  if (bf16) {
    if (g.d == 128)
      hipLaunchKernelGGL((pool_kernel<true, 128>), grid, dim3(kThreads), 0, s, q, k, ws.qp, ws.kpt, g.N, g.blk, g.Nb);
    else
      hipLaunchKernelGGL((pool_kernel<true, 64>), grid, dim3(kThreads), 0, s, q, k, ws.qp, ws.kpt, g.N, g.blk, g.Nb);
  } else {
    if (g.d == 128)
      hipLaunchKernelGGL((pool_kernel<false, 128>), grid, dim3(kThreads), 0, s, q, k, ws.qp, ws.kpt, g.N, g.blk, g.Nb);
    else
      hipLaunchKernelGGL((pool_kernel<false, 64>), grid, dim3(kThreads), 0, s, q, k, ws.qp, ws.kpt, g.N, g.blk, g.Nb);
  }
  return hipGetLastError();
}

hipError_t launch_scores(const MaskGeom& g, const MaskWorkspace& ws, hipStream_t s) {
  const int tiles = (g.Nb + kST - 1) / kST;
  const dim3 grid((unsigned)(g.B * g.H * tiles * tiles));
  if (g.d == 128)
    hipLaunchKernelGGL(score_kernel<128>, grid, dim3(kThreads), 0, s, ws.qp, ws.kpt, ws.score, g.Nb);
  else
    hipLaunchKernelGGL(score_kernel<64>, grid, dim3(kThreads), 0, s, ws.qp, ws.kpt, ws.score, g.Nb);
  return hipGetLastError();
}

hipError_t launch_select(const MaskGeom& g, const AdaptiveParams& p, const HeadTable& heads,
                         const MaskWorkspace& ws, hipStream_t s) {
  const dim3 grid((unsigned)(g.B * g.H * g.Nb));
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), 0, s, ws.score, ws.bits, ws.count, g, p, heads);
  return hipGetLastError();
}

hipError_t launch_static_rows(const MaskGeom& g, const HeadTable& heads, const MaskWorkspace& ws,
                              hipStream_t s) {
  const int rows = g.B * g.H * g.Nb;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL(static_kernel, grid, dim3(kThreads), 0, s, ws.bits, ws.count, g, heads, rows);
  return hipGetLastError();
}

hipError_t launch_csr(const MaskGeom& g, const MaskWorkspace& ws, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* order, hipStream_t s) {
  const int rows = g.B * g.H * g.Nb;
  // workgroup 0 scans the counts; with an order, workgroups 1..8 order one XCD range each
  hipLaunchKernelGGL(csr_scan_kernel, dim3(order ? 1 + kXcds : 1), dim3(kScanThreads), 0, s, ws.count,
                     row_ptr, order, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_fill_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s, ws.bits,
                     row_ptr, col_idx, g.words, rows);
  return hipGetLastError();
}

}  // namespace asa
