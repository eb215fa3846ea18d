// Block-sparse attention backward for gfx950 (MI355X), bf16 or fp32 inputs, fp32 gradients.
//
// The gradients of the masked attention of Sparse-vDiT ("Sparse-vDiT: Sparse Attention
// Acceleration for Video Diffusion Transformers", section 三 "核心公式"); BLADE
// ("BLADE: Block-Sparse Attention Meets Step Distillation for Efficient Video
// Generation", abstract) trains the sparse attention jointly with distillation.  With
// P_ij = exp(scale Q_i.K_j - lse_i) over the kept tokens j of query i's row:
//     dV_j = sum_i P_ij dO_i        dP_ij = dO_i . V_j        D_i = dO_i . O_i
//     dS_ij = P_ij (dP_ij - D_i)    dQ_i = scale sum_j dS_ij K_j
//     dK_j = scale sum_i dS_ij Q_i
// The weights are recomputed from Q, K and the forward's lse, so nothing of size N x N
// is stored.
//
// Kernels (all on the caller's stream):
//   bwd_prep_kernel  per query: (lse * log2 e, D = dO . O) -> workspace pairs.
//   csc_kernel       one workgroup per head: CSR -> CSC (key block -> query blocks in
//                    ascending order) through a transposed bitmask in LDS.
//   col_order_kernel the key-block schedule: an equal share of every list-length class per
//                    XCD, longest lists first.
//   dq_kernel        one workgroup per query-block row, like the forward (and in the CSR's
//                    processing order when there is one): K and V of every
//                    kept key block stream through an LDS ring; per 64-key step
//                    S^T = K Q^T, P^T = exp2(S^T s - lse), dP^T = V dO^T,
//                    dS^T = P^T (dP^T - D), dQ^T += K^T dS^T  (K^T by transpose reads).
//   dkv_kernel       one workgroup per key block (32 keys per wavefront: their K in
//                    registers, their V in lane-private LDS); Q, dO and the (lse, D) pairs
//                    of every query block that
//                    keeps it stream through an LDS ring; per 32-query step
//                    S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
//   dq_f32_kernel, dkv_f32_kernel   the same two passes for fp32 inputs (P and dS in
//                    fp32, operands read from global memory; see their section).
// Each gradient element is accumulated by one lane in a fixed order (no atomics), so the
// results are deterministic.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "order.h"

namespace asa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ preprocessing
// TPQ = D/8 consecutive threads per query, 8 elements each; D reduced with shuffles.
// Eight consecutive elements of a bf16 (uint16_t) or fp32 row as fp32.
__device__ inline void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(aw[j] << 16);
    x[2 * j + 1] = __uint_as_float(aw[j] & 0xffff0000u);
  }
}
__device__ inline void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename TG, typename TO, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const TG* __restrict__ dout,
                                                       const TO* __restrict__ o,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ ld, size_t nq) {
  constexpr int TPQ = D / 8;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t q = gid / TPQ;
  const int part = (int)(gid % TPQ);
  float acc = 0.f;
  if (q < nq) {
    float gv[8];
    load8(dout + q * D + part * 8, gv);
    float ov[8];
    load8(o + q * D + part * 8, ov);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_fmaf(gv[j], ov[j], acc);
  }
  for (int off = TPQ / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (q < nq && part == 0) {
    ld[2 * q] = lse[q] * kLog2e;
    ld[2 * q + 1] = acc;
  }
}

// ------------------------------------------------------------------ CSR -> CSC
// One workgroup per (b, h).  Bit (c, r) of an LDS bitmask marks "query block r keeps key
// block c"; column c's list is then read off in ascending r.  The head's CSC segment
// starts where its CSR segment does (same number of kept tiles).
constexpr int kCscThreads = 1024;
__global__ __launch_bounds__(kCscThreads) void csc_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx,
                                                          int32_t* __restrict__ col_ptr,
                                                          int32_t* __restrict__ row_idx, int Nb,
                                                          int heads) {
  __shared__ uint32_t bitT[kMaxMaskBlocks * (kMaxMaskBlocks / 32)];
  __shared__ int wsum[kCscThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int words = (Nb + 31) / 32;
  for (int i = tid; i < Nb * words; i += kCscThreads) bitT[i] = 0u;
  __syncthreads();
  const int rbase = bh * Nb;
  for (int r = tid; r < Nb; r += kCscThreads) {
    const int e1 = row_ptr[rbase + r + 1];
    for (int e = row_ptr[rbase + r]; e < e1; ++e) {
      const int c = col_idx[e];
      atomicOr(&bitT[c * words + (r >> 5)], 1u << (r & 31));
    }
  }
  __syncthreads();
  const int c = tid;   // Nb <= kCscThreads: one key block per thread
  int cnt = 0;
  if (c < Nb)
    for (int w = 0; w < words; ++w) cnt += __popc(bitT[c * words + w]);
  const int incl = wave_incl_sum(cnt);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    const int v0 = lane < kCscThreads / 64 ? wsum[lane] : 0;
    const int x = wave_incl_sum(v0);
    if (lane < kCscThreads / 64) wsum[lane] = x - v0;
  }
  __syncthreads();
  if (c < Nb) {
    int pos = row_ptr[rbase] + wsum[wv] + incl - cnt;
    col_ptr[rbase + c] = pos;
    for (int w = 0; w < words; ++w) {
      uint32_t b = bitT[c * words + w];
      while (b) {
        row_idx[pos++] = w * 32 + __ffs(b) - 1;
        b &= b - 1u;
      }
    }
  }
  if (bh == heads - 1 && tid == 0) col_ptr[heads * Nb] = row_ptr[heads * Nb];
}

// Key-block schedule for dkv_kernel (order_balanced over the lengths of the key blocks'
// query-block lists; skipped heads count as empty): every XCD gets an equal share of each
// length class, and the blocks kept by many query blocks start first.  One workgroup per
// XCD range.
__global__ __launch_bounds__(kOrderThreads) void col_order_kernel(const int32_t* __restrict__ col_ptr,
                                                                  int32_t* __restrict__ col_order,
                                                                  int Nb, int H, int total,
                                                                  SkipBits skip) {
  __shared__ OrderScratch sh;
  order_balanced(
      [&](int i) {
        const int h = (i / Nb) % H;
        return ((skip.bits[h >> 5] >> (h & 31)) & 1u) ? 0 : col_ptr[i + 1] - col_ptr[i];
      },
      col_order, total, blockIdx.x, sh);
}

// V^T-style fragment by transpose reads: rows kbase.. of a row-major swizzled [rows][D]
// bf16 tile, columns 32*io + ..; element j of lane half hf comes from row
// 16*u + 8*(j/4) + 4*hf + j%4 (the k order of the MFMA output layout).  Lane s of 16-lane
// group g supplies row 16u + 8tt + 4(g/2) + s/4, columns dcol.. (4 elements); lane i of the
// group receives column dcol + i of those four rows.
template <int D>
__device__ inline Frag<uint16_t> tr_frag(const uint16_t* tile, int io, int u, int lane) {
  constexpr int GPR = D * 2 / 16;
  const int g = lane >> 4, sl = lane & 15;
  const int dcol = 32 * io + 16 * (g & 1) + 4 * (sl & 3);
  short4_t part[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int kr = 16 * u + 8 * tt + 4 * (g >> 1) + (sl >> 2);
    const int gran = (dcol >> 3) ^ swz<GPR>(kr);
    const uint16_t* p = tile + kr * D + gran * 8 + (dcol & 7);
    part[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  }
  const uint2 lo = __builtin_bit_cast(uint2, part[0]);
  const uint2 hi = __builtin_bit_cast(uint2, part[1]);
  Frag<uint16_t> a;
  a.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return a;
}

// Pack 8 fp32 values to one bf16 fragment (round to nearest even).
__device__ inline Frag<uint16_t> pack_bf16(const float (&x)[8]) {
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2_t pk = {static_cast<__bf16>(x[2 * j]), static_cast<__bf16>(x[2 * j + 1])};
    wd[j] = __builtin_bit_cast(uint32_t, pk);
  }
  Frag<uint16_t> f;
  f.v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  return f;
}

// Clear the bf16 elements of a packed fragment whose index is in the pair masks: word j
// holds elements 2j (low half) and 2j+1.  keep_sign leaves the sign bit, which is what
// multiplying the value by +0 before packing gives.
__device__ inline void clear_bf16(Frag<uint16_t>& f, const uint32_t (&drop)[4], bool keep_sign) {
  const uint32_t keep = keep_sign ? 0x80008000u : 0u;
  f.v = make_uint4(f.v.x & (~drop[0] | keep), f.v.y & (~drop[1] | keep), f.v.z & (~drop[2] | keep),
                   f.v.w & (~drop[3] | keep));
}

// Store a transposed [32 x 32*kOut] accumulator (lane = token row, registers = columns)
// as fp32 rows of D: acc[io][4g + t] is column 32io + 8g + 4hf + t.
template <int kOut, int D>
__device__ inline void store_rows(float* row, const f32x16_t (&acc)[kOut], float mul, int hf) {
#pragma unroll
  for (int io = 0; io < kOut; ++io)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * io + 8 * g + 4 * hf;
      *reinterpret_cast<float4*>(row + d0) =
          make_float4(acc[io][4 * g] * mul, acc[io][4 * g + 1] * mul, acc[io][4 * g + 2] * mul,
                      acc[io][4 * g + 3] * mul);
    }
}

// ------------------------------------------------------------------ dQ over CSR rows
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2))) void dq_kernel(BwdArgs a) {
  using T = uint16_t;
  constexpr int KT = (D == 128 && BLK == 64) ? 32 : 64;
  constexpr int kSteps = BLK / KT;
  constexpr int kWaves = BLK / 32;
  constexpr int NT = 64 * kWaves;
  constexpr int GPR = D * 2 / 16;
  constexpr int NGS = KT * GPR;
  constexpr int NLD = NGS / NT;
  constexpr int kQk = D / 16, kSub = KT / 32, kPv = KT / 16, kOut = D / 32;
  static_assert(NGS % NT == 0 && BLK % KT == 0, "tile shape");

  __shared__ uint4 Kt[2][NGS];
  __shared__ uint4 Vt[2][NGS];

  const int N = a.N, Nb = a.Nb, H = a.H;
  const int total_rows = a.B * H * Nb;
  const int pos = xcd_row(blockIdx.x, total_rows);
  const int row = a.order ? __builtin_amdgcn_readfirstlane(a.order[pos]) : pos;
  const int bh = row / Nb, r = row - bh * Nb, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int qi = r * BLK + w * 32 + qn;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);

  const int e0 = __builtin_amdgcn_readfirstlane(a.row_ptr[row]);
  int e1 = __builtin_amdgcn_readfirstlane(a.row_ptr[row + 1]);
  if ((a.skip_bits[h >> 5] >> (h & 31)) & 1u) e1 = e0;

  f32x16_t acc[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) acc[io] = f32x16_t{};

  if (e1 > e0) {
    Frag<T> qf[kQk], df[kQk];
    float lse2 = 0.f, dd = 0.f;
#pragma unroll
    for (int t = 0; t < kQk; ++t) {
      if (qi < N) {
        qf[t] = lds_frag(Q + head + (size_t)qi * D + 16 * t + 8 * hf);
        df[t] = lds_frag(dO + head + (size_t)qi * D + 16 * t + 8 * hf);
      } else {
        qf[t] = Frag<T>{};
        df[t] = Frag<T>{};
      }
    }
    if (qi < N) {
      const float2 p = *reinterpret_cast<const float2*>(a.ld + 2 * ((size_t)bh * N + qi));
      lse2 = p.x;
      dd = p.y;
    }
    const uint32_t wave_off = (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
    const uint32_t k_lds[2] = {lds_addr(Kt[0]) + wave_off, lds_addr(Kt[1]) + wave_off};
    const uint32_t v_lds[2] = {lds_addr(Vt[0]) + wave_off, lds_addr(Vt[1]) + wave_off};
    uint32_t off[NLD];
#pragma unroll
    for (int it = 0; it < NLD; ++it) off[it] = dma_offset<T, D, NT>(it, tid, KT);
    auto dma_step = [&](const T* ksrc, const T* vsrc, int slot, int nv) {
      if (nv == KT) {
        static_for<NLD>([&](auto it) {
          dma16<it.value * NT * 16>(ksrc, off[it.value], k_lds[slot]);
          dma16<it.value * NT * 16>(vsrc, off[it.value], v_lds[slot]);
        });
      } else {
        static_for<NLD>([&](auto it) {
          const uint32_t o = dma_offset<T, D, NT>(it.value, tid, nv);
          dma16<it.value * NT * 16>(ksrc, o, k_lds[slot]);
          dma16<it.value * NT * 16>(vsrc, o, v_lds[slot]);
        });
      }
    };
    int cbase = e0;
    int cvec = e0 + lane < e1 ? a.col_idx[e0 + lane] : 0;
    // the query, dO, (lse, D) and index loads above are done before any transfer: the
    // compiler does not see the transfers and would otherwise wait on them in the loop
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    int e = e0, hh = 0;
    int c = __builtin_amdgcn_readlane(cvec, 0);
    int nkv = min(BLK, N - c * BLK);
    int slot = 0;
    {
      const size_t src = head + (size_t)c * BLK * D;
      dma_step(K + src, V + src, 0, min(KT, nkv));
    }
    for (;;) {
      int e_n = e, hh_n = hh + 1, c_n = c, nkv_n = nkv;
      if (hh_n >= kSteps || hh_n * KT >= nkv) {
        e_n = e + 1;
        hh_n = 0;
        if (e_n < e1) {
          if (e_n - cbase == 64) {
            cbase += 64;
            cvec = cbase + lane < e1 ? a.col_idx[cbase + lane] : 0;
          }
          c_n = __builtin_amdgcn_readlane(cvec, e_n - cbase);
          nkv_n = min(BLK, N - c_n * BLK);
        }
      }
      const bool more = e_n < e1;
      const int nv = min(KT, nkv - hh * KT);

      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      if (more) {
        const size_t src = head + ((size_t)c_n * BLK + hh_n * KT) * D;
        dma_step(K + src, V + src, slot ^ 1, min(KT, nkv_n - hh_n * KT));
      }
      const uint4* kt = Kt[slot];
      const uint4* vt = Vt[slot];

      // per 32-key subtile: S^T = K Q^T and dP^T = V dO^T (keys on rows, this lane's
      // query on the column), then P^T = exp2(S^T scale log2e - lse log2e) (keys past nv
      // weigh 0) and dS^T = P^T (dP^T - D), rounded to bf16 for the MFMA
      Frag<T> dsf[kPv];
#pragma unroll
      for (int is = 0; is < kSub; ++is) {
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
        const int kr = 32 * is + qn;
        // the K and V fragments of k-step t+2 are read before the products of k-step t
        // (an order fixed with scheduling fences)
        auto kv_frag = [&](int t, Frag<T>& ka, Frag<T>& va) {
          ka.v = kt[kr * GPR + ((2 * t + hf) ^ swz<GPR>(kr))];
          va.v = vt[kr * GPR + ((2 * t + hf) ^ swz<GPR>(kr))];
        };
        Frag<T> ka[3], va[3];
        kv_frag(0, ka[0], va[0]);
        kv_frag(1, ka[1], va[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kQk; ++t) {
          if (t + 2 < kQk) kv_frag(t + 2, ka[(t + 2) % 3], va[(t + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
          mma_k16(s, ka[t % 3], qf[t]);
          mma_k16(dp, va[t % 3], df[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * h2 + j;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -lse2));
            x[j] = p * (dp[i] - dd);
          }
          dsf[2 * is + h2] = pack_bf16(x);
          if (nv < KT) {   // keys past N (the last, partial key block only): P = 0, so dS = +-0
            // element 2j is key 32is + 8(2h2 + j/2) + 4hf + 2(j%2), compared as a constant
            // against nv - 4hf so that no key index stays live across the loop
            const int nvh = nv - 4 * hf;
            uint32_t drop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = 32 * is + 8 * (2 * h2 + (j >> 1)) + 2 * (j & 1);
              drop[j] = (key >= nvh ? 0x0000FFFFu : 0u) | (key + 1 >= nvh ? 0xFFFF0000u : 0u);
            }
            clear_bf16(dsf[2 * is + h2], drop, true);
          }
        }
      }
      // dQ^T += K^T dS^T (K^T fragments by transpose reads of the K tile, the next pair's
      // read before the current pair's product)
      const uint16_t* ktile = reinterpret_cast<const uint16_t*>(kt);
      {
        constexpr int kPairs = kOut * kPv;
        Frag<T> tk[2];
        tk[0] = tr_frag<D>(ktile, 0, 0, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pp = 0; pp < kPairs; ++pp) {
          if (pp + 1 < kPairs) tk[(pp + 1) % 2] = tr_frag<D>(ktile, (pp + 1) / kPv, (pp + 1) % kPv, lane);
          __builtin_amdgcn_sched_barrier(0);
          mma_k16(acc[pp / kPv], tk[pp % 2], dsf[pp % kPv]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      if (!more) break;
      e = e_n;
      hh = hh_n;
      c = c_n;
      nkv = nkv_n;
      slot ^= 1;
    }
  }
  if (qi < N) store_rows<kOut, D>(a.dq + head + (size_t)qi * D, acc, a.scale, hf);
}

// ------------------------------------------------------------------ dK, dV over CSC
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2))) void dkv_kernel(BwdArgs a) {
  using T = uint16_t;
  constexpr int QT = 32;                 // queries per step
  constexpr int kSteps = BLK / QT;       // steps per query block
  constexpr int kWaves = BLK / 32;
  constexpr int NT = 64 * kWaves;
  constexpr int GPR = D * 2 / 16;
  constexpr int NGS = QT * GPR;          // granules per Q (or dO) step tile
  constexpr int NLD = NGS / NT;
  constexpr int kLdGran = QT * 2 * 4 / 16;       // (lse, D) pairs of a step: 16 granules
  constexpr int kLdLanes = kLdGran / kWaves;     // lanes per wave that move them
  constexpr int kQk = D / 16, kPv = QT / 16, kOut = D / 32;
  static_assert(NGS % NT == 0 && kLdGran % kWaves == 0, "tile shape");

  __shared__ uint4 Qs[2][NGS];
  __shared__ uint4 Gs[2][NGS];           // dO
  __shared__ uint4 Ls[2][kLdGran];       // (lse * log2e, D) per query
  __shared__ uint4 Vf[kQk][NT];          // each lane's V fragments (lane-private, k-major)

  const int N = a.N, Nb = a.Nb, H = a.H;
  const int total = a.B * H * Nb;
  const int col = __builtin_amdgcn_readfirstlane(a.col_order[xcd_row(blockIdx.x, total)]);
  const int bh = col / Nb, c = col - bh * Nb, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int kk = c * BLK + w * 32 + qn;   // this lane's key (B-operand column, output row)
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* dO = static_cast<const T*>(a.dout);

  const int f0 = __builtin_amdgcn_readfirstlane(a.col_ptr[col]);
  int f1 = __builtin_amdgcn_readfirstlane(a.col_ptr[col + 1]);
  if ((a.skip_bits[h >> 5] >> (h & 31)) & 1u) f1 = f0;

  f32x16_t dk[kOut], dv[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) {
    dk[io] = f32x16_t{};
    dv[io] = f32x16_t{};
  }

  if (f1 > f0) {
    // this lane's K fragments stay in registers; its V fragments are parked in LDS (only
    // this lane reads them back), which keeps the accumulators out of scratch
    Frag<T> kf[kQk];
    const int kr = min(kk, N - 1);   // keys past N: any finite row (their outputs are not stored)
#pragma unroll
    for (int t = 0; t < kQk; ++t) {
      kf[t] = lds_frag(K + head + (size_t)kr * D + 16 * t + 8 * hf);
      Vf[t][tid] = lds_frag(V + head + (size_t)kr * D + 16 * t + 8 * hf).v;
    }
    const uint32_t wave_off = (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
    const uint32_t q_lds[2] = {lds_addr(Qs[0]) + wave_off, lds_addr(Qs[1]) + wave_off};
    const uint32_t g_lds[2] = {lds_addr(Gs[0]) + wave_off, lds_addr(Gs[1]) + wave_off};
    const uint32_t l_off = (uint32_t)__builtin_amdgcn_readfirstlane(w) * (uint32_t)(kLdLanes * 16);
    const uint32_t l_lds[2] = {lds_addr(Ls[0]) + l_off, lds_addr(Ls[1]) + l_off};
    const int lg = w * kLdLanes + lane;   // (lse, D) granule moved by this lane (if < kLdGran)
    auto dma_step = [&](int r, int hq, int slot, int nq) {
      const size_t qrow0 = (size_t)r * BLK + hq * QT;
      const T* qsrc = Q + head + qrow0 * D;
      const T* gsrc = dO + head + qrow0 * D;
      static_for<NLD>([&](auto it) {
        const uint32_t o = dma_offset<T, D, NT>(it.value, tid, nq);
        dma16<it.value * NT * 16>(qsrc, o, q_lds[slot]);
        dma16<it.value * NT * 16>(gsrc, o, g_lds[slot]);
      });
      if (lane < kLdLanes) {
        // granule lg holds queries 2lg, 2lg+1; past nq re-read the last valid pair
        const int gq = min(lg, (nq - 1) >> 1);
        dma16<0>(a.ld + 2 * ((size_t)bh * N + qrow0), (uint32_t)gq * 16u, l_lds[slot]);
      }
    };
    // cursor over (query block r, step hq) of this key block's query blocks
    int fbase = f0;
    int rvec = f0 + lane < f1 ? a.row_idx[f0 + lane] : 0;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // K, V fragments and indices before transfers
    int f = f0, hq = 0;
    int r = __builtin_amdgcn_readlane(rvec, 0);
    int nqb = min(BLK, N - r * BLK);
    int slot = 0;
    dma_step(r, 0, 0, min(QT, nqb));
    for (;;) {
      int f_n = f, hq_n = hq + 1, r_n = r, nqb_n = nqb;
      if (hq_n >= kSteps || hq_n * QT >= nqb) {
        f_n = f + 1;
        hq_n = 0;
        if (f_n < f1) {
          if (f_n - fbase == 64) {
            fbase += 64;
            rvec = fbase + lane < f1 ? a.row_idx[fbase + lane] : 0;
          }
          r_n = __builtin_amdgcn_readlane(rvec, f_n - fbase);
          nqb_n = min(BLK, N - r_n * BLK);
        }
      }
      const bool more = f_n < f1;
      const int nq = min(QT, nqb - hq * QT);

      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      wg_barrier();
      if (more) dma_step(r_n, hq_n, slot ^ 1, min(QT, nqb_n - hq_n * QT));
      const uint4* qt = Qs[slot];
      const uint4* gt = Gs[slot];
      const float* lt = reinterpret_cast<const float*>(Ls[slot]);

      // S = Q K^T, dP = dO V^T (queries on rows, this lane's key on the column); the
      // operands of k-step t+1 are read before the products of k-step t (scheduling fences)
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      {
        auto ops = [&](int t, Frag<T>& qa, Frag<T>& ga, Frag<T>& va) {
          qa.v = qt[qn * GPR + ((2 * t + hf) ^ swz<GPR>(qn))];
          ga.v = gt[qn * GPR + ((2 * t + hf) ^ swz<GPR>(qn))];
          va.v = Vf[t][tid];
        };
        Frag<T> qa[2], ga[2], va[2];
        ops(0, qa[0], ga[0], va[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kQk; ++t) {
          if (t + 1 < kQk) ops(t + 1, qa[(t + 1) % 2], ga[(t + 1) % 2], va[(t + 1) % 2]);
          __builtin_amdgcn_sched_barrier(0);
          mma_k16(s, qa[t % 2], kf[t]);
          mma_k16(dp, ga[t % 2], va[t % 2]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // P = exp2(S scale log2e - lse log2e), dS = P (dP - D); queries past nq get 0
      Frag<T> pf[kPv], dsf[kPv];
#pragma unroll
      for (int u = 0; u < kPv; ++u) {
        float pv[8], dsv[8];
#pragma unroll
        for (int j4 = 0; j4 < 2; ++j4) {
          const int q0 = 16 * u + 8 * j4 + 4 * hf;   // 4 consecutive queries
          const float4 l01 = *reinterpret_cast<const float4*>(lt + 2 * q0);
          const float4 l23 = *reinterpret_cast<const float4*>(lt + 2 * q0 + 4);
          const float ls[4] = {l01.x, l01.z, l23.x, l23.z};
          const float ds_[4] = {l01.y, l01.w, l23.y, l23.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int i = 8 * u + 4 * j4 + t;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -ls[t]));
            pv[4 * j4 + t] = p;
            dsv[4 * j4 + t] = p * (dp[i] - ds_[t]);
          }
        }
        pf[u] = pack_bf16(pv);
        dsf[u] = pack_bf16(dsv);
        if (nq < QT) {   // queries past N (the last, partial query block only): P = 0, dS = +-0
          // element 2j is query 16u + 8(j/2) + 4hf + 2(j%2), compared against nq - 4hf
          const int nqh = nq - 4 * hf;
          uint32_t drop[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int q = 16 * u + 8 * (j >> 1) + 2 * (j & 1);
            drop[j] = (q >= nqh ? 0x0000FFFFu : 0u) | (q + 1 >= nqh ? 0xFFFF0000u : 0u);
          }
          clear_bf16(pf[u], drop, false);
          clear_bf16(dsf[u], drop, true);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transpose reads)
      const uint16_t* qtile = reinterpret_cast<const uint16_t*>(qt);
      const uint16_t* gtile = reinterpret_cast<const uint16_t*>(gt);
      // product p: (io, u) = (p / 2kPv, p / 2 % kPv), dV for even p and dK for odd p; the
      // transposed operand of product p+3 is read before product p (scheduling fences).
      // Three ahead: the LDS round trip of each read stays under three products.
      {
        constexpr int kProd = 2 * kOut * kPv, AHEAD = 3;
        auto trf = [&](int p) { return tr_frag<D>((p & 1) ? qtile : gtile, p / (2 * kPv), (p / 2) % kPv, lane); };
        Frag<T> ta[AHEAD + 1];
#pragma unroll
        for (int p = 0; p < AHEAD; ++p) ta[p] = trf(p);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < kProd; ++p) {
          if (p + AHEAD < kProd) ta[(p + AHEAD) % (AHEAD + 1)] = trf(p + AHEAD);
          __builtin_amdgcn_sched_barrier(0);
          const int io = p / (2 * kPv), u = (p / 2) % kPv;
          if (p & 1)
            mma_k16(dk[io], ta[p % (AHEAD + 1)], dsf[u]);
          else
            mma_k16(dv[io], ta[p % (AHEAD + 1)], pf[u]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      if (!more) break;
      f = f_n;
      hq = hq_n;
      r = r_n;
      nqb = nqb_n;
      slot ^= 1;
    }
  }
  if (kk < N) {
    store_rows<kOut, D>(a.dk + head + (size_t)kk * D, dk, a.scale, hf);
    store_rows<kOut, D>(a.dv + head + (size_t)kk * D, dv, 1.f, hf);
  }
}

// ------------------------------------------------------------------ fp32 inputs
// fp32 Q, K, V and dO: the same products on the fp32 matrix cores (eight
// v_mfma_f32_32x32x2f32 per 16-wide k-step, through mma_k16) with P and dS kept in fp32.
// One such product does 4096 flops for 512 bytes of operands in 64 cycles, a sixteenth of
// the bf16 flop rate, so operand traffic is no constraint here: every wavefront reads its
// fragments straight from global memory (the wavefronts of a workgroup share them through
// the caches), with no LDS staging and no barriers.  Reads of keys or queries past N are
// clamped to the last valid row of the block, and those elements get weight 0.

// Column fragment: element j = rows[r(j) * D + col], r(j) = r0 + 8(j/4) + 4hf + j%4 clamped
// to `last` (the k order of the 32x32 output layout, as for the transposed bf16 fragments).
template <int D>
__device__ inline Frag<float> col_frag(const float* rows, int r0, int hf, int last, int col) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = min(r0 + 8 * (j >> 2) + 4 * hf + (j & 3), last);
    v[j] = rows[(size_t)r * D + col];
  }
  Frag<float> f;
  f.a = make_float4(v[0], v[1], v[2], v[3]);
  f.b = make_float4(v[4], v[5], v[6], v[7]);
  return f;
}

__device__ inline Frag<float> frag8(const float (&x)[16], int u) {
  Frag<float> f;
  f.a = make_float4(x[8 * u], x[8 * u + 1], x[8 * u + 2], x[8 * u + 3]);
  f.b = make_float4(x[8 * u + 4], x[8 * u + 5], x[8 * u + 6], x[8 * u + 7]);
  return f;
}

// dQ over CSR rows, 32-key steps: S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, dQ^T += K^T dS^T.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void dq_f32_kernel(BwdArgs a) {
  constexpr int kQk = D / 16, kOut = D / 32;
  const int N = a.N, Nb = a.Nb, H = a.H;
  const int total_rows = a.B * H * Nb;
  const int pos = xcd_row(blockIdx.x, total_rows);
  const int row = a.order ? __builtin_amdgcn_readfirstlane(a.order[pos]) : pos;
  const int bh = row / Nb, r = row - bh * Nb, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int qi = r * BLK + w * 32 + qn;
  const float* Q = static_cast<const float*>(a.q) + head;
  const float* K = static_cast<const float*>(a.k) + head;
  const float* V = static_cast<const float*>(a.v) + head;
  const float* dO = static_cast<const float*>(a.dout) + head;

  const int e0 = __builtin_amdgcn_readfirstlane(a.row_ptr[row]);
  int e1 = __builtin_amdgcn_readfirstlane(a.row_ptr[row + 1]);
  if ((a.skip_bits[h >> 5] >> (h & 31)) & 1u) e1 = e0;

  f32x16_t acc[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) acc[io] = f32x16_t{};
  if (e1 > e0) {
    const int qr = min(qi, N - 1);
    float lse2 = INFINITY, dd = 0.f;   // a query past N: +inf makes every weight 0
    if (qi < N) {
      const float2 p = *reinterpret_cast<const float2*>(a.ld + 2 * ((size_t)bh * N + qi));
      lse2 = p.x;
      dd = p.y;
    }
    Frag<float> qf[kQk];
#pragma unroll
    for (int t = 0; t < kQk; ++t) qf[t] = lds_frag(Q + (size_t)qr * D + 16 * t + 8 * hf);
    for (int e = e0; e < e1; ++e) {
      const int c = __builtin_amdgcn_readfirstlane(a.col_idx[e]);
      const int nkv = min(BLK, N - c * BLK);
      for (int k0 = 0; k0 < nkv; k0 += 32) {
        const int nv = min(32, nkv - k0);
        const float* kb = K + (size_t)(c * BLK + k0) * D;
        const float* vb = V + (size_t)(c * BLK + k0) * D;
        const int kr = min(qn, nv - 1);
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int t = 0; t < kQk; ++t) {
          mma_k16(s, lds_frag(kb + (size_t)kr * D + 16 * t + 8 * hf), qf[t]);
          mma_k16(dp, lds_frag(vb + (size_t)kr * D + 16 * t + 8 * hf),
                  lds_frag(dO + (size_t)qr * D + 16 * t + 8 * hf));
        }
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
          const float p = key < nv ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -lse2)) : 0.f;
          ds[i] = p * (dp[i] - dd);
        }
#pragma unroll
        for (int io = 0; io < kOut; ++io)
#pragma unroll
          for (int u = 0; u < 2; ++u) mma_k16(acc[io], col_frag<D>(kb, 16 * u, hf, nv - 1, 32 * io + qn), frag8(ds, u));
      }
    }
  }
  if (qi < N) store_rows<kOut, D>(a.dq + head + (size_t)qi * D, acc, a.scale, hf);
}

// dK, dV over the transposed mask, 32-query steps: S = Q K^T, dP = dO V^T, P, dS,
// dV^T += dO^T P, dK^T += Q^T dS (32 keys per wavefront, one key per lane column).
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void dkv_f32_kernel(BwdArgs a) {
  constexpr int kQk = D / 16, kOut = D / 32;
  const int N = a.N, Nb = a.Nb, H = a.H;
  const int total = a.B * H * Nb;
  const int col = __builtin_amdgcn_readfirstlane(a.col_order[xcd_row(blockIdx.x, total)]);
  const int bh = col / Nb, c = col - bh * Nb, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int kk = c * BLK + w * 32 + qn;
  const float* Q = static_cast<const float*>(a.q) + head;
  const float* K = static_cast<const float*>(a.k) + head;
  const float* V = static_cast<const float*>(a.v) + head;
  const float* dO = static_cast<const float*>(a.dout) + head;
  const float* ld = a.ld + 2 * (size_t)bh * N;

  const int f0 = __builtin_amdgcn_readfirstlane(a.col_ptr[col]);
  int f1 = __builtin_amdgcn_readfirstlane(a.col_ptr[col + 1]);
  if ((a.skip_bits[h >> 5] >> (h & 31)) & 1u) f1 = f0;

  f32x16_t dk[kOut], dv[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) {
    dk[io] = f32x16_t{};
    dv[io] = f32x16_t{};
  }
  if (f1 > f0) {
    const int kr = min(kk, N - 1);   // keys past N: any finite row (their outputs are not stored)
    Frag<float> kf[kQk];
#pragma unroll
    for (int t = 0; t < kQk; ++t) kf[t] = lds_frag(K + (size_t)kr * D + 16 * t + 8 * hf);
    for (int f = f0; f < f1; ++f) {
      const int r = __builtin_amdgcn_readfirstlane(a.row_idx[f]);
      const int nqb = min(BLK, N - r * BLK);
      for (int q0 = 0; q0 < nqb; q0 += 32) {
        const int nq = min(32, nqb - q0);
        const int qg = r * BLK + q0;
        const float* qb = Q + (size_t)qg * D;
        const float* gb = dO + (size_t)qg * D;
        const int qr = min(qn, nq - 1);
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int t = 0; t < kQk; ++t) {
          mma_k16(s, lds_frag(qb + (size_t)qr * D + 16 * t + 8 * hf), kf[t]);
          mma_k16(dp, lds_frag(gb + (size_t)qr * D + 16 * t + 8 * hf),
                  lds_frag(V + (size_t)kr * D + 16 * t + 8 * hf));
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = 8 * (i >> 2) + 4 * hf + (i & 3);
          float p = 0.f, dsi = 0.f;
          if (q < nq) {
            const float2 l = *reinterpret_cast<const float2*>(ld + 2 * (size_t)(qg + q));
            p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], a.scale_log2, -l.x));
            dsi = p * (dp[i] - l.y);
          }
          pv[i] = p;
          dsv[i] = dsi;
        }
#pragma unroll
        for (int io = 0; io < kOut; ++io)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            mma_k16(dv[io], col_frag<D>(gb, 16 * u, hf, nq - 1, 32 * io + qn), frag8(pv, u));
            mma_k16(dk[io], col_frag<D>(qb, 16 * u, hf, nq - 1, 32 * io + qn), frag8(dsv, u));
          }
      }
    }
  }
  if (kk < N) {
    store_rows<kOut, D>(a.dk + head + (size_t)kk * D, dk, a.scale, hf);
    store_rows<kOut, D>(a.dv + head + (size_t)kk * D, dv, 1.f, hf);
  }
}

template <int D, int BLK>
hipError_t launch_grads(const BwdArgs& a, hipStream_t s) {
  const int rows = a.B * a.H * a.Nb;
  if (a.in_f32)
    hipLaunchKernelGGL((dq_f32_kernel<D, BLK>), dim3((unsigned)rows), dim3(BLK * 2), 0, s, a);
  else
    hipLaunchKernelGGL((dq_kernel<D, BLK>), dim3((unsigned)rows), dim3(BLK * 2), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.in_f32)
    hipLaunchKernelGGL((dkv_f32_kernel<D, BLK>), dim3((unsigned)rows), dim3(BLK * 2), 0, s, a);
  else
    hipLaunchKernelGGL((dkv_kernel<D, BLK>), dim3((unsigned)rows), dim3(BLK * 2), 0, s, a);
  return hipGetLastError();
}

template <typename TG, int D>
void launch_prep(const BwdArgs& a, dim3 grid, size_t nq, hipStream_t s) {
  if (a.o_bf16)
    hipLaunchKernelGGL((bwd_prep_kernel<TG, uint16_t, D>), grid, dim3(256), 0, s,
                       static_cast<const TG*>(a.dout), static_cast<const uint16_t*>(a.o), a.lse, a.ld, nq);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<TG, float, D>), grid, dim3(256), 0, s,
                       static_cast<const TG*>(a.dout), static_cast<const float*>(a.o), a.lse, a.ld, nq);
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_layout(const BwdArgs& g, BwdArgs* a, void* base) {
  const size_t rows = (size_t)g.B * g.H * g.Nb;
  const size_t nq = (size_t)g.B * g.H * g.N;
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  // (lse, D) pairs, padded so a step's 16-byte granules never pass the end
  float* ld = static_cast<float*>(take((2 * nq + 64) * sizeof(float)));
  int32_t* col_ptr = static_cast<int32_t*>(take((rows + 1) * sizeof(int32_t)));
  int32_t* row_idx = static_cast<int32_t*>(take(rows * g.Nb * sizeof(int32_t)));
  int32_t* col_order = static_cast<int32_t*>(take(rows * sizeof(int32_t)));
  if (a) {
    a->ld = ld;
    a->col_ptr = col_ptr;
    a->row_idx = row_idx;
    a->col_order = col_order;
  }
  return off;
}

hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t s) {
  const size_t nq = (size_t)a.B * a.H * a.N;
  const size_t threads = nq * (size_t)(a.d / 8);
  const dim3 pgrid((unsigned)((threads + 255) / 256));
  if (a.in_f32)
    a.d == 128 ? launch_prep<float, 128>(a, pgrid, nq, s) : launch_prep<float, 64>(a, pgrid, nq, s);
  else
    a.d == 128 ? launch_prep<uint16_t, 128>(a, pgrid, nq, s) : launch_prep<uint16_t, 64>(a, pgrid, nq, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csc_kernel, dim3((unsigned)(a.B * a.H)), dim3(kCscThreads), 0, s, a.row_ptr, a.col_idx,
                     a.col_ptr, a.row_idx, a.Nb, a.B * a.H);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  SkipBits sk;
  for (int i = 0; i < kMaxHeads / 32; ++i) sk.bits[i] = a.skip_bits[i];
  hipLaunchKernelGGL(col_order_kernel, dim3(kXcds), dim3(kOrderThreads), 0, s, a.col_ptr, a.col_order, a.Nb,
                     a.H, a.B * a.H * a.Nb, sk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 128 && a.blk == 128) return launch_grads<128, 128>(a, s);
  if (a.d == 128 && a.blk == 64) return launch_grads<128, 64>(a, s);
  if (a.d == 64 && a.blk == 128) return launch_grads<64, 128>(a, s);
  return launch_grads<64, 64>(a, s);
}

}  // namespace asa
