// Block-sparse attention forward for gfx950 (MI355X).
//
// Computes, per head, softmax(Q K^T / sqrt(d)) V restricted to the kept
// (query-block, key-block) tiles of a CSR block mask: the masked attention
// Attention(Q, K, V, M) of Sparse-vDiT ("Sparse-vDiT: Sparse Attention Acceleration for
// Video Diffusion Transformers", section 三 "核心公式"), with M given per query block as
// the list of kept key blocks.  Skipped heads (mode M1 in the same page's
// "四种注意力模式" table) produce zeros.
//
// Work decomposition: one workgroup per (b, h, query block r); BLK/32 wavefronts, each
// owning 32 query rows.  Kept key blocks are consumed in steps of 32 or 64 keys (chosen per
// launch): K and V of a step
// land row-major (16-byte granules swizzled) in one slot of a two-slot LDS ring by direct
// global -> LDS transfers, and each wavefront computes
//     S^T = K_c Q^T          (32x32x16 bf16 MFMA, or 32x32x2 f32 MFMA for fp32 inputs)
//     online softmax          (exp2 with the scale folded in, running max / sum per row)
//     O^T += V_c^T P^T        (same MFMA shape; V^T fragments by transpose reads)
// Computing the transposed products makes every lane own one query row: the S^T
// accumulator layout puts 16 keys of query (lane % 32) in each lane, and the O^T layout
// puts 16 output columns of the same query there, so the softmax statistics and the
// rescale stay lane-local (one cross-half exchange per tile for the row max).
//
// MFMA 32x32 output layout used throughout: lane l, accumulator register i holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.
#include <hip/hip_runtime.h>

#include "attn_common.h"

namespace asa {
namespace {

// Each kept key block is consumed in steps of KT keys.  K and V of a step share one slot of
// a two-slot LDS ring: while the workgroup computes on one slot, the next step's K and V
// stream into the other, so a step needs a single barrier.  The step loop is unrolled by
// two so that each copy works on a fixed slot (fixed LDS addresses, no per-step address
// arithmetic).
// kSplit: the launch cuts long rows into chunks (meta.split_blocks > 0); a separate
// instantiation keeps the registers of the plain kernel untouched.
// KT: keys per step.  32-key steps keep a d = 128 kernel under 168 registers and 32 KB of
// LDS, so three wavefronts share a SIMD; launches with enough rows to fill those slots use
// them (128-query blocks), as do all d = 128 launches with 64-query blocks (two wavefronts
// per SIMD there).  64-key steps do more work per barrier, which wins when a compute unit
// holds fewer workgroups (small launches, d = 64).
template <typename T, typename TO, int D, int BLK, int KT, bool kSplit>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(KT == 32 && BLK == 128 ? 3 : 2))) void attn_fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, TO* __restrict__ O,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int H, int N, int Nb,
    int total_rows, float scale_log2, AttnArgs meta) {
  constexpr int kSteps = BLK / KT; // steps per key block
  constexpr int kWaves = BLK / 32;
  constexpr int NT = 64 * kWaves;
  constexpr int G = Elem<T>::kGran;
  constexpr int GPR = D * (int)sizeof(T) / 16;
  constexpr int NGS = KT * GPR;    // granules per step tile
  constexpr int NLD = NGS / NT;    // DMA instructions per thread per step tile
  constexpr int kQk = D / 16;      // k-steps of S^T = K Q^T
  constexpr int kSub = KT / 32;    // 32-key subtiles per step
  constexpr int kPv = KT / 16;     // k-steps of O^T = V^T P^T
  constexpr int kOut = D / 32;     // 32-column output subtiles
  constexpr bool kBf16 = sizeof(T) == 2;
  // The running max is only moved when a row's max grows by more than this (log2 units):
  // weights are then at most 2^32, exact up to rounding, and the O / l rescale is skipped.
  // The scores of a row span tens of log2 units on video attention, so a small slack
  // rescales often (about one step in six at 2^8, one in twenty-five at 2^32 on the Wan
  // layer).  The fp32 accumulator stays finite while 2^32 x max|V| x (kept keys) does,
  // i.e. for |V| below 2^79.
  constexpr float kRescaleSlack = 32.0f;
  static_assert(NGS % NT == 0, "tile must split evenly over the workgroup");
  static_assert(GPR >= 8, "swizzle needs at least 8 granules per row");
  static_assert(BLK % KT == 0, "block must be a whole number of steps");

  __shared__ uint4 Kt[2][NGS];
  __shared__ uint4 Vt[2][NGS];

  // work item -> position in the processing order (and, with split rows, the chunk of the
  // row).  Positions map to rows through a permutation from the mask builder, which gives
  // every XCD an equal share of each row-length class, long rows first, or the identity.
  int pos, chunk = 0;
  if constexpr (kSplit) {
    // each XCD walks its own range of rows, all chunks of a row together; the grid is
    // padded to 8 equal shares, so surplus items exit
    const int x = blockIdx.x % kXcds, t = blockIdx.x / kXcds;
    int lo, hi;
    xcd_range(x, total_rows, lo, hi);
    const int pl = t / meta.split_max;
    if (pl >= hi - lo) return;
    chunk = t - pl * meta.split_max;
    pos = lo + pl;
  } else {
    pos = xcd_row(blockIdx.x, total_rows);
  }
  const int row = meta.order ? __builtin_amdgcn_readfirstlane(meta.order[pos]) : pos;
  const int bh = row / Nb, r = row - bh * Nb, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int qi = r * BLK + w * 32 + qn;

  // CSR bounds and block indices are wave-uniform: keep them in scalar registers
  int e0 = __builtin_amdgcn_readfirstlane(row_ptr[row]);
  int e1 = __builtin_amdgcn_readfirstlane(row_ptr[row + 1]);
  if ((meta.skip_bits[h >> 5] >> (h & 31)) & 1u) e1 = e0;
  // a long row is cut into near-equal chunks of at most split_blocks kept blocks
  int n_chunks = 1;
  if constexpr (kSplit) {
    const int cnt = e1 - e0;
    if (cnt > meta.split_blocks) n_chunks = (cnt + meta.split_blocks - 1) / meta.split_blocks;
    if (chunk >= n_chunks) return;
    if (n_chunks > 1) {
      const int a0 = e0 + (int)(((long long)chunk * cnt) / n_chunks);
      e1 = e0 + (int)(((long long)(chunk + 1) * cnt) / n_chunks);
      e0 = a0;
    }
  }

  f32x16_t acc[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) acc[io] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  // bf16 inputs: the row sums of the rounded weights run on the matrix cores.  A 4x4x4
  // product with an all-ones operand adds the four weights a lane holds into that lane's
  // own accumulator column (its four elements carry the same sum).  A v_dot2 row sum issues
  // on the matrix pipeline as well but holds up the partner wavefronts' products.
  f32x4_t l_mma = f32x4_t{};
  auto psum = [&](const uint4& v) {
    const short4_t ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};   // bf16 1.0
    l_mma = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones, __builtin_bit_cast(short4_t, make_uint2(v.x, v.y)), l_mma, 0, 0, 0);
    l_mma = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones, __builtin_bit_cast(short4_t, make_uint2(v.z, v.w)), l_mma, 0, 0, 0);
  };

  if (e1 > e0) {
    Frag<T> qf[kQk];
#pragma unroll
    for (int t = 0; t < kQk; ++t) {
      if (qi < N) {
        qf[t] = lds_frag(Q + head + (size_t)qi * D + 16 * t + 8 * hf);   // global, same shape
      } else {
        qf[t] = Frag<T>{};
      }
    }
    const uint32_t wave_off = (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
    const uint32_t k_lds[2] = {lds_addr(Kt[0]) + wave_off, lds_addr(Kt[1]) + wave_off};
    const uint32_t v_lds[2] = {lds_addr(Vt[0]) + wave_off, lds_addr(Vt[1]) + wave_off};
    // full-step transfer offsets, shared by K and V (same layout)
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
    // Kept block indices of this row, 64 at a time, one per lane (read back with readlane).
    int cbase = e0;
    int cvec = e0 + lane < e1 ? col_idx[e0 + lane] : 0;
    // current step: block e (index c, nkv valid keys), step hh within it
    int e = e0, hh = 0;
    int c = __builtin_amdgcn_readlane(cvec, 0);
    int nkv = min(BLK, N - c * BLK);
    {
      const size_t src = head + (size_t)c * BLK * D;
      dma_step(K + src, V + src, 0, min(KT, nkv));
    }

    // One step on ring slot kSlot (a compile-time constant, so the LDS addresses of both
    // slots are fixed and the slot offset is an immediate); returns whether a step follows.
    auto step = [&](auto slot_c) -> bool {
      constexpr int kSlot = decltype(slot_c)::value;
        // the step after this one (skips steps holding no valid key)
        int e_n = e, hh_n = hh + 1, c_n = c, nkv_n = nkv;
        if (hh_n >= kSteps || hh_n * KT >= nkv) {
          e_n = e + 1;
          hh_n = 0;
          if (e_n < e1) {
            if (e_n - cbase == 64) {   // next batch of indices (rows longer than 64 blocks)
              cbase += 64;
              cvec = cbase + lane < e1 ? col_idx[cbase + lane] : 0;
            }
            c_n = __builtin_amdgcn_readlane(cvec, e_n - cbase);
            nkv_n = min(BLK, N - c_n * BLK);
          }
        }
        const bool more = e_n < e1;
        const int nv = min(KT, nkv - hh * KT);   // valid keys in this step (>= 1)

        // this step's K and V landed everywhere; every wave is done with the other slot
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        wg_barrier();
        if (more) {
          const size_t src = head + ((size_t)c_n * BLK + hh_n * KT) * D;
          dma_step(K + src, V + src, kSlot ^ 1, min(KT, nkv_n - hh_n * KT));
        }
        const uint4* kt = Kt[kSlot];
        const T* vt = reinterpret_cast<const T*>(Vt[kSlot]);

        // S^T = K Q^T; the K fragment of k-step t+3 is read before the product of k-step t
        // (fixed with scheduling fences, as for the V^T fragments below)
        f32x16_t s[kSub];
  #pragma unroll
        for (int is = 0; is < kSub; ++is) {
          s[is] = f32x16_t{};
          const int kr = 32 * is + qn;
          auto kfrag = [&](int t) {
            Frag<T> a;
            if constexpr (kBf16) {
              a.v = kt[kr * GPR + ((2 * t + hf) ^ swz<GPR>(kr))];
            } else {
              a.a = *reinterpret_cast<const float4*>(&kt[kr * GPR + ((4 * t + 2 * hf) ^ swz<GPR>(kr))]);
              a.b = *reinterpret_cast<const float4*>(&kt[kr * GPR + ((4 * t + 2 * hf + 1) ^ swz<GPR>(kr))]);
            }
            return a;
          };
          Frag<T> ka[4];
          ka[0] = kfrag(0);
          if constexpr (kQk > 1) ka[1] = kfrag(1);
          if constexpr (kQk > 2) ka[2] = kfrag(2);
          __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
  #pragma unroll
          for (int t = 0; t < kQk; ++t) {
            if (t + 3 < kQk) ka[(t + 3) % 4] = kfrag(t + 3);
            mma_k16(s[is], ka[t % 4], qf[t]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // keys past N exist only in the last, partial key block.  Element i of subtile is
        // is key 32is + 8(i/4) + 4hf + i%4: compared as a constant against nv - 4hf, so no
        // per-element key index stays live across the loop.
        if (nv < KT) {
          const int nvh = nv - 4 * hf;
  #pragma unroll
          for (int is = 0; is < kSub; ++is)
  #pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * is + 8 * (i >> 2) + (i & 3) >= nvh) s[is][i] = -INFINITY;
        }
        // row max of the raw scores (scale > 0 commutes with max), both lane halves
        float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // independent chains
  #pragma unroll
        for (int is = 0; is < kSub; ++is)
  #pragma unroll
          for (int i = 0; i < 16; i += 2) mc[(i >> 1) & 3] = max3(mc[(i >> 1) & 3], s[is][i], s[is][i + 1]);
        float mx = max3(mc[0], mc[1], max3(mc[2], mc[3], mc[3]));
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = max3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1]));
        }
        const float m_tile = mx * scale_log2;
        if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
          const float m_new = __builtin_fmaxf(m_run, m_tile);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          l_mma *= alpha;
  #pragma unroll
          for (int io = 0; io < kOut; ++io) acc[io] *= alpha;
        }
        // V^T fragment (io, u): rows of key group u (16 keys), columns 32io .. 32io+31
        auto vfrag = [&](int io, int u) {
          Frag<T> a;
          if constexpr (kBf16) {
            // transpose reads: lane s of 16-lane group g supplies row kbase + s/4, columns
            // dbase + 4*(s%4) .. +3; lane i of the group receives column dbase + i of rows
            // kbase .. kbase+3, i.e. V^T[d][4 consecutive keys].
            const int g = lane >> 4, sl = lane & 15;
            const int dcol = 32 * io + 16 * (g & 1) + 4 * (sl & 3);
            short4_t part[2];
  #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const int kr = 16 * u + 8 * tt + 4 * (g >> 1) + (sl >> 2);
              const int gran = (dcol >> 3) ^ swz<GPR>(kr);
              const uint16_t* p = vt + kr * D + gran * 8 + (dcol & 7);
              part[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) short4_t*)(p));
            }
            const uint2 lo = __builtin_bit_cast(uint2, part[0]);
            const uint2 hi = __builtin_bit_cast(uint2, part[1]);
            a.v = make_uint4(lo.x, lo.y, hi.x, hi.y);
          } else {
            const int d = 32 * io + qn;
            float av[8];
  #pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int kr = 16 * u + 8 * (jj >> 2) + 4 * hf + (jj & 3);
              av[jj] = vt[(kr * GPR + ((d / G) ^ swz<GPR>(kr))) * G + (d % G)];
            }
            a.a = make_float4(av[0], av[1], av[2], av[3]);
            a.b = make_float4(av[4], av[5], av[6], av[7]);
          }
          return a;
        };
        const float neg_m = -m_run;
        Frag<T> pf[kPv];
        // P^T in bf16, two weights per word, and the row sum of the rounded weights
        auto p_word = [&](int u, int j) {
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u >> 1][8 * (u & 1) + 2 * j], scale_log2, neg_m));
          const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u >> 1][8 * (u & 1) + 2 * j + 1], scale_log2, neg_m));
          const bf16x2_t pk = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
          return __builtin_bit_cast(uint32_t, pk);
        };
        constexpr int kPairs = kOut * kPv;
        if constexpr (kBf16 && D == 64) {
          // O^T += V^T P^T with key group u outer: the weights of group u+1 are formed beside
          // the products of group u (kOut products, 4/kOut words after each).  At d = 64 the
          // step is bound by the vector work and this overlap inside the wavefront pays
          // (CogVideoX-shaped layer -1.9 %); at d = 128 the three wavefronts of a SIMD
          // already overlap it, and the plain order below is 0.5 % faster.  The V^T
          // fragment of product p+2 is read before product p; the order is fixed with
          // scheduling fences.  Every accumulator still adds its groups in order.
          constexpr int kWords = 4 / kOut;
          static_assert(kWords * kOut == 4, "whole words per product");
          uint32_t wd[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) wd[j] = p_word(0, j);
          pf[0].v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          psum(pf[0].v);
          Frag<T> va[3];
          va[0] = vfrag(0, 0);
          va[1] = vfrag(1 % kOut, 1 / kOut);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int pp = 0; pp < kPairs; ++pp) {
            const int io = pp % kOut, u = pp / kOut;
            if (pp + 2 < kPairs) va[(pp + 2) % 3] = vfrag((pp + 2) % kOut, (pp + 2) / kOut);
            __builtin_amdgcn_sched_barrier(0);
            mma_k16(acc[io], va[pp % 3], pf[u]);
            if (u + 1 < kPv) {
  #pragma unroll
              for (int j = 0; j < kWords; ++j) wd[kWords * io + j] = p_word(u + 1, kWords * io + j);
              if (io == kOut - 1) {
                pf[u + 1].v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                psum(pf[u + 1].v);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
  #pragma unroll
          for (int u = 0; u < kPv; ++u) {
            if constexpr (kBf16) {
              uint32_t wd[4];
  #pragma unroll
              for (int j = 0; j < 4; ++j) wd[j] = p_word(u, j);
              pf[u].v = make_uint4(wd[0], wd[1], wd[2], wd[3]);
              psum(pf[u].v);
            } else {
              float pv[8];
  #pragma unroll
              for (int j = 0; j < 8; ++j)
                pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u >> 1][8 * (u & 1) + j], scale_log2, neg_m));
  #pragma unroll
              for (int j = 0; j < 8; ++j) l_run += pv[j];
              pf[u].a = make_float4(pv[0], pv[1], pv[2], pv[3]);
              pf[u].b = make_float4(pv[4], pv[5], pv[6], pv[7]);
            }
          }
          // O^T += V^T P^T; the V^T fragment of pair p+2 is read before the product of pair
          // p, in an order fixed with scheduling fences (left to itself the scheduler puts
          // each read right before its product and waits for it there)
          Frag<T> va[3];
          va[0] = vfrag(0, 0);
          va[1] = vfrag(1 / kPv, 1 % kPv);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int pp = 0; pp < kPairs; ++pp) {
            if (pp + 2 < kPairs) va[(pp + 2) % 3] = vfrag((pp + 2) / kPv, (pp + 2) % kPv);
            __builtin_amdgcn_sched_barrier(0);
            mma_k16(acc[pp / kPv], va[pp % 3], pf[pp % kPv]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      if (!more) return false;
      e = e_n;
      hh = hh_n;
      c = c_n;
      nkv = nkv_n;
      return true;
    };
    for (;;) {
      if (!step(std::integral_constant<int, 0>{})) break;
      if (!step(std::integral_constant<int, 1>{})) break;
    }
  }

  // epilogue: O = acc / l   (zero for empty rows and skipped heads)
  float l_tot;
  {
    const float l_lane = kBf16 ? l_mma[0] : l_run;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (kSplit && n_chunks > 1) {
    // one chunk of a split row: the unnormalised accumulator and (running max, sum) per
    // query, merged into O by the combine kernel
    if (qi < N) {
      const size_t prow = ((size_t)chunk * total_rows + row) * BLK + (w * 32 + qn);
      float* po = meta.part_o + prow * D;
#pragma unroll
      for (int io = 0; io < kOut; ++io)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(po + 32 * io + 8 * g + 4 * hf) =
              make_float4(acc[io][4 * g + 0], acc[io][4 * g + 1], acc[io][4 * g + 2], acc[io][4 * g + 3]);
      if (hf == 0) reinterpret_cast<float2*>(meta.part_ml)[prow] = make_float2(m_run, l_tot);
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // log of the softmax normaliser, natural units: the running max is in log2 units of the
  // scaled scores, l sums 2^(s*scale*log2e - max); -inf for an empty row
  if (meta.lse && hf == 0 && qi < N)
    meta.lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  if (qi < N) {
    TO* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int io = 0; io < kOut; ++io) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * io + 8 * g + 4 * hf;
        const float o0 = acc[io][4 * g + 0] * inv, o1 = acc[io][4 * g + 1] * inv;
        const float o2 = acc[io][4 * g + 2] * inv, o3 = acc[io][4 * g + 3] * inv;
        if constexpr (sizeof(TO) == 4) {
          *reinterpret_cast<float4*>(orow + d0) = make_float4(o0, o1, o2, o3);
        } else {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
          *reinterpret_cast<uint2*>(orow + d0) = make_uint2(lo, hi);
        }
      }
    }
  }
}

// Merge the chunks of every split row: O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c with
// M the largest chunk max; lse from M and the merged sum.  Rows that were not split were
// finished by the attention kernel and are left alone.  One workgroup per 32 queries of a
// row (grid = rows * blk / 32).
constexpr int kCombineQ = 32;
template <typename TO>
__global__ __launch_bounds__(256) void split_combine_kernel(AttnArgs a, int total_rows) {
  const int qs = a.blk / kCombineQ;
  const int row = blockIdx.x / qs, q0 = (blockIdx.x - row * qs) * kCombineQ;
  const int bh = row / a.Nb, r = row - bh * a.Nb, h = bh % a.H;
  int cnt = a.row_ptr[row + 1] - a.row_ptr[row];
  if ((a.skip_bits[h >> 5] >> (h & 31)) & 1u) cnt = 0;
  if (cnt <= a.split_blocks) return;
  const int n = (cnt + a.split_blocks - 1) / a.split_blocks;
  const int blk = a.blk, D = a.d, C4 = D / 4;
  const int nq = min(blk, a.N - r * blk);
  if (q0 >= nq) return;
  const int qn = min(kCombineQ, nq - q0);
  const float4* po = reinterpret_cast<const float4*>(a.part_o);
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml);
  TO* O = static_cast<TO*>(a.o);
  for (int idx = threadIdx.x; idx < qn * C4; idx += 256) {
    const int q = q0 + idx / C4, c4 = idx % C4;
    float M = -INFINITY;
    for (int c = 0; c < n; ++c) M = fmaxf(M, pml[((size_t)c * total_rows + row) * blk + q].x);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
      for (int c = 0; c < n; ++c) {
        const size_t pr = ((size_t)c * total_rows + row) * blk + q;
        const float2 ml = pml[pr];
        if (ml.x == -INFINITY) continue;
        const float wgt = __builtin_amdgcn_exp2f(ml.x - M);
        const float4 v = po[pr * C4 + c4];
        L = __builtin_fmaf(wgt, ml.y, L);
        o.x = __builtin_fmaf(wgt, v.x, o.x);
        o.y = __builtin_fmaf(wgt, v.y, o.y);
        o.z = __builtin_fmaf(wgt, v.z, o.z);
        o.w = __builtin_fmaf(wgt, v.w, o.w);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t qg = (size_t)bh * a.N + (size_t)r * blk + q;
    TO* orow = O + qg * D + 4 * c4;
    if constexpr (sizeof(TO) == 4) {
      *reinterpret_cast<float4*>(orow) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(o.x * inv) | ((uint32_t)f32_to_bf16_rne(o.y * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(o.z * inv) | ((uint32_t)f32_to_bf16_rne(o.w * inv) << 16);
      *reinterpret_cast<uint2*>(orow) = make_uint2(lo, hi);
    }
    if (c4 == 0 && a.lse) a.lse[qg] = (M + __log2f(L)) * 0.69314718055994531f;
  }
}

// Rows from which a d = 128, 128-query-block launch takes 32-key steps: three workgroups
// per compute unit.  The split path follows the same rule, so rows it leaves whole match
// the plain kernel bit for bit.
constexpr int kShortStepRows = 768;

template <typename T, typename TO, int D, int BLK, int KT>
hipError_t launch_kt(const AttnArgs& a, hipStream_t s) {
  const int total = a.B * a.H * a.Nb;
  if (a.split_blocks > 0) {
    // 8 equal shares of (rows of the XCD's range) x (chunks per row)
    const long long items = (long long)kXcds * ((total + kXcds - 1) / kXcds) * a.split_max;
    hipLaunchKernelGGL((attn_fwd_kernel<T, TO, D, BLK, KT, true>), dim3((unsigned)items), dim3(BLK * 2), 0, s,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<TO*>(a.o), a.row_ptr, a.col_idx, a.H, a.N, a.Nb, total, a.scale_log2, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<T, TO, D, BLK, KT, false>), dim3((unsigned)total), dim3(BLK * 2), 0, s,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<TO*>(a.o), a.row_ptr, a.col_idx, a.H, a.N, a.Nb, total, a.scale_log2, a);
  }
  return hipGetLastError();
}

template <typename T, typename TO, int D, int BLK>
hipError_t launch_typed(const AttnArgs& a, hipStream_t s) {
  if constexpr (D == 128 && BLK == 128) {
    if ((long long)a.B * a.H * a.Nb >= kShortStepRows) return launch_kt<T, TO, D, BLK, 32>(a, s);
  }
  // d = 128 with 64-query blocks: two wavefronts per workgroup, so a 64-key step costs each
  // thread twice the transfers of a 128-block launch and more registers than two wavefronts
  // per SIMD leave.  32-key steps fit two wavefronts without spills; LDS (32 KB per
  // two-wavefront workgroup) holds five workgroups per compute unit, so a three-wavefront
  // register target would only add spills.
  if constexpr (D == 128 && BLK == 64) return launch_kt<T, TO, D, BLK, 32>(a, s);
  return launch_kt<T, TO, D, BLK, 64>(a, s);
}

template <typename T, typename TO>
hipError_t launch_shape(const AttnArgs& a, hipStream_t s) {
  if (a.d == 128 && a.blk == 128) return launch_typed<T, TO, 128, 128>(a, s);
  if (a.d == 128 && a.blk == 64) return launch_typed<T, TO, 128, 64>(a, s);
  if (a.d == 64 && a.blk == 128) return launch_typed<T, TO, 64, 128>(a, s);
  return launch_typed<T, TO, 64, 64>(a, s);
}

}  // namespace

hipError_t launch_split_combine(const AttnArgs& a, hipStream_t s) {
  const int total = a.B * a.H * a.Nb;
  const dim3 grid((unsigned)(total * (a.blk / kCombineQ)));
  if (a.out_bf16)
    hipLaunchKernelGGL(split_combine_kernel<uint16_t>, grid, dim3(256), 0, s, a, total);
  else
    hipLaunchKernelGGL(split_combine_kernel<float>, grid, dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.in_bf16) {
    return a.out_bf16 ? launch_shape<uint16_t, uint16_t>(a, s) : launch_shape<uint16_t, float>(a, s);
  }
  return a.out_bf16 ? launch_shape<float, uint16_t>(a, s) : launch_shape<float, float>(a, s);
}

}  // namespace asa
