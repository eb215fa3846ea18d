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
// owning 32 query rows.  For every kept key block the workgroup stages K (row-major) and
// V (transposed, key-permuted) in LDS, then each wavefront computes
//     S^T = K_c Q^T          (32x32x16 bf16 MFMA, or 32x32x2 f32 MFMA for fp32 inputs)
//     online softmax          (exp2 with the scale folded in, running max / sum per row)
//     O^T += V_c^T P^T        (same MFMA shape)
// Computing the transposed products makes every lane own one query row: the S^T
// accumulator layout puts 16 keys of query (lane % 32) in each lane, and the O^T layout
// puts 16 output columns of the same query there, so the softmax statistics and the
// rescale stay lane-local (one cross-half exchange per tile for the row max).
//
// MFMA 32x32 output layout used throughout: lane l, accumulator register i holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.
#include <hip/hip_runtime.h>

#include "asa_internal.h"

namespace asa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Eight consecutive operand elements along the contraction (k) axis of one lane.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {   // bf16 bits
  uint4 v;
};
template <> struct Frag<float> {
  float4 a, b;
};

__device__ inline Frag<uint16_t> lds_frag(const uint16_t* p) {
  Frag<uint16_t> f;
  f.v = *reinterpret_cast<const uint4*>(p);
  return f;
}
__device__ inline Frag<float> lds_frag(const float* p) {
  Frag<float> f;
  f.a = *reinterpret_cast<const float4*>(p);
  f.b = *reinterpret_cast<const float4*>(p + 4);
  return f;
}

// acc += A * B over one 16-wide k-step.  Lane half hf supplies k = 8*hf + j (j = 0..7)
// for both operands, so any k permutation applied identically to A and B cancels.
__device__ inline void mma_k16(f32x16_t& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ inline void mma_k16(f32x16_t& acc, const Frag<float>& a, const Frag<float>& b) {
  const float av[8] = {a.a.x, a.a.y, a.a.z, a.a.w, a.b.x, a.b.y, a.b.z, a.b.w};
  const float bv[8] = {b.a.x, b.a.y, b.a.z, b.a.w, b.b.x, b.b.y, b.b.z, b.b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
}

// Round to bf16 (round to nearest even) and return both the bits and the rounded value.
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  const __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Position of key kk inside a transposed V row: bits 2 and 3 of the index are swapped so
// that the 8 keys a lane half feeds to one PV k-step are contiguous (16 bytes for bf16).
__device__ inline int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// Workgroup id -> row, keeping consecutive rows (same head) on one XCD: dispatch assigns
// workgroup ids round-robin over the 8 XCDs, so XCD x receives ids x, x+8, ...
__device__ inline int xcd_row(int wg, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int x = wg % kXcd, local = wg / kXcd;
  return x * per + min(x, rem) + local;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kGran = 8; };   // elements per 16 B
template <> struct Elem<float> { static constexpr int kGran = 4; };

template <typename T, typename TO, int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_fwd_kernel(const T* __restrict__ Q,
                                                           const T* __restrict__ K,
                                                           const T* __restrict__ V,
                                                           TO* __restrict__ O,
                                                           const int32_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ col_idx,
                                                           int H, int N, int Nb, int total_rows,
                                                           float scale_log2, AttnArgs meta) {
  constexpr int kWaves = BLK / 32;
  constexpr int kThreadsWg = 64 * kWaves;
  constexpr int G = Elem<T>::kGran;
  constexpr int KSTR = D + G;      // K row stride (elements): 16 bytes of padding
  constexpr int VSTR = BLK + G;    // transposed-V row stride (elements)
  constexpr int kQk = D / 16;      // k-steps of S^T = K Q^T
  constexpr int kSub = BLK / 32;   // 32-key subtiles per key block
  constexpr int kPv = BLK / 16;    // k-steps of O^T = V^T P^T
  constexpr int kOut = D / 32;     // 32-column output subtiles
  constexpr bool kBf16 = sizeof(T) == 2;

  __shared__ __attribute__((aligned(16))) T Ks[BLK * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

  const int row = xcd_row(blockIdx.x, total_rows);
  const int bh = row / Nb, r = row - bh * Nb, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qn = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const int qi = r * BLK + w * 32 + qn;

  int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  if ((meta.skip_bits[h >> 5] >> (h & 31)) & 1u) e1 = e0;

  f32x16_t acc[kOut];
#pragma unroll
  for (int io = 0; io < kOut; ++io) acc[io] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

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

    for (int e = e0; e < e1; ++e) {
      const int c = col_idx[e];
      const int kv0 = c * BLK;
      const int nkv = min(BLK, N - kv0);
      __syncthreads();   // previous tile fully consumed
      // K tile, row-major with padding
      for (int i = tid; i < BLK * (D / G); i += kThreadsWg) {
        const int kr = i / (D / G), gc = i - kr * (D / G);
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (kr < nkv) val = *reinterpret_cast<const uint4*>(K + head + (size_t)(kv0 + kr) * D + gc * G);
        *reinterpret_cast<uint4*>(Ks + kr * KSTR + gc * G) = val;
      }
      // V tile, transposed: item = (4-key group a, 8-column group g)
      for (int i = tid; i < (BLK / 4) * (D / 8); i += kThreadsWg) {
        const int a = i / (D / 8), g = i - a * (D / 8);
        T vv[4][8];
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int kr = 4 * a + e4;
#pragma unroll
          for (int hh = 0; hh < 8 / G; ++hh) {
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (kr < nkv) val = *reinterpret_cast<const uint4*>(V + head + (size_t)(kv0 + kr) * D + 8 * g + hh * G);
            *reinterpret_cast<uint4*>(&vv[e4][hh * G]) = val;
          }
        }
        const int pos = vt_pos(4 * a);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          T* dst = Vt + (8 * g + jj) * VSTR + pos;
          if (kBf16) {
            const uint32_t lo = (uint32_t)(uint16_t)vv[0][jj] | ((uint32_t)(uint16_t)vv[1][jj] << 16);
            const uint32_t hi = (uint32_t)(uint16_t)vv[2][jj] | ((uint32_t)(uint16_t)vv[3][jj] << 16);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<float4*>(dst) =
                make_float4((float)vv[0][jj], (float)vv[1][jj], (float)vv[2][jj], (float)vv[3][jj]);
          }
        }
      }
      __syncthreads();

      // S^T = K Q^T
      f32x16_t s[kSub];
#pragma unroll
      for (int is = 0; is < kSub; ++is) {
        s[is] = f32x16_t{};
#pragma unroll
        for (int t = 0; t < kQk; ++t)
          mma_k16(s[is], lds_frag(Ks + (32 * is + qn) * KSTR + 16 * t + 8 * hf), qf[t]);
      }
      // scale (log2 domain), mask keys past N, row max
      float mx = -INFINITY;
#pragma unroll
      for (int is = 0; is < kSub; ++is) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 32 * is + 8 * (i >> 2) + 4 * hf + (i & 3);
          float v = s[is][i] * scale_log2;
          if (kk >= nkv) v = -INFINITY;
          s[is][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f;
      Frag<T> pf[kPv];
#pragma unroll
      for (int u = 0; u < kPv; ++u) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(s[u >> 1][8 * (u & 1) + j] - m_new);
        if constexpr (kBf16) {
          uint16_t b[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            b[j] = f32_to_bf16_rne(pv[j]);
            lsum += bf16_bits_to_f32(b[j]);
          }
          pf[u].v = make_uint4((uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16),
                               (uint32_t)b[4] | ((uint32_t)b[5] << 16), (uint32_t)b[6] | ((uint32_t)b[7] << 16));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) lsum += pv[j];
          pf[u].a = make_float4(pv[0], pv[1], pv[2], pv[3]);
          pf[u].b = make_float4(pv[4], pv[5], pv[6], pv[7]);
        }
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int io = 0; io < kOut; ++io) acc[io] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int io = 0; io < kOut; ++io) {
#pragma unroll
        for (int u = 0; u < kPv; ++u)
          mma_k16(acc[io], lds_frag(Vt + (32 * io + qn) * VSTR + 16 * u + 8 * hf), pf[u]);
      }
    }
  }

  // epilogue: O = acc / l   (zero for empty rows and skipped heads)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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

template <typename T, typename TO, int D, int BLK>
hipError_t launch_typed(const AttnArgs& a, hipStream_t s) {
  const int total = a.B * a.H * a.Nb;
  hipLaunchKernelGGL((attn_fwd_kernel<T, TO, D, BLK>), dim3((unsigned)total), dim3(BLK * 2), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<TO*>(a.o), a.row_ptr, a.col_idx, a.H, a.N, a.Nb, total, a.scale_log2, a);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_shape(const AttnArgs& a, hipStream_t s) {
  if (a.d == 128 && a.blk == 128) return launch_typed<T, TO, 128, 128>(a, s);
  if (a.d == 128 && a.blk == 64) return launch_typed<T, TO, 128, 64>(a, s);
  if (a.d == 64 && a.blk == 128) return launch_typed<T, TO, 64, 128>(a, s);
  return launch_typed<T, TO, 64, 64>(a, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.in_bf16) {
    return a.out_bf16 ? launch_shape<uint16_t, uint16_t>(a, s) : launch_shape<uint16_t, float>(a, s);
  }
  return a.out_bf16 ? launch_shape<float, uint16_t>(a, s) : launch_shape<float, float>(a, s);
}

}  // namespace asa
