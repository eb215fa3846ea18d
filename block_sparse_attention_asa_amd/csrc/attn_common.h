// Device helpers shared by the attention kernels (forward and backward) for gfx950:
// MFMA operand fragments, the LDS tile swizzle, global -> LDS transfers, barriers and
// the XCD-aware row mapping.  Included by the .hip sources only.
//
// MFMA 32x32 output layout used throughout: lane l, accumulator register i holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "asa_internal.h"

namespace asa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

// max(a, b, c) in one instruction.  Written out because fmaxf on MFMA results makes the
// compiler quiet each input first (the scores here are never NaN).
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Round to bf16 (round to nearest even) and return both the bits and the rounded value.
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  const __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// LDS tile layout (K and V alike): row-major [keys][D], no padding, 16-byte granules
// XOR-swizzled per row: physical granule = logical granule ^ swz(row).  gfx950 LDS serves
// 256 bytes (64 banks) per cycle: 16 lanes of a 16-byte read or 32 lanes of an 8-byte read.
// For rows of >= 16 granules, swz(r) = 4*(r%4) + (r/4)%4 is distinct over any 16
// consecutive rows (conflict-free K-fragment reads: 16 lanes, 16 rows, one logical
// granule) and, inside every aligned 4-row group, changes only bits 2-3 (conflict-free
// transpose reads: 32 lanes covering 4 rows x 4 adjacent granules).  Rows of 8 granules
// (bf16, d = 64) use a 3-bit variant.
template <int GPR>
__device__ inline int swz(int row) {
  if constexpr (GPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Workgroup id -> row, keeping consecutive rows (same head) on one XCD: dispatch assigns
// workgroup ids round-robin over the 8 XCDs, so XCD x receives ids x, x+8, ...
__device__ inline int xcd_row(int wg, int total) {
  int lo, hi;
  xcd_range(wg % kXcds, total, lo, hi);
  return lo + wg / kXcds;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kGran = 8; };   // elements per 16 B
template <> struct Elem<float> { static constexpr int kGran = 4; };

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without a memory fence: the caller has already waited for whatever
// must be visible (vmcnt for LDS DMA, lgkmcnt for its own LDS traffic).  A fenced
// __syncthreads() would also wait for LDS DMA still in flight for the next tile.
__device__ inline void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short short4_t __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4): lane L reads
// 16 bytes at gbase + voff and they land at LDS byte address lds_base + kLdsOff + 16 * L.
// Written as an asm block so that the compiler's wait insertion does not serialize it
// against unrelated LDS reads; the instruction has no register results, and every reader
// of the destination waits on vmcnt and a barrier first.  The block may only touch M0 (the
// LDS base; one wait state after writing it), which the compiler does not use in these
// kernels: s_mov_b32 leaves SCC alone, unlike an s_add into M0 would.
template <int kLdsOff>
__device__ inline void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  const uint64_t g = reinterpret_cast<uint64_t>(gbase);
  // readfirstlane returns int: go through uint32_t so the low half is zero-extended
  const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(g >> 32));
  const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)g);
  const uint64_t gu = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
  const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds_base + (uint32_t)kLdsOff));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(m0v), "v"(voff), "s"(gu)
      : "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. n-1.
template <int I, int N_, typename F>
__device__ inline void static_for_impl(F&& f) {
  if constexpr (I < N_) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N_>(f);
  }
}
template <int N_, typename F>
__device__ inline void static_for(F&& f) { static_for_impl<0, N_>(f); }

// Per-thread byte offsets (within one key step of KT rows) of the 16-byte granules this
// thread transfers: instruction `it` of wave w fills LDS granule slots it*NT + 64*w + lane,
// which hold logical granule (slot % GPR) ^ swz(row) of row slot / GPR.  Rows at or past
// nkv re-read row nkv-1 (finite data that the softmax masks out).
template <typename T, int D, int NT>
__device__ inline uint32_t dma_offset(int it, int tid, int nkv) {
  constexpr int GPR = D * (int)sizeof(T) / 16;
  const int slot = it * NT + tid;
  const int row = slot / GPR, pg = slot - row * GPR;
  const int srow = min(row, nkv - 1);
  return (uint32_t)((srow * GPR + (pg ^ swz<GPR>(row))) * 16);
}

}  // namespace
}  // namespace asa
