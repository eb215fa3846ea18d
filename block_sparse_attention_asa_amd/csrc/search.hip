// Per-head pattern search (Sparse-vDiT, section 三: the offline search loss
// L_i = MSE(O_i - O_0) + lambda (1 - S_i) and the pattern-selection formula).
//
// The attention outputs themselves come from the forward kernel.  This file holds the two
// reductions that turn them into a choice:
//   sq_err_kernel   one workgroup per CSR row (b, h, query block r): the float64 sum of
//                   (O_i - O_0)^2 over the row's n_r x d outputs, and the number of
//                   (query, key) token pairs its kept tiles hold.  HBM-bound: it streams
//                   two fp32 outputs once.
//   choose_kernel   one workgroup per head: sums the row partials of every candidate in a
//                   fixed order (deterministic), forms MSE, S_i and L_i, and picks full
//                   attention when every L_i > eps, else the smallest L_i (first on ties).
#include <hip/hip_runtime.h>

#include "asa_internal.h"

namespace asa {
namespace {

constexpr int kRedThreads = 256;
constexpr int kRedWaves = kRedThreads / 64;

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Workgroup sum in a fixed order: lanes by butterfly, then the four waves in index order.
template <typename T>
__device__ inline T group_sum(T v, T* lds) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  T t = lds[0];
#pragma unroll
  for (int w = 1; w < kRedWaves; ++w) t += lds[w];
  __syncthreads();
  return t;
}

__device__ inline double sq4(const float4& x, const float4& y) {
  const double a = (double)x.x - (double)y.x, b = (double)x.y - (double)y.y;
  const double c = (double)x.z - (double)y.z, e = (double)x.w - (double)y.w;
  return a * a + b * b + c * c + e * e;
}

__global__ __launch_bounds__(kRedThreads) void sq_err_kernel(
    const float* __restrict__ o0, const float* __restrict__ oi, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int N, int d, int blk, int Nb, double* __restrict__ sq,
    long long* __restrict__ pairs) {
  __shared__ double red_d[kRedWaves];
  __shared__ long long red_l[kRedWaves];
  const int row = blockIdx.x;
  const int r = row % Nb;
  const int bh = row / Nb;
  const int lo = r * blk;
  const int nr = min(blk, N - lo);
  const size_t base = ((size_t)bh * N + lo) * (size_t)d;
  const int n4 = nr * d / 4;                     // d is 64 or 128: whole float4s, 256 B aligned
  const float4* a = reinterpret_cast<const float4*>(o0 + base);
  double acc = 0.0;
  if (oi) {
    const float4* b = reinterpret_cast<const float4*>(oi + base);
    constexpr int kU = 4;                        // loads in flight per thread
    for (int i0 = threadIdx.x; i0 < n4; i0 += kU * kRedThreads) {
      float4 x[kU], y[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = i0 + u * kRedThreads;
        if (i < n4) { x[u] = a[i]; y[u] = b[i]; }
        else { x[u] = make_float4(0.f, 0.f, 0.f, 0.f); y[u] = x[u]; }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) acc += sq4(x[u], y[u]);
    }
  } else {                                       // the candidate's output is zero (skip)
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int kU = 8;
    for (int i0 = threadIdx.x; i0 < n4; i0 += kU * kRedThreads) {
      float4 x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = i0 + u * kRedThreads;
        x[u] = i < n4 ? a[i] : z;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) acc += sq4(x[u], z);
    }
  }
  long long keys = 0;                            // key tokens of the row's kept tiles
  const int c0 = row_ptr[row], c1 = row_ptr[row + 1];
  for (int j = c0 + threadIdx.x; j < c1; j += kRedThreads) {
    const int c = col_idx[j];
    keys += min(blk, N - c * blk);
  }
  acc = group_sum(acc, red_d);
  keys = group_sum(keys, red_l);
  if (threadIdx.x == 0) {
    sq[row] = acc;
    pairs[row] = (long long)nr * keys;
  }
}

__global__ __launch_bounds__(kRedThreads) void choose_kernel(
    const double* __restrict__ sq, const long long* __restrict__ pairs, int B, int H, int Nb,
    int n_cand, double elems, double all_pairs, double lam, double eps, double* __restrict__ loss,
    double* __restrict__ mse, int32_t* __restrict__ choice) {
  __shared__ double red_d[kRedWaves];
  __shared__ long long red_l[kRedWaves];
  const int h = blockIdx.x;
  const int per_head = B * Nb;
  const size_t rows = (size_t)B * H * Nb;
  double best = 0.0;
  int best_i = -1;
  bool all_above = true;
  for (int i = 0; i < n_cand; ++i) {
    double acc = 0.0;
    long long pc = 0;
    for (int j = threadIdx.x; j < per_head; j += kRedThreads) {
      const int b = j / Nb, r = j - b * Nb;
      const size_t row = i * rows + ((size_t)b * H + h) * Nb + r;
      acc += sq[row];
      pc += pairs[row];
    }
    acc = group_sum(acc, red_d);
    pc = group_sum(pc, red_l);
    // MSE over the head's B*N*d outputs; kept fraction 1 - S_i = kept token pairs / (B N^2)
    const double m = acc / elems;
    const double L = m + lam * ((double)pc / all_pairs);
    if (threadIdx.x == 0) {
      loss[(size_t)h * n_cand + i] = L;
      if (mse) mse[(size_t)h * n_cand + i] = m;
    }
    all_above = all_above && (L > eps);
    if (best_i < 0 || L < best) { best = L; best_i = i; }
  }
  if (threadIdx.x == 0) choice[h] = (n_cand == 0 || all_above) ? 0 : best_i + 1;
}

}  // namespace

hipError_t launch_search_sq_err(const float* o0, const float* oi, const int32_t* row_ptr,
                                const int32_t* col_idx, int B, int H, int N, int d, int blk, int Nb,
                                double* sq, long long* pairs, hipStream_t s) {
  const int rows = B * H * Nb;
  hipLaunchKernelGGL(sq_err_kernel, dim3((unsigned)rows), dim3(kRedThreads), 0, s, o0, oi, row_ptr,
                     col_idx, N, d, blk, Nb, sq, pairs);
  return hipGetLastError();
}

hipError_t launch_search_choose(const double* sq, const long long* pairs, int B, int H, int N, int d,
                                int Nb, int n_cand, double lam, double eps, double* loss, double* mse,
                                int32_t* choice, hipStream_t s) {
  const double elems = (double)B * N * d;
  const double all_pairs = (double)B * N * (double)N;
  hipLaunchKernelGGL(choose_kernel, dim3((unsigned)H), dim3(kRedThreads), 0, s, sq, pairs, B, H, Nb,
                     n_cand, elems, all_pairs, lam, eps, loss, mse, choice);
  return hipGetLastError();
}

}  // namespace asa
