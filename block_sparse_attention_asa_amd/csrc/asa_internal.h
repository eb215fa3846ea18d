// Internal launch interface between the C ABI host layer and the gfx950 kernels.
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace asa {

constexpr int kMaxHeads = 256;       // per-head pattern table travels as a kernel argument
constexpr int kMaxMaskBlocks = 1024; // row bitmask (32 words) and LDS sort width
constexpr int kXcds = 8;             // accelerator complex dies sharing one dispatcher

// Rows [lo, hi) of the `total` CSR rows form the contiguous range processed on XCD x.
// Dispatch hands workgroup ids to the XCDs round-robin; the attention kernel maps the ids
// an XCD receives onto its range, and the mask builders order rows inside each range.
__host__ __device__ inline void xcd_range(int x, int total, int& lo, int& hi) {
  const int per = total / kXcds, rem = total % kXcds;
  lo = x * per + (x < rem ? x : rem);
  hi = lo + per + (x < rem ? 1 : 0);
}

// Skipped heads as a bitmask, passed by value.
struct SkipBits {
  uint32_t bits[kMaxHeads / 32];
};

// Per-head pattern table passed by value (2 KiB of kernel arguments).
struct HeadTable {
  int32_t id[kMaxHeads];
  int32_t param[kMaxHeads];
};

struct MaskGeom {
  int32_t B, H, N, d, blk, Nb, words;  // words = ceil(Nb / 32) bitmask words per row
};

struct AdaptiveParams {
  int32_t mode, k, k_cap, n_text_blocks, keep_diag;
  double tau;
};

// Workspace carve-up for the mask builders (all offsets 256-byte aligned).
struct MaskWorkspace {
  double* qp;      // [B*H*Nb*d]  pooled queries, row-major
  double* kpt;     // [B*H*d*Nb]  pooled keys, transposed per head
  uint32_t* bits;  // [B*H*Nb*words] kept-block bitmask per row
  int32_t* count;  // [B*H*Nb] kept blocks per row
};

size_t mask_workspace_layout(const MaskGeom& g, bool adaptive, MaskWorkspace* ws, void* base);

// Device scratch of asa_build_mask_noalloc: a static device array of this many bytes on
// every GPU the library runs on.  noalloc_scratch returns its address on the current
// device (looked up once per device, then cached).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// Mask pipeline stages (enqueue only; return the launch status).
hipError_t launch_pool(const void* q, const void* k, bool bf16, const MaskGeom& g,
                       const MaskWorkspace& ws, hipStream_t s);
hipError_t launch_rank(const MaskGeom& g, const AdaptiveParams& p, const HeadTable& heads,
                       const MaskWorkspace& ws, hipStream_t s);
hipError_t launch_static_rows(const MaskGeom& g, const HeadTable& heads, const MaskWorkspace& ws,
                              hipStream_t s);
hipError_t launch_csr(const MaskGeom& g, const MaskWorkspace& ws, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* order, hipStream_t s);

// Attention forward.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* order;  // processing order of the rows, or NULL for row order
  float* lse;            // [B,H,N] log of each query's softmax normaliser, or NULL
  int32_t B, H, N, d, blk, Nb;
  bool in_bf16, out_bf16;
  float scale_log2;      // softmax scale times log2(e)
  uint32_t skip_bits[kMaxHeads / 32];   // heads whose output is zero
  // Split rows (0 = off): a row keeping more than split_blocks key blocks is cut into
  // ceil(count / split_blocks) chunks of near-equal length, one workgroup each.  Chunks
  // write unnormalised partials; launch_split_combine merges them into O (and lse).
  int32_t split_blocks;
  int32_t split_max;     // chunks per row at most: ceil(Nb / split_blocks)
  float* part_o;         // [split_max][B*H*Nb][blk][d] fp32 partial O (unnormalised)
  float* part_ml;        // [split_max][B*H*Nb][blk][2] running max (log2 units) and sum
};

constexpr int kMaxSplit = 64;   // chunks per row at most

hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_split_combine(const AttnArgs& a, hipStream_t s);

// Attention backward (bf16 inputs, fp32 gradients).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;        // [B,H,N] natural-log softmax normaliser from the forward
  float* dq;
  float* dk;
  float* dv;
  const int32_t* row_ptr;  // CSR mask
  const int32_t* col_idx;
  int32_t* col_ptr;        // transposed mask (workspace): [B*H*Nb + 1]
  int32_t* row_idx;        // [B*H*Nb*Nb] capacity, query blocks ascending per key block
  int32_t* col_order;      // [B*H*Nb] key-block processing order (workspace)
  const int32_t* order;    // [B*H*Nb] row processing order from the CSR, or NULL
  float* ld;               // [B*H*N][2] (lse * log2(e), D = dO . O) per query (workspace)
  int32_t B, H, N, d, blk, Nb;
  bool o_bf16;
  bool in_f32;             // Q, K, V, dO are fp32 (else bf16)
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e)
  uint32_t skip_bits[kMaxHeads / 32];
};

// Workspace carve-up for the backward; returns the bytes needed (base may be NULL).
size_t bwd_workspace_layout(const BwdArgs& geom, BwdArgs* a, void* base);
hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t s);

// Pattern search reductions.  sq_err: per CSR row, the float64 sum of (oi - o0)^2 over the
// row's outputs (oi NULL = zero output) and its kept token pairs.  choose: per head, the
// loss of each of n_cand candidates (partials laid out [n_cand][B*H*Nb]) and the choice.
constexpr int kMaxSearchCandidates = 8;
hipError_t launch_search_sq_err(const float* o0, const float* oi, const int32_t* row_ptr,
                                const int32_t* col_idx, int B, int H, int N, int d, int blk, int Nb,
                                double* sq, long long* pairs, hipStream_t s);
hipError_t launch_search_choose(const double* sq, const long long* pairs, int B, int H, int N, int d,
                                int Nb, int n_cand, double lam, double eps, double* loss, double* mse,
                                int32_t* choice, hipStream_t s);

}  // namespace asa
