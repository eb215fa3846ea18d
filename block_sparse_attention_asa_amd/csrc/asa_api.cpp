// C ABI entry points: host-side validation, workspace layout and kernel enqueueing.
// Every check runs before anything is enqueued; no HIP call is made for an invalid call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "asa.h"
#include "asa_internal.h"

static_assert(ASA_NOALLOC_SCRATCH_BYTES == asa::kNoAllocScratchBytes, "scratch size in asa.h and the library differ");

namespace {

thread_local char g_last_error[512] = "";

asa_status fail(asa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
asa_status fail(asa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

asa_status hip_fail(hipError_t e, const char* what) {
  return fail(ASA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t num_blocks(const asa_shape* s) { return ((int64_t)s->N + s->blk - 1) / s->blk; }

// Shape checks shared by every entry point.  need_mask: Nb must fit the mask kernels.
asa_status check_shape(const asa_shape* s, bool need_mask) {
  if (!s) return fail(ASA_ERR_NULL_ARG, "shape is NULL");
  if (s->B <= 0 || s->H <= 0 || s->N <= 0)
    return fail(ASA_ERR_BAD_SHAPE, "B=%d H=%d N=%d must be positive", s->B, s->H, s->N);
  if (s->in_dtype != ASA_F32 && s->in_dtype != ASA_BF16)
    return fail(ASA_ERR_BAD_DTYPE, "in_dtype=%d is not ASA_F32 or ASA_BF16", s->in_dtype);
  if (s->d != 64 && s->d != 128) return fail(ASA_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", s->d);
  if (s->blk != 64 && s->blk != 128)
    return fail(ASA_ERR_UNSUPPORTED, "blk=%d (supported: 64, 128)", s->blk);
  const int64_t Nb = num_blocks(s);
  const int64_t rows = (int64_t)s->B * s->H * Nb;
  if (s->H > asa::kMaxHeads)
    return fail(ASA_ERR_UNSUPPORTED, "H=%d exceeds the per-head table limit %d", s->H, asa::kMaxHeads);
  if ((int64_t)s->N * s->d >= ((int64_t)1 << 31))
    return fail(ASA_ERR_BAD_SHAPE, "N*d=%lld overflows int32 token offsets", (long long)s->N * s->d);
  if (rows >= ((int64_t)1 << 31) - 1) return fail(ASA_ERR_BAD_SHAPE, "B*H*Nb=%lld rows overflow int32", (long long)rows);
  if (need_mask) {
    if (Nb > asa::kMaxMaskBlocks)
      return fail(ASA_ERR_UNSUPPORTED, "Nb=%lld key blocks exceeds the mask builders' limit %d",
                  (long long)Nb, asa::kMaxMaskBlocks);
    if (rows * Nb >= ((int64_t)1 << 31) - 1)
      return fail(ASA_ERR_BAD_SHAPE, "B*H*Nb*Nb=%lld overflows int32 CSR offsets", (long long)(rows * Nb));
  }
  return ASA_OK;
}

asa_status fill_heads(const asa_shape* s, const asa_head_pattern* pats, bool allow_adaptive,
                      asa::HeadTable* t) {
  std::memset(t, 0, sizeof(*t));
  if (!pats) return ASA_OK;
  const int64_t Nb = num_blocks(s);
  for (int h = 0; h < s->H; ++h) {
    const int id = pats[h].id, prm = pats[h].param;
    switch (id) {
      case ASA_PAT_ADAPTIVE:
        if (!allow_adaptive) return fail(ASA_ERR_BAD_PATTERN, "head %d: ASA_PAT_ADAPTIVE in a static-only call", h);
        break;
      case ASA_PAT_FULL:
      case ASA_PAT_SKIP:
      case ASA_PAT_DIAG:
        break;
      case ASA_PAT_MULTIDIAG:
        if (prm <= 0) return fail(ASA_ERR_BAD_PATTERN, "head %d: multi-diagonal stride %d must be > 0", h, prm);
        break;
      case ASA_PAT_VSTRIPE:
        if (prm < 0) return fail(ASA_ERR_BAD_PATTERN, "head %d: vertical-stripe width %d must be >= 0", h, prm);
        break;
      case ASA_PAT_FRAME_TILE:
        if (prm <= 0) return fail(ASA_ERR_BAD_PATTERN, "head %d: frame-tile frame length %d must be > 0", h, prm);
        break;
      default:
        return fail(ASA_ERR_BAD_PATTERN, "head %d: unknown pattern id %d", h, id);
    }
    t->id[h] = id;
    t->param[h] = (id == ASA_PAT_VSTRIPE && prm > Nb) ? (int)Nb : prm;
  }
  return ASA_OK;
}

asa::MaskGeom geom_of(const asa_shape* s) {
  asa::MaskGeom g{};
  g.B = s->B; g.H = s->H; g.N = s->N; g.d = s->d; g.blk = s->blk;
  g.Nb = (int)num_blocks(s);
  g.words = (g.Nb + 31) / 32;
  return g;
}

asa_status check_csr_out(const asa_shape* s, const asa_csr* out) {
  if (!out) return fail(ASA_ERR_NULL_ARG, "csr is NULL");
  if (!out->row_ptr || !out->col_idx) return fail(ASA_ERR_NULL_ARG, "csr row_ptr/col_idx is NULL");
  const int64_t need = asa_csr_capacity(s);
  if (out->capacity < need)
    return fail(ASA_ERR_CAPACITY, "csr capacity %lld < required %lld", (long long)out->capacity, (long long)need);
  return ASA_OK;
}

asa_status check_workspace(void* ws, size_t have, size_t need) {
  if (!ws) return fail(ASA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (have < need) return fail(ASA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", have, need);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(ASA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return ASA_OK;
}

// Workspace carve-up for asa_pattern_search (all offsets 256-byte aligned): the full
// attention output O_0 and one candidate output (fp32 [B,H,N,d] each), one CSR mask with
// the static builder's workspace, and the per-row partials of every candidate.
struct SearchWorkspace {
  float* o0;
  float* oi;
  int32_t* row_ptr;
  int32_t* col_idx;
  void* mask_ws;
  double* sq;        // [n][B*H*Nb]
  long long* pairs;  // [n][B*H*Nb]
};

size_t search_workspace_layout(const asa_shape* s, int n, SearchWorkspace* w, void* base) {
  const asa::MaskGeom g = geom_of(s);
  const size_t rows = (size_t)s->B * s->H * g.Nb;
  const size_t out = (size_t)s->B * s->H * s->N * s->d * sizeof(float);
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return b ? b + at : nullptr;
  };
  SearchWorkspace t{};
  t.o0 = reinterpret_cast<float*>(take(out));
  t.oi = reinterpret_cast<float*>(take(out));
  t.row_ptr = reinterpret_cast<int32_t*>(take((rows + 1) * sizeof(int32_t)));
  t.col_idx = reinterpret_cast<int32_t*>(take(rows * (size_t)g.Nb * sizeof(int32_t)));
  t.mask_ws = take(asa::mask_workspace_layout(g, false, nullptr, nullptr));
  t.sq = reinterpret_cast<double*>(take((size_t)n * rows * sizeof(double)));
  t.pairs = reinterpret_cast<long long*>(take((size_t)n * rows * sizeof(long long)));
  if (w) *w = t;
  return off;
}

asa::AttnArgs attn_args(const void* Q, const void* K, const void* V, void* O, bool out_bf16,
                        const asa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                        const int32_t* order, float scale, float* lse) {
  asa::AttnArgs a{};
  a.q = Q; a.k = K; a.v = V; a.o = O;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.order = order;
  a.lse = lse;
  a.B = shape->B; a.H = shape->H; a.N = shape->N; a.d = shape->d; a.blk = shape->blk;
  a.Nb = (int)num_blocks(shape);
  a.in_bf16 = shape->in_dtype == ASA_BF16;
  a.out_bf16 = out_bf16;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)shape->d);
  a.scale_log2 = (float)(sc * 1.4426950408889634);   // log2(e)
  return a;
}

// Split-row plan: chunk length T (kept blocks per workgroup) and chunks per row at most.
// split_blocks = 0 chooses T from the shape: a launch of fewer than kSplitRows rows (about
// 1.5 workgroups per compute unit) leaves compute units idle, so each row is cut into
// ceil(kSplitItems / rows) chunks (two workgroups per compute unit), none shorter than
// kMinChunk blocks (shorter chunks cost more in partial outputs than they gain).  A plan
// that can never split a row returns 0.
constexpr int64_t kSplitRows = 384;
constexpr int64_t kSplitItems = 512;
constexpr int64_t kMinChunk = 16;

int split_plan(const asa_shape* s, int32_t split_blocks, int* split_max) {
  const int64_t Nb = num_blocks(s);
  const int64_t rows = (int64_t)s->B * s->H * Nb;
  int64_t t = split_blocks;
  if (t == 0) {
    if (rows >= kSplitRows) {
      *split_max = 1;
      return 0;
    }
    const int64_t n = (kSplitItems + rows - 1) / rows;
    t = (Nb + n - 1) / n;
    if (t < kMinChunk) t = kMinChunk;
    const int64_t floor_t = (Nb + asa::kMaxSplit - 1) / asa::kMaxSplit;
    if (t < floor_t) t = floor_t;
  }
  if (t >= Nb) {
    *split_max = 1;
    return 0;
  }
  *split_max = (int)((Nb + t - 1) / t);
  return (int)t;
}

size_t split_workspace_layout(const asa_shape* s, int split_max, float** part_o, float** part_ml, void* base) {
  const size_t rows = (size_t)s->B * s->H * num_blocks(s);
  const size_t o_bytes = ((size_t)split_max * rows * s->blk * s->d * sizeof(float) + 255) & ~(size_t)255;
  const size_t ml_bytes = ((size_t)split_max * rows * s->blk * 2 * sizeof(float) + 255) & ~(size_t)255;
  if (part_o) *part_o = base ? reinterpret_cast<float*>(base) : nullptr;
  if (part_ml) *part_ml = base ? reinterpret_cast<float*>(static_cast<char*>(base) + o_bytes) : nullptr;
  return o_bytes + ml_bytes;
}

}  // namespace

extern "C" {

int32_t asa_version(void) { return 10800; }

const char* asa_status_string(asa_status st) {
  switch (st) {
    case ASA_OK: return "ASA_OK";
    case ASA_ERR_NULL_ARG: return "ASA_ERR_NULL_ARG";
    case ASA_ERR_BAD_SHAPE: return "ASA_ERR_BAD_SHAPE";
    case ASA_ERR_BAD_DTYPE: return "ASA_ERR_BAD_DTYPE";
    case ASA_ERR_UNSUPPORTED: return "ASA_ERR_UNSUPPORTED";
    case ASA_ERR_CAPACITY: return "ASA_ERR_CAPACITY";
    case ASA_ERR_WORKSPACE: return "ASA_ERR_WORKSPACE";
    case ASA_ERR_BAD_PATTERN: return "ASA_ERR_BAD_PATTERN";
    case ASA_ERR_BAD_PARAM: return "ASA_ERR_BAD_PARAM";
    case ASA_ERR_HIP: return "ASA_ERR_HIP";
  }
  return "ASA_ERR_UNKNOWN";
}

const char* asa_last_error(void) { return g_last_error; }

int64_t asa_csr_capacity(const asa_shape* shape) {
  if (check_shape(shape, true) != ASA_OK) return -1;   // the shapes the mask builders accept
  const int64_t Nb = num_blocks(shape);
  return (int64_t)shape->B * shape->H * Nb * Nb;
}

size_t asa_build_mask_workspace_size(const asa_shape* shape) {
  if (check_shape(shape, true) != ASA_OK) return 0;
  return asa::mask_workspace_layout(geom_of(shape), true, nullptr, nullptr);
}

size_t asa_static_mask_workspace_size(const asa_shape* shape) {
  if (check_shape(shape, true) != ASA_OK) return 0;
  return asa::mask_workspace_layout(geom_of(shape), false, nullptr, nullptr);
}

// asa_build_mask and its variant without allocation (no_alloc: the workspace is the
// device's static scratch array, found after every argument check has passed).
static asa_status build_mask_impl(const void* Q, const void* K, const asa_shape* shape,
                                  const asa_adaptive* ad, const asa_head_pattern* patterns,
                                  const asa_csr* out, void* workspace, size_t workspace_bytes,
                                  void* stream, bool no_alloc) {
  g_last_error[0] = '\0';
  asa_status st = check_shape(shape, true);
  if (st != ASA_OK) return st;
  if (!Q || !K) return fail(ASA_ERR_NULL_ARG, "Q or K is NULL");
  if (!ad) return fail(ASA_ERR_NULL_ARG, "adaptive parameters are NULL");
  if (ad->mode != ASA_MODE_TOPK && ad->mode != ASA_MODE_TAU)
    return fail(ASA_ERR_BAD_PARAM, "adaptive mode %d is not TOPK or TAU", ad->mode);
  if (ad->mode == ASA_MODE_TOPK && ad->k < 0) return fail(ASA_ERR_BAD_PARAM, "k=%d must be >= 0", ad->k);
  if (ad->mode == ASA_MODE_TAU && !(ad->tau >= 0.0 && std::isfinite(ad->tau)))
    return fail(ASA_ERR_BAD_PARAM, "tau=%g must be finite and >= 0", ad->tau);
  if (ad->k_cap < 0) return fail(ASA_ERR_BAD_PARAM, "k_cap=%d must be >= 0", ad->k_cap);
  if (ad->n_text < 0 || ad->n_text > shape->N)
    return fail(ASA_ERR_BAD_PARAM, "n_text=%d must lie in [0, N]", ad->n_text);
  if (ad->keep_diag != 0 && ad->keep_diag != 1) return fail(ASA_ERR_BAD_PARAM, "keep_diag must be 0 or 1");
  asa::HeadTable heads;
  if ((st = fill_heads(shape, patterns, true, &heads)) != ASA_OK) return st;
  if ((st = check_csr_out(shape, out)) != ASA_OK) return st;
  const asa::MaskGeom g = geom_of(shape);
  const size_t need = asa::mask_workspace_layout(g, true, nullptr, nullptr);
  if (no_alloc) {
    if (need > asa::kNoAllocScratchBytes)
      return fail(ASA_ERR_WORKSPACE, "shape needs %zu workspace bytes, more than the %zu-byte static scratch", need,
                  asa::kNoAllocScratchBytes);
    hipError_t e = asa::noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    workspace_bytes = asa::kNoAllocScratchBytes;
  }
  if ((st = check_workspace(workspace, workspace_bytes, need)) != ASA_OK) return st;

  asa::MaskWorkspace ws;
  asa::mask_workspace_layout(g, true, &ws, workspace);
  asa::AdaptiveParams p{};
  p.mode = ad->mode;
  p.k = ad->k;
  p.tau = ad->tau;
  p.k_cap = ad->k_cap;
  p.n_text_blocks = ad->n_text > 0 ? (int)((ad->n_text + shape->blk - 1) / shape->blk) : 0;
  p.keep_diag = ad->keep_diag;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = asa::launch_pool(Q, K, shape->in_dtype == ASA_BF16, g, ws, s)) != hipSuccess) return hip_fail(e, "pool");
  if ((e = asa::launch_rank(g, p, heads, ws, s)) != hipSuccess) return hip_fail(e, "rank");
  if ((e = asa::launch_csr(g, ws, out->row_ptr, out->col_idx, out->order, s)) != hipSuccess) return hip_fail(e, "csr");
  return ASA_OK;
}

asa_status asa_build_mask(const void* Q, const void* K, const asa_shape* shape,
                          const asa_adaptive* ad, const asa_head_pattern* patterns,
                          const asa_csr* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return build_mask_impl(Q, K, shape, ad, patterns, out, workspace, workspace_bytes, stream, false);
}

asa_status asa_build_mask_noalloc(const void* Q, const void* K, const asa_shape* shape,
                                  const asa_adaptive* ad, const asa_head_pattern* patterns,
                                  const asa_csr* out, void* stream) {
  return build_mask_impl(Q, K, shape, ad, patterns, out, nullptr, 0, stream, true);
}

asa_status asa_static_mask(const asa_shape* shape, const asa_head_pattern* patterns,
                           const asa_csr* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_last_error[0] = '\0';
  asa_status st = check_shape(shape, true);
  if (st != ASA_OK) return st;
  if (!patterns) return fail(ASA_ERR_NULL_ARG, "patterns is NULL (required for the static call)");
  asa::HeadTable heads;
  if ((st = fill_heads(shape, patterns, false, &heads)) != ASA_OK) return st;
  if ((st = check_csr_out(shape, out)) != ASA_OK) return st;
  const asa::MaskGeom g = geom_of(shape);
  const size_t need = asa::mask_workspace_layout(g, false, nullptr, nullptr);
  if ((st = check_workspace(workspace, workspace_bytes, need)) != ASA_OK) return st;
  asa::MaskWorkspace ws;
  asa::mask_workspace_layout(g, false, &ws, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = asa::launch_static_rows(g, heads, ws, s)) != hipSuccess) return hip_fail(e, "static rows");
  if ((e = asa::launch_csr(g, ws, out->row_ptr, out->col_idx, out->order, s)) != hipSuccess) return hip_fail(e, "csr");
  return ASA_OK;
}

static asa_status attention_fwd_impl(const void* Q, const void* K, const void* V, void* O,
                                     int32_t o_dtype, const asa_shape* shape, const asa_csr* csr,
                                     const asa_head_pattern* patterns, float scale, float* lse,
                                     bool need_lse, void* stream, bool split_call = false,
                                     int32_t split_blocks = 0, void* workspace = nullptr,
                                     size_t workspace_bytes = 0) {
  g_last_error[0] = '\0';
  if (need_lse && !lse) return fail(ASA_ERR_NULL_ARG, "lse is NULL");
  asa_status st = check_shape(shape, false);
  if (st != ASA_OK) return st;
  if (!Q || !K || !V || !O) return fail(ASA_ERR_NULL_ARG, "Q, K, V or O is NULL");
  if (o_dtype != ASA_F32 && o_dtype != ASA_BF16)
    return fail(ASA_ERR_BAD_DTYPE, "o_dtype=%d is not ASA_F32 or ASA_BF16", o_dtype);
  if (!csr) return fail(ASA_ERR_NULL_ARG, "csr is NULL");
  if (!csr->row_ptr || !csr->col_idx) return fail(ASA_ERR_NULL_ARG, "csr row_ptr/col_idx is NULL");
  if (!(std::isfinite(scale))) return fail(ASA_ERR_BAD_PARAM, "scale must be finite");
  asa::HeadTable heads;
  if ((st = fill_heads(shape, patterns, true, &heads)) != ASA_OK) return st;

  asa::AttnArgs a = attn_args(Q, K, V, O, o_dtype == ASA_BF16, shape, csr->row_ptr, csr->col_idx,
                              csr->order, scale, lse);
  if (patterns)
    for (int h = 0; h < shape->H; ++h)
      if (patterns[h].id == ASA_PAT_SKIP) a.skip_bits[h >> 5] |= 1u << (h & 31);
  if (split_call) {
    if (split_blocks < 0) return fail(ASA_ERR_BAD_PARAM, "split_blocks=%d must be >= 0", split_blocks);
    int smax = 1;
    const int t = split_plan(shape, split_blocks, &smax);
    if (smax > asa::kMaxSplit)
      return fail(ASA_ERR_BAD_PARAM, "split_blocks=%d cuts a %lld-block row into more than %d chunks", split_blocks,
                  (long long)num_blocks(shape), asa::kMaxSplit);
    if (t > 0) {
      const size_t need = split_workspace_layout(shape, smax, nullptr, nullptr, nullptr);
      if ((st = check_workspace(workspace, workspace_bytes, need)) != ASA_OK) return st;
      a.split_blocks = t;
      a.split_max = smax;
      split_workspace_layout(shape, smax, &a.part_o, &a.part_ml, workspace);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = asa::launch_attention(a, s);
  if (e != hipSuccess) return hip_fail(e, "attention");
  if (a.split_blocks > 0 && (e = asa::launch_split_combine(a, s)) != hipSuccess) return hip_fail(e, "split combine");
  return ASA_OK;
}

asa_status asa_attention_fwd(const void* Q, const void* K, const void* V, void* O, int32_t o_dtype,
                             const asa_shape* shape, const asa_csr* csr,
                             const asa_head_pattern* patterns, float scale, void* stream) {
  return attention_fwd_impl(Q, K, V, O, o_dtype, shape, csr, patterns, scale, nullptr, false, stream);
}

asa_status asa_attention_fwd_lse(const void* Q, const void* K, const void* V, void* O, int32_t o_dtype,
                                 const asa_shape* shape, const asa_csr* csr,
                                 const asa_head_pattern* patterns, float scale, float* lse,
                                 void* stream) {
  return attention_fwd_impl(Q, K, V, O, o_dtype, shape, csr, patterns, scale, lse, true, stream);
}

size_t asa_attention_fwd_split_workspace_size(const asa_shape* shape, int32_t split_blocks) {
  if (check_shape(shape, false) != ASA_OK || split_blocks < 0) return 0;
  int smax = 1;
  if (split_plan(shape, split_blocks, &smax) == 0 || smax > asa::kMaxSplit) return 0;
  return split_workspace_layout(shape, smax, nullptr, nullptr, nullptr);
}

asa_status asa_attention_fwd_split(const void* Q, const void* K, const void* V, void* O, int32_t o_dtype,
                                   const asa_shape* shape, const asa_csr* csr,
                                   const asa_head_pattern* patterns, float scale, float* lse,
                                   int32_t split_blocks, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return attention_fwd_impl(Q, K, V, O, o_dtype, shape, csr, patterns, scale, lse, false, stream, true,
                            split_blocks, workspace, workspace_bytes);
}

size_t asa_attention_bwd_workspace_size(const asa_shape* shape) {
  if (check_shape(shape, true) != ASA_OK) return 0;
  asa::BwdArgs g{};
  g.B = shape->B; g.H = shape->H; g.N = shape->N; g.d = shape->d; g.blk = shape->blk;
  g.Nb = (int)num_blocks(shape);
  return asa::bwd_workspace_layout(g, nullptr, nullptr);
}

asa_status asa_attention_bwd(const void* Q, const void* K, const void* V, const void* O,
                             int32_t o_dtype, const void* dO, const float* lse, float* dQ, float* dK,
                             float* dV, const asa_shape* shape, const asa_csr* csr,
                             const asa_head_pattern* patterns, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  asa_status st = check_shape(shape, true);
  if (st != ASA_OK) return st;
  if (!Q || !K || !V || !O || !dO || !lse) return fail(ASA_ERR_NULL_ARG, "Q, K, V, O, dO or lse is NULL");
  if (!dQ || !dK || !dV) return fail(ASA_ERR_NULL_ARG, "dQ, dK or dV is NULL");
  if (o_dtype != ASA_F32 && o_dtype != ASA_BF16)
    return fail(ASA_ERR_BAD_DTYPE, "o_dtype=%d is not ASA_F32 or ASA_BF16", o_dtype);
  if (!csr) return fail(ASA_ERR_NULL_ARG, "csr is NULL");
  if (!csr->row_ptr || !csr->col_idx) return fail(ASA_ERR_NULL_ARG, "csr row_ptr/col_idx is NULL");
  if (!(std::isfinite(scale))) return fail(ASA_ERR_BAD_PARAM, "scale must be finite");
  asa::HeadTable heads;
  if ((st = fill_heads(shape, patterns, true, &heads)) != ASA_OK) return st;
  asa::BwdArgs a{};
  a.B = shape->B; a.H = shape->H; a.N = shape->N; a.d = shape->d; a.blk = shape->blk;
  a.Nb = (int)num_blocks(shape);
  const size_t need = asa::bwd_workspace_layout(a, nullptr, nullptr);
  if ((st = check_workspace(workspace, workspace_bytes, need)) != ASA_OK) return st;
  asa::bwd_workspace_layout(a, &a, workspace);
  a.q = Q; a.k = K; a.v = V; a.o = O; a.dout = dO; a.lse = lse;
  a.dq = dQ; a.dk = dK; a.dv = dV;
  a.row_ptr = csr->row_ptr;
  a.col_idx = csr->col_idx;
  a.order = csr->order;
  a.o_bf16 = o_dtype == ASA_BF16;
  a.in_f32 = shape->in_dtype == ASA_F32;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)shape->d);
  a.scale = (float)sc;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  if (patterns)
    for (int h = 0; h < shape->H; ++h)
      if (patterns[h].id == ASA_PAT_SKIP) a.skip_bits[h >> 5] |= 1u << (h & 31);
  hipError_t e = asa::launch_attention_bwd(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention backward");
  return ASA_OK;
}

size_t asa_pattern_search_workspace_size(const asa_shape* shape, int32_t n_candidates) {
  if (check_shape(shape, true) != ASA_OK) return 0;
  if (n_candidates < 0 || n_candidates > asa::kMaxSearchCandidates) return 0;
  return search_workspace_layout(shape, n_candidates, nullptr, nullptr);
}

asa_status asa_pattern_search(const void* Q, const void* K, const void* V, const asa_shape* shape,
                              const asa_head_pattern* candidates, int32_t n_candidates, double lambda,
                              double eps, float scale, double* loss, double* mse, int32_t* choice,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  asa_status st = check_shape(shape, true);
  if (st != ASA_OK) return st;
  if (!Q || !K || !V) return fail(ASA_ERR_NULL_ARG, "Q, K or V is NULL");
  if (!choice) return fail(ASA_ERR_NULL_ARG, "choice is NULL");
  if (!loss && n_candidates > 0) return fail(ASA_ERR_NULL_ARG, "loss is NULL");
  if (n_candidates < 0 || n_candidates > asa::kMaxSearchCandidates)
    return fail(ASA_ERR_BAD_PARAM, "n_candidates=%d must lie in [0, %d]", n_candidates,
                asa::kMaxSearchCandidates);
  if (n_candidates > 0 && !candidates) return fail(ASA_ERR_NULL_ARG, "candidates is NULL");
  for (int i = 0; i < n_candidates; ++i) {
    const int id = candidates[i].id, prm = candidates[i].param;
    if (id == ASA_PAT_ADAPTIVE || id < ASA_PAT_ADAPTIVE || id > ASA_PAT_FRAME_TILE)
      return fail(ASA_ERR_BAD_PATTERN, "candidate %d: pattern id %d is not a static pattern", i, id);
    if (id == ASA_PAT_MULTIDIAG && prm <= 0)
      return fail(ASA_ERR_BAD_PATTERN, "candidate %d: multi-diagonal stride %d must be > 0", i, prm);
    if (id == ASA_PAT_VSTRIPE && prm < 0)
      return fail(ASA_ERR_BAD_PATTERN, "candidate %d: vertical-stripe width %d must be >= 0", i, prm);
    if (id == ASA_PAT_FRAME_TILE && prm <= 0)
      return fail(ASA_ERR_BAD_PATTERN, "candidate %d: frame-tile frame length %d must be > 0", i, prm);
  }
  if (!std::isfinite(lambda) || !std::isfinite(eps))
    return fail(ASA_ERR_BAD_PARAM, "lambda and eps must be finite");
  if (!std::isfinite(scale)) return fail(ASA_ERR_BAD_PARAM, "scale must be finite");
  const size_t need = search_workspace_layout(shape, n_candidates, nullptr, nullptr);
  if ((st = check_workspace(workspace, workspace_bytes, need)) != ASA_OK) return st;

  SearchWorkspace w;
  search_workspace_layout(shape, n_candidates, &w, workspace);
  const asa::MaskGeom g = geom_of(shape);
  asa::MaskWorkspace mws;
  asa::mask_workspace_layout(g, false, &mws, w.mask_ws);
  const size_t rows = (size_t)shape->B * shape->H * g.Nb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  asa::HeadTable heads;

  // M0: full attention, the reference every candidate is scored against.
  std::memset(&heads, 0, sizeof(heads));
  for (int h = 0; h < shape->H; ++h) heads.id[h] = ASA_PAT_FULL;
  if ((e = asa::launch_static_rows(g, heads, mws, s)) != hipSuccess) return hip_fail(e, "full mask rows");
  if ((e = asa::launch_csr(g, mws, w.row_ptr, w.col_idx, nullptr, s)) != hipSuccess) return hip_fail(e, "full mask csr");
  asa::AttnArgs a = attn_args(Q, K, V, w.o0, false, shape, w.row_ptr, w.col_idx, nullptr, scale, nullptr);
  if ((e = asa::launch_attention(a, s)) != hipSuccess) return hip_fail(e, "full attention");

  for (int i = 0; i < n_candidates; ++i) {
    const int id = candidates[i].id;
    int prm = candidates[i].param;
    if (id == ASA_PAT_VSTRIPE && prm > g.Nb) prm = g.Nb;
    for (int h = 0; h < shape->H; ++h) { heads.id[h] = id; heads.param[h] = prm; }
    if ((e = asa::launch_static_rows(g, heads, mws, s)) != hipSuccess) return hip_fail(e, "candidate mask rows");
    if ((e = asa::launch_csr(g, mws, w.row_ptr, w.col_idx, nullptr, s)) != hipSuccess)
      return hip_fail(e, "candidate mask csr");
    const float* oi = nullptr;   // a skipped head's output is zero: nothing to compute
    if (id != ASA_PAT_SKIP) {
      a = attn_args(Q, K, V, w.oi, false, shape, w.row_ptr, w.col_idx, nullptr, scale, nullptr);
      if ((e = asa::launch_attention(a, s)) != hipSuccess) return hip_fail(e, "candidate attention");
      oi = w.oi;
    }
    if ((e = asa::launch_search_sq_err(w.o0, oi, w.row_ptr, w.col_idx, shape->B, shape->H, shape->N,
                                       shape->d, shape->blk, g.Nb, w.sq + i * rows, w.pairs + i * rows, s)) !=
        hipSuccess)
      return hip_fail(e, "squared error");
  }
  if ((e = asa::launch_search_choose(w.sq, w.pairs, shape->B, shape->H, shape->N, shape->d, g.Nb, n_candidates,
                                     lambda, eps, loss, mse, choice, s)) != hipSuccess)
    return hip_fail(e, "choose");
  return ASA_OK;
}

}  // extern "C"
