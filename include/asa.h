/*
 * asa.h -- C ABI of the MI355X (gfx950) content-aware block-sparse attention library.
 *
 * The library builds block masks over (query-block, key-block) tiles and computes
 * softmax(Q K^T / sqrt(d)) V over the kept tiles only.
 *
 * Sources of the operations (page title, then section / formula / table):
 *  - "Sparse-vDiT: Sparse Attention Acceleration for Video Diffusion Transformers",
 *    section 三 "核心公式": full attention per head softmax(Q_h K_h^T / sqrt(d)) V_h of
 *    shape B x N x d, and the masked form Attention(Q, K, V, M).
 *  - same page, "四种注意力模式" table: the static mask sources M0 full, M1 skip (output
 *    set to zero), M2 diagonal, M3 multi-diagonal, M4 vertical stripe.
 *  - "BLADE: Block-Sparse Attention Meets Step Distillation for Efficient Video
 *    Generation", abstract: Adaptive Block-Sparse Attention (ASA) generates a
 *    content-aware sparsity mask from the input.  The pages leave ASA's rule open; the
 *    rule implemented here is stated at asa_build_mask below.
 *
 * Conventions shared by every entry point
 *  - Tensors are contiguous row-major [B, H, N, d] device arrays.  d is 64 or 128; the
 *    block size blk (used for both query and key blocks, so the diagonal is defined) is
 *    64 or 128.  Nb = ceil(N / blk); block r covers tokens [r*blk, min((r+1)*blk, N)).
 *  - Every pointer argument that names tensor data is a DEVICE pointer.  Struct
 *    arguments (asa_shape, asa_adaptive, asa_head_pattern arrays, asa_csr) are HOST
 *    memory read during the call only.
 *  - Ownership: the caller allocates every buffer (outputs and workspace).  The library
 *    allocates nothing, keeps no state between calls and never synchronizes: all work is
 *    enqueued on `stream` (a hipStream_t; NULL means the default stream).  The one
 *    exception is asa_build_mask_noalloc, whose workspace is a static device array.
 *  - Errors: arguments are validated on the host before anything is enqueued; an invalid
 *    call returns a negative asa_status, enqueues nothing, and asa_last_error() returns a
 *    thread-local message.  Launch failures return ASA_ERR_HIP.  Faults inside kernels
 *    surface at the caller's next synchronization.  No C++ exception crosses the ABI.
 *  - Determinism: identical inputs give bit-identical CSR arrays and outputs.
 */
#ifndef ASA_H_
#define ASA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum asa_status {
  ASA_OK = 0,
  ASA_ERR_NULL_ARG = -1,     /* a required pointer is NULL                         */
  ASA_ERR_BAD_SHAPE = -2,    /* B, H, N <= 0, or sizes overflow int32 indexing      */
  ASA_ERR_BAD_DTYPE = -3,    /* dtype code not ASA_F32 / ASA_BF16                   */
  ASA_ERR_UNSUPPORTED = -4,  /* d not in {64,128}, blk not in {64,128}, Nb > 1024    */
  ASA_ERR_CAPACITY = -5,     /* csr->capacity below asa_csr_capacity()              */
  ASA_ERR_WORKSPACE = -6,    /* workspace NULL or smaller than the *_workspace_size  */
  ASA_ERR_BAD_PATTERN = -7,  /* unknown pattern id or invalid pattern parameter      */
  ASA_ERR_BAD_PARAM = -8,    /* adaptive parameters out of range                     */
  ASA_ERR_HIP = -9           /* a HIP runtime call or kernel launch failed           */
} asa_status;

typedef enum asa_dtype { ASA_F32 = 0, ASA_BF16 = 1 } asa_dtype;

/* Per-head mask sources.  Codes follow the Sparse-vDiT mode table (M0..M4), plus the
 * adaptive ASA source and Efficient-vDiT's frame tiles. */
enum {
  ASA_PAT_ADAPTIVE = 0,   /* adaptive only (asa_build_mask)                                 */
  ASA_PAT_FULL = 1,       /* M0: every key block                                           */
  ASA_PAT_SKIP = 2,       /* M1: no key block; the head's output is zero                   */
  ASA_PAT_DIAG = 3,       /* M2: key block c == query block r                              */
  ASA_PAT_MULTIDIAG = 4,  /* M3: param = stride S in tokens (> 0); tile (r,c) kept iff some
                             query i in block r and key j in block c have (j - i) % S == 0  */
  ASA_PAT_VSTRIPE = 5,    /* M4: param = s >= 0 leading key blocks (global tokens), c < s   */
  ASA_PAT_FRAME_TILE = 6  /* frame tiles, after "Efficient-vDiT: Efficient Video Diffusion
                             Transformers With Attention Tile", section 3.1: param = F > 0
                             tokens per frame, frame(t) = floor(t / F); tile (r,c) kept iff
                             some query i in block r and key j in block c have
                             frame(j) == frame(i) or frame(j) == 0.  The page names no tile
                             set; this one (own frame + first frame) costs O(N F).        */
};

enum { ASA_MODE_TOPK = 0, ASA_MODE_TAU = 1 };

typedef struct asa_shape {
  int32_t B, H, N, d, blk;
  int32_t in_dtype;        /* asa_dtype of Q, K, V */
} asa_shape;

typedef struct asa_adaptive {
  int32_t mode;            /* ASA_MODE_TOPK or ASA_MODE_TAU                                  */
  int32_t k;               /* TOPK: number of key blocks kept per row (>= 0)                 */
  double tau;              /* TAU: cumulative probability mass to reach, in [0, +inf)        */
  int32_t k_cap;           /* TAU: cap on the adaptive prefix length (0 = no cap)            */
  int32_t n_text;          /* leading text tokens: blocks holding any are kept as rows and
                              columns (0 = none)                                             */
  int32_t keep_diag;       /* 1 = always keep the diagonal block                             */
} asa_adaptive;

typedef struct asa_head_pattern {
  int32_t id;              /* ASA_PAT_* */
  int32_t param;           /* stride in tokens (MULTIDIAG) or leading blocks (VSTRIPE) */
} asa_head_pattern;

/* Block mask in CSR form: one row per (b, h, query block r), rows in [B, H, Nb] order.
 * row_ptr has B*H*Nb + 1 entries (row_ptr[0] = 0, row_ptr[last] = number of kept tiles);
 * col_idx lists the kept key blocks of each row in ascending order.  Both are device
 * int32 arrays owned by the caller; capacity is the length of col_idx in elements.
 *
 * order (optional, may be NULL) is the attention schedule: a device int32 array of
 * B*H*Nb entries holding a permutation of the rows.  The pages leave the work order open;
 * this schedule exists for load balance.  Its positions split into 8 contiguous ranges,
 * one per XCD of the MI355X (range x starts at x*floor(R/8) + min(x, R%8) for R rows, and
 * the first R%8 ranges hold one extra position); the rows at the positions of range x run
 * on XCD x.
 *   - asa_build_mask / asa_static_mask fill it when non-NULL, as follows.  A row's length
 *     class is 0 when it is empty, else 1 + floor(log2 of its kept count).  The rows of each
 *     class, in row order, are cut into 8 consecutive slices; range x holds slice x of every
 *     class, longest class first, each slice in row order.  Class c (s_c rows) has slices
 *     of floor(s_c/8) rows, and s_c%8 of them one row more: those go to the XCDs
 *     cursor, cursor+1, ... (mod 8), where cursor starts at 0 for the longest class and
 *     advances by s_c%8 (mod 8) after each class.  So every XCD gets an equal share of the
 *     long rows, a slice is a run of neighbouring rows, and each range has exactly its
 *     number of positions.  The result is deterministic.
 *   - asa_attention_fwd processes the rows in this order when it is non-NULL, and in row
 *     order otherwise.  The outputs are bit-identical either way.  A caller-made order
 *     must be a permutation of 0..B*H*Nb-1, or rows go unwritten (not checked: the array
 *     is device memory). */
typedef struct asa_csr {
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t capacity;
  int32_t* order;
} asa_csr;

/* Library version (major*10000 + minor*100 + patch).  1.1.0 added asa_csr.order;
 * 1.2.0 added asa_pattern_search; 1.3.0 added asa_attention_fwd_split; 1.4.0 added
 * ASA_PAT_FRAME_TILE; 1.5.0: asa_attention_bwd follows asa_csr.order, and asa_csr_capacity
 * returns -1 for every shape the mask builders reject; 1.6.0 added asa_build_mask_noalloc;
 * 1.7.0: the schedule gives every XCD an equal share of each row-length class; 1.8.0:
 * asa_attention_bwd takes fp32 inputs. */
int32_t asa_version(void);

/* Human-readable name of a status code (static storage). */
const char* asa_status_string(asa_status status);

/* Message describing the last failed call on this thread ("" if none). */
const char* asa_last_error(void);

/* Number of col_idx elements the mask builders require: B*H*Nb*Nb (the worst case, since
 * the kept count is known only on the device).  Returns -1 for a shape the mask builders
 * reject (see the status codes), with the reason in asa_last_error(). */
int64_t asa_csr_capacity(const asa_shape* shape);

/* Workspace bytes for asa_build_mask (pooled Q and K, row bitmasks and counts).  Returns 0 for an invalid shape. */
size_t asa_build_mask_workspace_size(const asa_shape* shape);

/* Workspace bytes for asa_static_mask (row bitmasks and counts).  0 for an invalid shape. */
size_t asa_static_mask_workspace_size(const asa_shape* shape);

/*
 * asa_build_mask -- adaptive (ASA) block mask, unioned with forced and static blocks.
 *
 * Source: BLADE abstract (content-aware adaptive block mask, rule left open by the pages)
 * and the Sparse-vDiT mode table (static sources).  The rule computed, in float64:
 *   1. Qp[r] = mean of Q over the tokens of block r; Kp[c] likewise (a partial last block
 *      is averaged over its own tokens).
 *   2. S[r,c] = Qp[r] . Kp[c] / sqrt(d).
 *   3. P[r,:] = softmax of S[r,:] over all Nb key blocks.
 *   4. Order the key blocks by P descending, ties by smaller index.
 *   5. Adaptive set A_r: TOPK keeps the first min(k, Nb); TAU keeps the shortest prefix
 *      whose running sum (in rank order) is >= tau (all Nb if none), then at most k_cap.
 *   6. kept_r = A_r, plus block r if keep_diag, plus every key block holding a text token;
 *      a query block holding a text token keeps every key block.
 *   7. Heads whose pattern id is not ASA_PAT_ADAPTIVE add their static pattern's blocks;
 *      an ASA_PAT_SKIP head gets empty rows.
 *
 * Q, K       device [B,H,N,d] of shape->in_dtype.
 * adaptive   host struct (see asa_adaptive).
 * patterns   host array [H] or NULL (NULL = every head ASA_PAT_ADAPTIVE).
 * out        host struct with device row_ptr / col_idx; capacity >= asa_csr_capacity().
 * workspace  device buffer of at least asa_build_mask_workspace_size(shape) bytes,
 *            256-byte aligned; its contents on entry are ignored.
 */
asa_status asa_build_mask(const void* Q, const void* K, const asa_shape* shape,
                          const asa_adaptive* adaptive, const asa_head_pattern* patterns,
                          const asa_csr* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of the static device scratch array behind asa_build_mask_noalloc (per GPU). */
#define ASA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * asa_build_mask_noalloc -- asa_build_mask for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Computes exactly what asa_build_mask computes (the same kernels; bit-identical CSR and
 * order), but takes no workspace argument: the pooled Q and K, row bitmasks and counts live
 * in a static device array of ASA_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends.  The call allocates nothing and frees
 * nothing; the first call on a device looks up that device's copy of the array (with the
 * device current), later calls reuse the address.  It runs on the current device, and
 * `stream` must belong to it.
 *
 * Every argument as asa_build_mask.  Limit: asa_build_mask_workspace_size(shape) must not
 * exceed ASA_NOALLOC_SCRATCH_BYTES (enough for B*H*Nb*d*16 bytes of pooled Q and K plus
 * the bitmask: e.g. 24 heads, N = 75600, d = 128 at blk = 128); a larger shape returns
 * ASA_ERR_WORKSPACE and enqueues nothing.
 * Concurrency: every call on one GPU shares that GPU's array, and each call overwrites it
 * entirely before reading it (nothing has to start at zero).  Calls whose work overlaps on
 * one GPU -- on different streams, or from different threads without ordering -- race on
 * the array and give undefined masks; order them on one stream.
 */
asa_status asa_build_mask_noalloc(const void* Q, const void* K, const asa_shape* shape,
                                  const asa_adaptive* adaptive, const asa_head_pattern* patterns,
                                  const asa_csr* out, void* stream);

/*
 * asa_static_mask -- block mask from per-head static patterns alone (Sparse-vDiT mode
 * table: full, skip, diagonal, multi-diagonal, vertical stripe).  No tensor is read.
 * Every entry of `patterns` (host array [H], required) must be a static id (not
 * ASA_PAT_ADAPTIVE).  shape->d and shape->in_dtype are not used by this call but must be
 * valid.  Workspace: asa_static_mask_workspace_size(shape) bytes, 256-byte aligned.
 */
asa_status asa_static_mask(const asa_shape* shape, const asa_head_pattern* patterns,
                           const asa_csr* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * asa_attention_fwd -- block-sparse attention forward over the kept tiles.
 *
 * Source: Sparse-vDiT section 三 "核心公式" (attention formula and masked attention M).
 * For each query token i of block r: O_i = sum_j softmax_j(Q_i . K_j * scale) V_j over
 * the tokens j of the key blocks listed in CSR row (b,h,r); O_i = 0 when the row is empty
 * or the head's pattern is ASA_PAT_SKIP.  No token-level masking inside kept tiles.
 *
 * Q, K, V    device [B,H,N,d] of shape->in_dtype.  For ASA_BF16 inputs the products run
 *            on bf16 matrix cores with fp32 accumulation (softmax weights are rounded to
 *            bf16 before the PV product, and the normalizer sums those rounded weights);
 *            ASA_F32 inputs run entirely in fp32.
 * O          device [B,H,N,d] of o_dtype (ASA_F32 recommended; ASA_BF16 rounds to bf16).
 * csr        host struct with device arrays, e.g. from asa_build_mask / asa_static_mask;
 *            col_idx entries must lie in [0, Nb) (not checked on the device).
 * patterns   host array [H] or NULL; used only to zero ASA_PAT_SKIP heads without
 *            reading their CSR rows.
 * scale      softmax scale; <= 0 selects 1/sqrt(d).
 */
asa_status asa_attention_fwd(const void* Q, const void* K, const void* V, void* O,
                             int32_t o_dtype, const asa_shape* shape, const asa_csr* csr,
                             const asa_head_pattern* patterns, float scale, void* stream);

/*
 * asa_attention_fwd_lse -- asa_attention_fwd that also returns what the backward needs to
 * recompute the softmax weights: per query, the log of its normaliser.
 *
 * Source: Sparse-vDiT section 三 "核心公式" (the softmax of the masked attention).
 * lse  device float32 [B,H,N]: lse_i = ln sum_{j in J_i} exp(scale * Q_i . K_j) over the
 *      kept tokens J_i of query i's row; -INFINITY where the row is empty or the head is
 *      ASA_PAT_SKIP.  Computed from the same running max and sum as O.
 * All other arguments and errors as asa_attention_fwd; lse NULL is ASA_ERR_NULL_ARG.
 */
asa_status asa_attention_fwd_lse(const void* Q, const void* K, const void* V, void* O,
                                 int32_t o_dtype, const asa_shape* shape, const asa_csr* csr,
                                 const asa_head_pattern* patterns, float scale, float* lse,
                                 void* stream);

/* Workspace bytes for asa_attention_fwd_split with the same split_blocks: the chunk partials
 * of split rows, split_max x B*H*Nb x blk x (d + 2) floats where split_max is the number of
 * chunks a full row would get.  Returns 0 when the plan splits nothing (the workspace may
 * then be NULL) or the arguments are invalid (the call reports which). */
size_t asa_attention_fwd_split_workspace_size(const asa_shape* shape, int32_t split_blocks);

/*
 * asa_attention_fwd_split -- asa_attention_fwd with long rows split over several
 * workgroups, for launches whose rows are few or uneven (few heads, short sequences, text
 * rows or full heads beside sparse ones).
 *
 * Same result as asa_attention_fwd (Sparse-vDiT section 三 "核心公式", the masked
 * attention), up to rounding: the pages fix no work decomposition.  A CSR row keeping
 * more than T = split_blocks key blocks is cut into n = ceil(count / T) chunks of
 * near-equal length (chunk c holds kept entries [c*count/n, (c+1)*count/n) of the row).
 * Each chunk runs the online softmax over its blocks and leaves its unnormalised output
 * and (running max, sum) per query in the workspace; a combine pass merges the chunks,
 * O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c with M = max_c m_c.  Rows of at most
 * T blocks are computed exactly as asa_attention_fwd computes them (bit-identical).
 *
 * split_blocks  T > 0, with ceil(Nb / T) <= 64; or 0 to choose T from the shape alone: a
 *               launch of R < 384 rows (B*H*Nb; fewer than about 1.5 workgroups per
 *               compute unit) gets T = max(16, ceil(Nb / ceil(512 / R))), so a row keeping
 *               every block is cut into ceil(512 / R) chunks (two per compute unit);
 *               launches of 384 rows or more are not split.  When T >= Nb nothing is split and no workspace is needed.
 * lse           device float32 [B,H,N] as asa_attention_fwd_lse, or NULL.
 * workspace     device buffer of asa_attention_fwd_split_workspace_size() bytes, 256-byte
 *               aligned (may be NULL when that size is 0).
 * Other arguments and errors as asa_attention_fwd; a negative or too small split_blocks
 * is ASA_ERR_BAD_PARAM.
 */
asa_status asa_attention_fwd_split(const void* Q, const void* K, const void* V, void* O,
                                   int32_t o_dtype, const asa_shape* shape, const asa_csr* csr,
                                   const asa_head_pattern* patterns, float scale, float* lse,
                                   int32_t split_blocks, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace bytes for asa_attention_bwd: the per-query (lse, D) pairs, the transposed
 * mask (key block -> query blocks), sized for the worst case B*H*Nb*Nb kept tiles, and the
 * key-block processing order.
 * Returns 0 for an invalid shape (including Nb > 1024). */
size_t asa_attention_bwd_workspace_size(const asa_shape* shape);

/*
 * asa_attention_bwd -- gradients of the block-sparse attention forward.
 *
 * Source: the masked attention of Sparse-vDiT section 三 "核心公式"; BLADE (abstract)
 * trains the sparse attention jointly with step distillation, which needs its gradients.
 * With P_ij = exp(scale Q_i.K_j - lse_i) over the kept tokens j of query i's CSR row:
 *   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . V_j,   D_i = dO_i . O_i,
 *   dS_ij = P_ij (dP_ij - D_i),   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i.
 * dQ sums over each row's kept key blocks; dK and dV over the query blocks that keep each
 * key block (the transposed mask, built in the workspace).  With bf16 inputs P and dS are
 * rounded to bf16 for the matrix products; with fp32 inputs they stay fp32 (fp32 matrix
 * products).  All accumulation is fp32.  Deterministic (no atomics).
 *
 * Q, K, V, dO  device [B,H,N,d] of shape->in_dtype (ASA_BF16 or ASA_F32).
 * O            device [B,H,N,d] of o_dtype: the forward's output for the same inputs.
 * lse          device float32 [B,H,N] from asa_attention_fwd_lse for the same inputs.
 * dQ, dK, dV   device float32 [B,H,N,d], fully written (zero where no kept tile
 *              contributes, and for ASA_PAT_SKIP heads).
 * csr          the mask the forward used (col_idx entries in [0, Nb), unique per row).  A
 *              non-NULL csr->order is the dQ pass's row schedule, as for the forward; the
 *              dK/dV pass schedules key blocks by the same rule (longest lists first inside
 *              each XCD range).  The gradients are bit-identical either way.
 * patterns     host array [H] or NULL; ASA_PAT_SKIP heads get zero gradients.
 * scale        the forward's scale; <= 0 selects 1/sqrt(d).
 * workspace    device buffer of at least asa_attention_bwd_workspace_size(shape) bytes,
 *              256-byte aligned; its contents on entry are ignored.
 * Limits: Nb <= 1024 (the transposed-mask builder), as for the mask builders.
 */
asa_status asa_attention_bwd(const void* Q, const void* K, const void* V, const void* O,
                             int32_t o_dtype, const void* dO, const float* lse, float* dQ, float* dK,
                             float* dV, const asa_shape* shape, const asa_csr* csr,
                             const asa_head_pattern* patterns, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Workspace bytes for asa_pattern_search with n_candidates candidates: two fp32 [B,H,N,d]
 * outputs (full attention and one candidate at a time), one CSR mask with the static
 * builder's workspace, and per-row partial sums.  Returns 0 for an invalid shape
 * (including Nb > 1024) or n_candidates outside [0, 8]. */
size_t asa_pattern_search_workspace_size(const asa_shape* shape, int32_t n_candidates);

/*
 * asa_pattern_search -- one layer of the per-head sparse-pattern search.
 *
 * Source: Sparse-vDiT section 三, the offline search loss L_i = MSE(O_i - O_0) +
 * lambda (1 - S_i), the pattern-selection formula, and the per-layer step of its offline
 * sparse diffusion search (run M0 and each candidate, score, choose).  The page suggests
 * lambda = 0.01, eps = 0.1 (its Table 3 ablation).  For every head h:
 *   O_0      = full attention (M0) of the head, computed here with the forward kernel;
 *   O_i      = the head's attention under candidate i's static pattern (zero for
 *              ASA_PAT_SKIP), i = 1..n_candidates;
 *   MSE_i[h] = mean over the head's B x N x d outputs of (O_i - O_0)^2, summed in float64
 *              from the fp32 outputs;
 *   S_i      = fraction of the N x N (query, key) token pairs the pattern does not attend
 *              (a kept tile counts n_r * n_c pairs, so partial blocks count at their size);
 *   L_i[h]   = MSE_i[h] + lambda * (1 - S_i);
 *   choice[h] = 0 (full attention) if L_i[h] > eps for every i (strictly), else the 1-based
 *              index of the smallest L_i[h] (the lowest index on ties).  n_candidates = 0
 *              gives choice 0 everywhere.
 * The reductions run in a fixed order: the results are deterministic.
 *
 * Q, K, V       device [B,H,N,d] of shape->in_dtype (attention as asa_attention_fwd, fp32 out).
 * candidates    host array [n_candidates] of static patterns (any id but ASA_PAT_ADAPTIVE,
 *               with that id's parameter rules), applied to every head; n_candidates <= 8.
 * lambda, eps   finite; scale as asa_attention_fwd (<= 0 selects 1/sqrt(d)).
 * loss          device float64 [H, n_candidates]: L_i[h] at h * n_candidates + (i - 1)
 *               (may be NULL only when n_candidates is 0).
 * mse           device float64 [H, n_candidates] or NULL: MSE_i[h], same layout.
 * choice        device int32 [H].
 * workspace     device buffer of at least asa_pattern_search_workspace_size() bytes,
 *               256-byte aligned; its contents on entry are ignored.
 * Errors: ASA_ERR_BAD_PATTERN for an adaptive/unknown candidate or a bad parameter,
 * ASA_ERR_BAD_PARAM for n_candidates out of range or a non-finite lambda / eps / scale.
 */
asa_status asa_pattern_search(const void* Q, const void* K, const void* V, const asa_shape* shape,
                              const asa_head_pattern* candidates, int32_t n_candidates, double lambda,
                              double eps, float scale, double* loss, double* mse, int32_t* choice,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ASA_H_ */
