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
//   rank_kernel      one workgroup per 16 rows of a head: S = Qp KpT / sqrt(d) on the
//                    fp64 matrix cores into LDS, then per row (one wavefront for 4 rows)
//                    the softmax where needed, a bitonic sort of the packed rank keys in
//                    registers, prefix selection and the union with forced / static
//                    blocks -> bitmask and count.
//   static_kernel    one wavefront per row: static pattern bitmask only.
//   csr_kernel       per-row counts -> row_ptr (each workgroup sums the counts before its
//                    rows), bitmask -> ascending col_idx; optionally the processing order
//                    (an equal share of every row-length class per XCD, long rows first)
//                    from eight more workgroups.
#include <hip/hip_runtime.h>

#include <mutex>

#include "asa_internal.h"
#include "order.h"

// Workspace of asa_build_mask_noalloc, for callers that cannot allocate device memory.
// Each GPU holds its own copy until the process ends.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol): it takes the device
// address from noalloc_scratch below.
static __device__ __align__(256) unsigned char scratch[asa::kNoAllocScratchBytes];

namespace asa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;

__device__ inline double bf16_to_f64(uint16_t x) {
  return (double)__uint_as_float(((uint32_t)x) << 16);
}

// ------------------------------------------------------------------ static patterns
// Is key block c kept in query-block row r by static pattern (id, param)?  Everything is
// 32-bit: token indices lie in [0, N) and their differences in (-N, N), with N an int, and
// the divisions are by a per-head constant (64-bit integer division is a long emulated
// sequence on the GPU).
__device__ inline bool static_keep(int id, int param, int r, int c, int N, int blk, int Nb) {
  switch (id) {
    case 1:  // full
      return true;
    case 3:  // diagonal
      return c == r;
    case 5:  // vertical stripe: leading `param` key blocks
      return c < param;
    case 4: {  // multi-diagonal, stride `param` tokens
      const int qlo = r * blk, qhi = qlo + min(blk, N - qlo) - 1;
      const int klo = c * blk, khi = klo + min(blk, N - klo) - 1;
      const int lo = klo - qhi, width = (khi - qlo) - lo;   // j - i spans [lo, lo + width]
      // the first multiple of S at or above lo is lo + (S - lo mod S) unless S divides lo
      int m = lo % param;
      if (m < 0) m += param;
      return m == 0 || width >= param - m;
    }
    case 6: {  // frame tiles of `param` tokens: the query's own frames and frame 0
      const unsigned F = (unsigned)param;
      const unsigned qlo = (unsigned)(r * blk), qhi = qlo + (unsigned)min(blk, N - (int)qlo) - 1u;
      const unsigned klo = (unsigned)(c * blk), khi = klo + (unsigned)min(blk, N - (int)klo) - 1u;
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
  // per-thread partial sums, one row per row group; each thread's VEC columns are followed
  // by one unused double, so that the lanes of a store (VEC apart) and the lanes of the
  // column sums (consecutive columns) fall on different banks
  constexpr int kRedRow = TPR * (VEC + 1);
  __shared__ double red[RPP][kRedRow];

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
  const int cg = t % TPR;   // col = cg * VEC
#pragma unroll
  for (int j = 0; j < VEC; ++j) red[sub][cg * (VEC + 1) + j] = acc[j];
  __syncthreads();
  if (t < D) {   // one thread per column sums the row groups in a fixed order
    const int slot = t + t / VEC;
    double v = 0.0;
#pragma unroll
    for (int s = 0; s < RPP; ++s) v += red[s][slot];
    const double nn = (double)n;
    if (blockIdx.y == 0) qp[(size_t)row * D + t] = v / nn;
    else kpt[((size_t)bh * D + t) * Nb + r] = v / nn;
  }
}

// ------------------------------------------------------------------ block scores + selection
// One workgroup owns `rows` (at most kRankRows) consecutive query-block rows of one head;
// the launch picks `rows` (rank_rows) so that the selection work spreads evenly over the
// compute units.
//
// Scores: S = Qp KpT / sqrt(d) for those rows against all Nb key blocks, a dense float64
// contraction on the fp64 matrix cores (v_mfma_f64_16x16x4f64), written to LDS.  Operand
// layout of the instruction, per lane l: A holds row l%16, k = l/16; B holds k = l/16,
// column l%16; result component e holds row 4e + l/16, column l%16.  The rows' pooled
// queries are copied once into LDS with 16-byte loads; the wavefronts take 16-column tiles
// in turn, with two accumulators on alternate k-steps.  The workgroup size depends on d:
// at d = 128 the contraction streams twice the KpT bytes per tile, and sixteen wavefronts
// (four per SIMD, one row each, the A operand read from LDS at each k-step) hide that
// latency best; at d = 64 eight wavefronts keep the whole A operand in registers and take
// two rows each, which lets the mass-prefix path sort two rows side by side.
//
// Selection: each wavefront ranks rows_per_wave rows.  Rank order is value
// descending, then block index ascending, and a key packs both into one uint64: the
// value's bits made order-preserving as an unsigned integer, its lowest 10 bits replaced
// by 1023 - c.  Dropping those bits merges values closer than 2^-42 relative (far inside
// the near-tie gap, where rows are ambiguous anyway); every other pair of blocks keeps its
// order, and keys of distinct blocks never tie.  Padding slots get key 0, after every
// real block.  Slot i of a row lives in register i % PER of lane i / PER (PER = NP2 / 64).
// Top-k needs only the k-th largest key (select_kth).  The mass prefix needs the rank
// order: a bitonic network sorts the NP2 slots, where exchanges at distance J < PER stay
// inside a lane's registers and the others cross lanes at distance J / PER; RI rows go
// through the network side by side for instruction-level parallelism.
constexpr int kRankRows = 16;       // rows of the score tile (the fp64 MFMA's 16 rows)
constexpr int kComputeUnits = 256;  // MI355X
constexpr int rank_threads(int d) { return d >= 128 ? 1024 : 512; }
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__device__ inline uint64_t rank_key(double v, int c) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  b = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (b & ~(uint64_t)0x3FF) | (uint64_t)(1023 - c);
}
__device__ inline int key_block(uint64_t k) { return 1023 - (int)(k & 0x3FF); }

// Compare-exchange stages J, J/2, .., 1 of the merge of runs of KK slots (runs whose index
// has bit KK clear sort descending).  Each exchange is one 64-bit compare and two selects:
// a slot takes its partner's key when the compare disagrees with the slot's role.
template <int PER, int RI, int KK, int J>
__device__ inline void rank_stage(uint64_t (&kv)[RI][PER], int lane) {
  if constexpr (J < PER) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if ((e ^ J) > e) {
        const bool desc = ((lane * PER + e) & KK) == 0;
#pragma unroll
        for (int j = 0; j < RI; ++j) {
          const uint64_t a = kv[j][e], b = kv[j][e ^ J];
          const bool sw = (a < b) == desc;
          kv[j][e] = sw ? b : a;
          kv[j][e ^ J] = sw ? a : b;
        }
      }
    }
  } else {
    constexpr int LJ = J / PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = lane * PER + e;
      const bool hi = ((i & KK) == 0) == ((i & J) == 0);   // this slot keeps the larger key
#pragma unroll
      for (int j = 0; j < RI; ++j) {
        const uint64_t a = kv[j][e];
        const uint64_t b = lane_xor64<LJ>(a);
        const bool keep = (a > b) == hi;
        kv[j][e] = keep ? a : b;
      }
    }
  }
  if constexpr (J > 1) rank_stage<PER, RI, KK, J / 2>(kv, lane);
}
template <int PER, int RI, int NP2, int KK>
__device__ inline void rank_sort_desc(uint64_t (&kv)[RI][PER], int lane) {
  rank_stage<PER, RI, KK, KK / 2>(kv, lane);
  if constexpr (KK < NP2) rank_sort_desc<PER, RI, NP2, KK * 2>(kv, lane);
}

// Butterfly reductions over the wavefront (every lane ends with the same bits), exchanging
// with lanes 32, 16, .., 1 apart.
template <int LJ>
__device__ inline double lane_xor_f64(double v) {
  return __builtin_bit_cast(double, lane_xor64<LJ>(__builtin_bit_cast(uint64_t, v)));
}
__device__ inline double wave_max(double v) {
  v = fmax(v, lane_xor_f64<32>(v));
  v = fmax(v, lane_xor_f64<16>(v));
  v = fmax(v, lane_xor_f64<8>(v));
  v = fmax(v, lane_xor_f64<4>(v));
  v = fmax(v, lane_xor_f64<2>(v));
  return fmax(v, lane_xor_f64<1>(v));
}
__device__ inline double wave_sum(double v) {
  v += lane_xor_f64<32>(v);
  v += lane_xor_f64<16>(v);
  v += lane_xor_f64<8>(v);
  v += lane_xor_f64<4>(v);
  v += lane_xor_f64<2>(v);
  return v + lane_xor_f64<1>(v);
}
__device__ inline int wave_min_int(int v) {
  v = min(v, (int)lane_xor<32>((uint32_t)v));
  v = min(v, (int)lane_xor<16>((uint32_t)v));
  v = min(v, (int)lane_xor<8>((uint32_t)v));
  v = min(v, (int)lane_xor<4>((uint32_t)v));
  v = min(v, (int)lane_xor<2>((uint32_t)v));
  return min(v, (int)lane_xor<1>((uint32_t)v));
}

__device__ inline uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// The m-th largest key of a row held by one wavefront (slot e of each lane; `real` marks
// the lanes whose slot e holds a block; real keys are distinct; 1 <= m <= real count).
// Each round reads one candidate as the pivot (from the first slot holding candidates, the
// first candidate lane at or after a rotating lane, so that an order of the keys by block
// index cannot force many rounds), counts the
// candidates above it with ballots, and keeps the side that holds the answer.  A round
// returns or removes the pivot from the candidates, and the rank sought stays >= 1, so the
// rounds are bounded by candidates + m; the loop bound enforces that.
template <int PER>
__device__ inline uint64_t select_kth(const uint64_t (&kv)[PER], const uint64_t (&real)[PER], int m) {
  uint64_t cand[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) cand[e] = real[e];
  int r = m;
  uint64_t piv = 0;
  for (int it = 0; it < 2 * 64 * PER + 2; ++it) {
    const int o = (it * 37) & 63;
    int esel = PER;
    uint64_t msk = 0ull;
#pragma unroll
    for (int e = PER - 1; e >= 0; --e)
      if (cand[e] != 0ull) { esel = e; msk = cand[e]; }
    if (esel == PER) break;   // no candidate left (only for keys that are not distinct)
    const uint64_t rot = o ? ((msk >> o) | (msk << (64 - o))) : msk;
    const int lsel = (__ffsll((unsigned long long)rot) - 1 + o) & 63;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (e == esel) piv = readlane64(kv[e], lsel);
    uint64_t gt[PER];
    int above = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      gt[e] = __ballot(kv[e] > piv) & cand[e];
      above += __popcll(gt[e]);
    }
    if (above == r - 1) return piv;
    if (above >= r) {
#pragma unroll
      for (int e = 0; e < PER; ++e) cand[e] = gt[e];
    } else {
      r -= above + 1;
#pragma unroll
      for (int e = 0; e < PER; ++e) cand[e] &= __ballot(kv[e] < piv);
    }
  }
  return piv;
}

// grid = B*H*ceil(Nb/rows) workgroups; NP2 = max(64, Nb rounded up to a power of two).
// The ids an XCD receives map onto one contiguous range of row tiles, so the tiles of a
// head (which all read that head's KpT) share an L2.
template <int D, int NP2>
__global__ __launch_bounds__(rank_threads(D)) void rank_kernel(const double* __restrict__ qp,
                                                        const double* __restrict__ kpt,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ count, MaskGeom g,
                                                        AdaptiveParams p, HeadTable heads, int rows) {
  constexpr int kRankThreads = rank_threads(D);
  constexpr int kRankWaves = kRankThreads / 64;
  constexpr int kRankRowsPerWave = kRankRows / kRankWaves;
  constexpr int PER = NP2 / 64;
  constexpr int RI = (PER >= 16 || kRankRowsPerWave < 2) ? 1 : 2;
  static_assert(kRankRowsPerWave % RI == 0, "rows per wavefront split into equal passes");
  __shared__ double srow[kRankRows][NP2];
  __shared__ uint32_t word[kRankRows][kMaxMaskBlocks / 32];
  __shared__ double qtile[kRankRows][D + 1];   // the rows' pooled queries (padded rows)

  const int Nb = g.Nb;
  const int tiles = (Nb + rows - 1) / rows;
  int lo, hi;
  xcd_range((int)(blockIdx.x % kXcds), g.B * g.H * tiles, lo, hi);
  const int tile = lo + (int)(blockIdx.x / kXcds);
  const int bh = tile / tiles, r0 = (tile - bh * tiles) * rows, h = bh % g.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int pid = heads.id[h], prm = heads.param[h];
  const size_t row0 = (size_t)bh * Nb + r0;
  const int nrows = min(rows, Nb - r0);   // the score tile's rows past nrows are not used

  if (pid == 2) {   // skip head: empty rows
    for (int i = tid; i < nrows * g.words; i += kRankThreads) bits[row0 * g.words + i] = 0u;
    if (tid < nrows) count[row0 + tid] = 0;
    return;
  }
  for (int i = tid; i < kRankRows * (kMaxMaskBlocks / 32); i += kRankThreads) (&word[0][0])[i] = 0u;

  {  // scores of the tile's rows
    // Rows past Nb and columns past Nb read clamped (valid) addresses: they only feed
    // outputs that are never used, and unconditional loads can all be in flight at once.
    // The 16 rows' pooled queries are contiguous in Qp: they go through LDS once, in
    // 16-byte loads, and the A fragments are read from there.
    const double* q = qp + (size_t)bh * Nb * D;
    const double* kt = kpt + (size_t)bh * D * Nb;
    for (int i = tid; i < kRankRows * (D / 2); i += kRankThreads) {
      const int rr = i / (D / 2), c2 = i - rr * (D / 2);
      const double2 v = reinterpret_cast<const double2*>(q + (size_t)min(r0 + rr, Nb - 1) * D)[c2];
      qtile[rr][2 * c2] = v.x;
      qtile[rr][2 * c2 + 1] = v.y;
    }
    __syncthreads();
    const int kl = lane >> 4;
    double a[kRankWaves > 8 ? 1 : D / 4];
    if constexpr (kRankWaves <= 8) {
#pragma unroll
      for (int s = 0; s < D / 4; ++s) a[s] = qtile[lane & 15][4 * s + kl];
    }
    const double sqrt_d = sqrt((double)D);
    const int ctiles = (Nb + 15) / 16;
    for (int ct = w; ct < ctiles; ct += kRankWaves) {
      const int c = ct * 16 + (lane & 15);
      const int cc = min(c, Nb - 1);
      f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
      if constexpr (kRankWaves > 8) {
        // A from LDS at each k-step, B streamed from KpT eight k-steps at a time
#pragma unroll 1
        for (int s0 = 0; s0 < D / 4; s0 += 8) {
          double b[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) b[j] = kt[(size_t)(4 * (s0 + j) + kl) * Nb + cc];
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qtile[lane & 15][4 * (s0 + j) + kl], b[j], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qtile[lane & 15][4 * (s0 + j + 1) + kl], b[j + 1], acc1, 0, 0, 0);
          }
        }
      } else {
        // A held in registers across tiles, all of B loaded before the first product
        double b[D / 4];
#pragma unroll
        for (int s = 0; s < D / 4; ++s) b[s] = kt[(size_t)(4 * s + kl) * Nb + cc];
#pragma unroll
        for (int s = 0; s < D / 4; s += 2) {
          acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s + 1], b[s + 1], acc1, 0, 0, 0);
        }
      }
      if (c < Nb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) srow[4 * e + kl][c] = (acc0[e] + acc1[e]) / sqrt_d;
      }
    }
  }
  __syncthreads();

  // Marks the kept blocks of tile row rr (block row r): slots for which kept(e) holds, plus
  // the forced and static blocks; a query block holding text tokens keeps every block.
  auto mark_row = [&](int rr, int r, const uint64_t (&kv)[PER], auto kept) {
    if (r >= Nb) return;
    if (r < p.n_text_blocks) {
      for (int c = lane; c < Nb; c += 64) atomicOr(&word[rr][c >> 5], 1u << (c & 31));
      return;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (kept(e)) {
        const int c = key_block(kv[e]);
        atomicOr(&word[rr][c >> 5], 1u << (c & 31));
      }
    }
    if (p.keep_diag && lane == (r & 63)) atomicOr(&word[rr][r >> 5], 1u << (r & 31));
    // text columns and the head's static pattern (none for an adaptive-only head)
    if (p.n_text_blocks > 0 || pid != 0) {
      for (int c = lane; c < Nb; c += 64) {
        const bool forced = (c < p.n_text_blocks) || static_keep(pid, prm, r, c, g.N, g.blk, Nb);
        if (forced) atomicOr(&word[rr][c >> 5], 1u << (c & 31));
      }
    }
  };

  if (p.mode == 0) {
    // Top-k ranks by the score itself: exp is increasing, so the order by P equals the
    // order by S wherever the S values differ by more than float64 rounding of P can hide
    // (a top-k boundary closer than that is a near-tie, see ambiguous rows).  The kept set
    // is every key at or above the m-th largest, found without sorting.
    const int m = min(max(p.k, 0), Nb);
    for (int t = 0; t < kRankRowsPerWave; ++t) {
      const int rr = w * kRankRowsPerWave + t;
      if (rr >= nrows) break;   // no barrier in this loop
      uint64_t kv[PER], real[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int c = lane * PER + e;
        kv[e] = c < Nb ? rank_key(srow[rr][c], c) : 0ull;
        real[e] = __ballot(c < Nb);
      }
      const uint64_t thr = m > 0 && m < Nb ? select_kth<PER>(kv, real, m) : 0ull;
      mark_row(rr, r0 + rr, kv, [&](int e) { return m > 0 && lane * PER + e < Nb && kv[e] >= thr; });
    }
  } else {
    // The mass prefix needs P itself (softmax over all key blocks of the row, whose
    // numerators replace the scores in LDS) and the rank order up to its end: the rows are
    // sorted, RI at a time.
    for (int pass = 0; pass < kRankRowsPerWave / RI; ++pass) {
      const int rr0 = w * kRankRowsPerWave + pass * RI;   // first tile row of this pass
      // a pass past the tile's rows skips its work but not the barrier
      const bool live = rr0 < nrows;
      uint64_t kv[RI][PER] = {};
      double z[RI] = {};
      if (live) {
#pragma unroll
      for (int j = 0; j < RI; ++j) {
        double* sr = srow[rr0 + j];
        double mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int c = lane * PER + e;
          if (c < Nb) mx = fmax(mx, sr[c]);
        }
        mx = wave_max(mx);
        double ex[PER], part = 0.0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int c = lane * PER + e;
          ex[e] = c < Nb ? exp(sr[c] - mx) : 0.0;
          part += ex[e];
          if (c < Nb) sr[c] = ex[e];
        }
        z[j] = wave_sum(part);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int c = lane * PER + e;
          kv[j][e] = c < Nb ? rank_key(ex[e] / z[j], c) : 0ull;
        }
      }
      rank_sort_desc<PER, RI, NP2, 2>(kv, lane);
      }
      __syncthreads();   // numerators visible to every lane
#pragma unroll
      for (int j = 0; j < RI && live; ++j) {
        const int rr = rr0 + j;
        // running mass in rank order: a sequential sum over each lane's slots, then a
        // wavefront scan of the lane totals; the first rank reaching tau ends the prefix
        double cum[PER], run = 0.0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int i = lane * PER + e;
          run += i < Nb ? srow[rr][key_block(kv[j][e])] / z[j] : 0.0;
          cum[e] = run;
        }
        double incl = run;
        for (int off = 1; off < 64; off <<= 1) {
          const double u = __shfl_up(incl, off, 64);
          if (lane >= off) incl += u;
        }
        double excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.0;
        int first = 0x7fffffff;
#pragma unroll
        for (int e = PER - 1; e >= 0; --e) {
          const int i = lane * PER + e;
          if (i < Nb && excl + cum[e] >= p.tau) first = i;
        }
        first = wave_min_int(first);
        int m = first == 0x7fffffff ? Nb : first + 1;
        if (p.k_cap > 0) m = min(m, p.k_cap);
        mark_row(rr, r0 + rr, kv[j], [&](int e) { return lane * PER + e < m; });
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < nrows * g.words; i += kRankThreads) bits[row0 * g.words + i] = word[i / g.words][i % g.words];
  if (tid < nrows) {
    int pc = 0;
    for (int x = 0; x < g.words; ++x) pc += __popc(word[tid][x]);
    count[row0 + tid] = pc;
  }
}

// ------------------------------------------------------------------ static-only rows
// One wavefront per row, 4 rows per workgroup; each pass tests 64 key blocks, one per lane,
// and a ballot gives two 32-bit words of the row.
__global__ __launch_bounds__(kThreads) void static_kernel(uint32_t* __restrict__ bits,
                                                          int32_t* __restrict__ count,
                                                          MaskGeom g, HeadTable heads, int rows) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int bh = row / g.Nb, r = row - bh * g.Nb, h = bh % g.H;
  const int pid = heads.id[h], prm = heads.param[h];
  uint32_t* out = bits + (size_t)row * g.words;
  int pc = 0;
  for (int c0 = 0; c0 < g.Nb; c0 += 64) {
    const int c = c0 + lane;
    const uint64_t m = __ballot(c < g.Nb && static_keep(pid, prm, r, c, g.N, g.blk, g.Nb));
    const int wi = (c0 >> 5) + lane;
    if (lane < 2 && wi < g.words) out[wi] = (uint32_t)(lane ? m >> 32 : m);
    pc += __popcll(m);
  }
  if (lane == 0) count[row] = pc;
}

// ------------------------------------------------------------------ CSR
// One launch builds the whole CSR (and, when asked, the processing order).  Workgroups
// 0 .. nfill-1 own kFillRows consecutive rows each: the row offset of their first row is
// the sum of every earlier row's count (all threads read a strided share, then a
// workgroup sum in a fixed order), a scan of their own counts gives row_ptr, and each
// wavefront then turns kFillRows / 16 rows' bitmasks into ascending block indices.
// Workgroups nfill .. nfill+7 build the order of one XCD range each.
constexpr int kCsrThreads = kOrderThreads;
constexpr int kFillRows = 64;
constexpr int kFillWaves = kCsrThreads / 64;
constexpr int kRowsPerFillWave = kFillRows / kFillWaves;

__global__ __launch_bounds__(kCsrThreads) void csr_kernel(const uint32_t* __restrict__ bits,
                                                          const int32_t* __restrict__ count,
                                                          int32_t* __restrict__ row_ptr,
                                                          int32_t* __restrict__ col_idx,
                                                          int32_t* __restrict__ order, int words,
                                                          int rows) {
  __shared__ OrderScratch osh;
  __shared__ int wsum[kFillWaves];
  __shared__ int start[kFillRows];
  const int nfill = (rows + kFillRows - 1) / kFillRows;
  if ((int)blockIdx.x >= nfill) {
    order_balanced([&](int i) { return count[i]; }, order, rows, (int)blockIdx.x - nfill, osh);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row0 = (int)blockIdx.x * kFillRows;
  // offset of row0: counts of rows 0 .. row0-1
  int part = 0;
  for (int i = tid; i < row0; i += kCsrThreads) part += count[i];
  part = wave_incl_sum(part);
  if (lane == 63) wsum[wv] = part;
  __syncthreads();
  if (wv == 0) {
    int base = 0;
    for (int w = 0; w < kFillWaves; ++w) base += wsum[w];
    const int cnt = row0 + lane < rows ? count[row0 + lane] : 0;   // kFillRows == 64 lanes
    const int incl = wave_incl_sum(cnt);
    start[lane] = base + incl - cnt;
    if (row0 + lane < rows) row_ptr[row0 + lane + 1] = base + incl;
    if (row0 == 0 && lane == 0) row_ptr[0] = 0;
  }
  __syncthreads();
  for (int k = 0; k < kRowsPerFillWave; ++k) {
    const int rr = wv * kRowsPerFillWave + k, row = row0 + rr;
    if (row >= rows) break;
    // 64 key blocks per pass, one per lane: lanes 0-31 test bits of word 2p, lanes 32-63
    // of word 2p+1 (read from the lanes that loaded them); a ballot and the lane's rank
    // among the set lanes place each index
    const uint32_t w = lane < words ? bits[(size_t)row * words + lane] : 0u;
    int out = start[rr];
    for (int p = 0; 2 * p < words; ++p) {
      const uint32_t w0 = (uint32_t)__builtin_amdgcn_readlane((int)w, 2 * p);
      const uint32_t w1 = (uint32_t)__builtin_amdgcn_readlane((int)w, 2 * p + 1);
      const uint32_t wl = lane < 32 ? w0 : w1;
      const bool set = (wl >> (lane & 31)) & 1u;
      const uint64_t m = __ballot(set);
      if (set) col_idx[out + __popcll(m & ((1ull << lane) - 1ull))] = 64 * p + lane;
      out += __popcll(m);
    }
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

// Rows per rank workgroup.  A launch of fewer than one 16-row workgroup per compute unit
// takes the fewest rows (down to 8) that still keep it to one workgroup per unit: the
// selection, bound by each unit's scalar issue, then has fewer rows per unit and every
// unit works.  Larger launches keep 16 (fewer workgroups reading KpT).
static int rank_rows(const MaskGeom& g) {
  const long heads = (long)g.B * g.H;
  if (heads * ((g.Nb + kRankRows - 1) / kRankRows) >= kComputeUnits) return kRankRows;
  int rows = kRankRows;
  for (int r = kRankRows - 1; r >= 8; --r)
    if (heads * ((g.Nb + r - 1) / r) <= kComputeUnits) rows = r;
  return rows;
}

template <int D>
static hipError_t launch_rank_d(const MaskGeom& g, const AdaptiveParams& p, const HeadTable& heads,
                                const MaskWorkspace& ws, hipStream_t s) {
  const int rows = rank_rows(g);
  const int tiles = (g.Nb + rows - 1) / rows;
  const dim3 grid((unsigned)(g.B * g.H * tiles)), block(rank_threads(D));
  int np2 = 64;
  while (np2 < g.Nb) np2 <<= 1;
  switch (np2) {
    case 64: hipLaunchKernelGGL((rank_kernel<D, 64>), grid, block, 0, s, ws.qp, ws.kpt, ws.bits, ws.count, g, p, heads, rows); break;
    case 128: hipLaunchKernelGGL((rank_kernel<D, 128>), grid, block, 0, s, ws.qp, ws.kpt, ws.bits, ws.count, g, p, heads, rows); break;
    case 256: hipLaunchKernelGGL((rank_kernel<D, 256>), grid, block, 0, s, ws.qp, ws.kpt, ws.bits, ws.count, g, p, heads, rows); break;
    case 512: hipLaunchKernelGGL((rank_kernel<D, 512>), grid, block, 0, s, ws.qp, ws.kpt, ws.bits, ws.count, g, p, heads, rows); break;
    default: hipLaunchKernelGGL((rank_kernel<D, 1024>), grid, block, 0, s, ws.qp, ws.kpt, ws.bits, ws.count, g, p, heads, rows); break;
  }
  return hipGetLastError();
}

hipError_t launch_rank(const MaskGeom& g, const AdaptiveParams& p, const HeadTable& heads,
                       const MaskWorkspace& ws, hipStream_t s) {
  return g.d == 128 ? launch_rank_d<128>(g, p, heads, ws, s) : launch_rank_d<64>(g, p, heads, ws, s);
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
  const int nfill = (rows + kFillRows - 1) / kFillRows;
  hipLaunchKernelGGL(csr_kernel, dim3((unsigned)(nfill + (order ? kXcds : 0))), dim3(kCsrThreads), 0, s, ws.bits,
                     ws.count, row_ptr, col_idx, order, g.words, rows);
  return hipGetLastError();
}

}  // namespace asa
