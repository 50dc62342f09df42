// Internal declarations shared by the host API and the HIP kernels of the
// lightning-indexer scoring library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/idx_logits.h"

namespace idx {

// ---------------------------------------------------------------------------
// Plan layout (device memory, 256-byte aligned sections)
//
//   PlanHeader                      (256 B)
//   int32 win_start[B*S_q]          window start per row
//   int32 win_end[B*S_q]            window end per row
//   int32 slot_row[n_tiles*tile_rows]  global row (b*S_q+i) of every tile slot,
//                                   -1 for the padding slots of a ragged tail;
//                                   with explicit windows the rows of every
//                                   kSortRows-row segment are reordered so that
//                                   rows with alike windows share tiles
//   int32 tile_lo[n_tiles]          first column computed for the tile
//   int32 tile_hi[n_tiles]          one past the last column computed
//   int32 tile_order[n_seg*tps]     per sort segment g (tps = kSortRows /
//                                   tile_rows slots each), the segment's
//                                   tiles by descending cost (covered columns
//                                   x rows), then -1 for the missing tiles of
//                                   a batch's last, partial segment
//
// A tile is tile_rows consecutive slots of one batch.  [tile_lo,
// tile_hi) is the union of its rows' windows widened to kColAlign columns
// and clipped to [0, S_k); cells of a row outside it are cleanup work.
// A tile always holds 512 (row, head) pairs, so tile_rows = 512 / H: 8 rows
// at 64 heads, 16 at 32, 32 at 16, 64 at 8.
// ---------------------------------------------------------------------------
constexpr uint32_t kPlanMagic = 0x50584449u;  // "IDXP"
constexpr int kTileRows = 8;                   // query rows per tile at 64 heads
constexpr int kColAlign = 32;                  // coverage granularity in columns
constexpr int kSortRows = 1024;                // rows ordered together when building a plan
constexpr int kSortThreads = 256;
static_assert(kSortRows % 64 == 0, "sort segments hold whole tiles at every head count");

// Query heads per row the kernels are built for, and the tile height for each.
__host__ __device__ constexpr bool supported_heads(int H) { return H == 8 || H == 16 || H == 32 || H == 64; }
__host__ __device__ constexpr int tile_rows_for(int H) { return supported_heads(H) ? 512 / H : 0; }

struct PlanHeader {
  uint32_t magic;
  int32_t B, S_q, S_k, H, D;
  int32_t n_tiles, tile_rows;
  int32_t reserved[56];
};
static_assert(sizeof(PlanHeader) == 256, "plan header is one 256-byte section");

struct PlanLayout {
  size_t off_start, off_end, off_slot, off_lo, off_hi, off_order, total;
  int64_t n_rows, n_tiles, n_seg;
  int32_t tile_rows, tiles_per_seg;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline int64_t tiles_per_batch(int64_t S_q, int64_t tile_rows) {
  return (S_q + tile_rows - 1) / tile_rows;
}

// Workgroups that build a plan: one per kSortRows rows of a batch.
__host__ __device__ inline int64_t plan_segments(int64_t B, int64_t S_q) {
  return B * ((S_q + kSortRows - 1) / kSortRows);
}

// Layout of a plan for H heads; total == 0 when the sizes overflow or H is
// not supported.  The window arrays do not depend on H.
inline PlanLayout plan_layout(int64_t B, int64_t S_q, int H) {
  PlanLayout L{};
  L.tile_rows = tile_rows_for(H);
  if (L.tile_rows == 0 || B <= 0 || S_q <= 0) return L;
  L.n_rows = B * S_q;
  L.n_tiles = B * tiles_per_batch(S_q, L.tile_rows);
  if (L.n_rows > (int64_t(1) << 31) - 1 || L.n_tiles * L.tile_rows > (int64_t(1) << 31) - 1) return L;
  size_t off = align256(sizeof(PlanHeader));
  L.off_start = off;
  off += align256(size_t(L.n_rows) * 4);
  L.off_end = off;
  off += align256(size_t(L.n_rows) * 4);
  L.off_slot = off;
  off += align256(size_t(L.n_tiles) * L.tile_rows * 4);
  L.off_lo = off;
  off += align256(size_t(L.n_tiles) * 4);
  L.off_hi = off;
  off += align256(size_t(L.n_tiles) * 4);
  L.n_seg = plan_segments(B, S_q);
  L.tiles_per_seg = kSortRows / L.tile_rows;
  L.off_order = off;
  off += align256(size_t(L.n_seg) * L.tiles_per_seg * 4);
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Weighted-query pieces (FP8, MXFP8 and MXFP4 inputs)
//
// Those formats score with ReLU(x) = (x + |x|) / 2:
//   sum_h w_h ReLU(S_h) = ( sum_h w_h |S_h| + qt . k ) / 2,  qt = sum_h w_h q_h,
// so the epilogue needs one FMA (with |.| as a free source modifier) per head
// instead of a max and an FMA, and the linear term qt . k comes from MFMA
// blocks of its own.  qt (fp32) is written as pieces with one E8M0 scale per
// 32 elements, each piece encoding the exact fp32 residual of the ones before
// it:
//  - FP8 / MXFP8: kPieces e4m3 rows (128 B); each shrinks the residual's block
//    maximum 16-fold, so they sum to qt within 2^-16 of its block maxima (the
//    scoring kernel's 16x16 linear blocks hold four pieces per row);
//  - MXFP4: kPiecesE2M1 e2m1 rows (64 B, packed like MXFP4 Q), so the linear
//    block multiplies e2m1 by e2m1 at the fp4 rate; with the block maximum
//    scaled into [2, 4) each piece shrinks it at least 4-fold, 2^-16 in all.
// Each row has kPieceRowBytes of pieces and kPieceSlots scale words in the
// workspace (WorkspaceLayout below).
// ---------------------------------------------------------------------------
constexpr int kPieces = 4;
constexpr int kPiecesE2M1 = 8;
constexpr int kPieceSlots = 8;        // scale words reserved per row
constexpr int kPieceRowBytes = 768;   // piece bytes reserved per row
template <int F>
struct PieceFmt {
  static constexpr int N = F == IDX_IN_MXFP4_E2M1 ? kPiecesE2M1 : kPieces;   // pieces per row
  static constexpr int BYTES = F == IDX_IN_MXFP4_E2M1 ? 64 : 128;           // bytes per piece
  static constexpr int SLOTS = F == IDX_IN_MXFP4_E2M1 ? kPieceSlots : kPieces;  // scale words per row
  static_assert(N * BYTES <= kPieceRowBytes && SLOTS <= kPieceSlots && N <= 8, "pieces fit their row");
};

// ---------------------------------------------------------------------------
// Kernel formats
//
// The scoring kernels are instantiated per kernel format: the input format
// itself, or kInBF16RowScale.  With accumulate = IDX_ACCUM_FP32, FP8 and MXFP8
// inputs are converted by the preparation into bf16 operands, exactly (an
// e4m3 value has four significant bits; an MX block scale is a power of two
// folded into the value), and scored on the bf16 matrix core, whose products
// and sums keep fp32 precision: MXFP8 then runs the BF16 kernels, FP8 the
// BF16 kernels with its per-row K scale applied after the head-sum
// (kInBF16RowScale).  The e4m3 matrix core sums each group of eight products
// aligned to the group's largest with about 13 fraction bits (measured), which
// the native path accepts for its speed.
// ---------------------------------------------------------------------------
constexpr int kInBF16RowScale = 4;

struct Exec {
  int kf;        // kernel format: an idx_in_t or kInBF16RowScale
  bool convert;  // Q and K converted to bf16 by the preparation
};
inline Exec exec_of(idx_in_t f, int32_t accumulate) {
  if (accumulate == IDX_ACCUM_FP32 && (f == IDX_IN_FP8_E4M3 || f == IDX_IN_MXFP8_E4M3))
    return Exec{f == IDX_IN_FP8_E4M3 ? kInBF16RowScale : int(IDX_IN_BF16), true};
  return Exec{int(f), false};
}
__host__ __device__ constexpr bool bf16_operands(int kf) { return kf == IDX_IN_BF16 || kf == kInBF16RowScale; }

// Only the 64-head kernels of the narrow formats take the linear term from
// pieces; the others use max + FMA.
inline bool uses_pieces(int kf, int H) { return !bf16_operands(kf) && H == 64; }

// ---------------------------------------------------------------------------
// K in fragment order
//
// The scoring kernel feeds K to the MFMAs as B operands, 32 key rows at a
// time; lane (c, g) needs 16-byte chunks of row c at format-specific offsets.
// Read straight from [S_k, D] rows, every such load touches 32 cache lines.
// Each call therefore first copies K into fragment order: block u (rows
// 32u..32u+31) is ROWB*32 contiguous bytes, chunk v of lane l = c + 32g at
// u*32*ROWB + v*1024 + l*16, so each fragment load is 1 KB contiguous.  The
// last block is zero-padded.
// ---------------------------------------------------------------------------
// Formats with a per-K-row scale also get it in block order: for block u,
// 64 words, lane l's word being that of column 32u + l%32 as lane half l/32
// of the scoring kernel uses it (MX: the int32 word shifted right by 8 or 16
// bits for lane half 1, so that op_sel picks the right E8M0 byte; FP8: the
// fp32 scale).  Columns past S_k get 0.
inline bool has_kscale(int kf) { return kf != IDX_IN_BF16; }

// Where lane half g of the scoring kernel holds K row bytes: 16-byte chunk v
// at CBASE * g + CSTRIDE * v (ROWB bytes per row); SHIFT is the right shift of
// an MX scale word for lane half 1.  The reorder writes K in this placement,
// and the scoring kernel's operand formats are checked against it.
template <int F>
struct KLayout;
template <>
struct KLayout<IDX_IN_BF16> {
  static constexpr int ROWB = 256, CBASE = 128, CSTRIDE = 16, SHIFT = 0;
};
template <>
struct KLayout<kInBF16RowScale> {
  static constexpr int ROWB = 256, CBASE = 128, CSTRIDE = 16, SHIFT = 0;
};
template <>
struct KLayout<IDX_IN_FP8_E4M3> {
  static constexpr int ROWB = 128, CBASE = 16, CSTRIDE = 32, SHIFT = 0;
};
template <>
struct KLayout<IDX_IN_MXFP8_E4M3> {
  static constexpr int ROWB = 128, CBASE = 16, CSTRIDE = 32, SHIFT = 8;
};
template <>
struct KLayout<IDX_IN_MXFP4_E2M1> {
  static constexpr int ROWB = 64, CBASE = 32, CSTRIDE = 16, SHIFT = 16;
};

// bytes of one K (or Q head) row of 128 elements as the kernels read it
inline int row_bytes_of(int kf) {
  return bf16_operands(kf) ? 256 : (kf == IDX_IN_MXFP4_E2M1 ? 64 : 128);
}

// Workspace of one call (256-byte aligned sections, in this order):
//   [pieces, piece scales]        64-head calls of the narrow formats
//   [Q converted to bf16]         calls that convert (Exec::convert)
//   [K in fragment order]
//   [K scales in block order]     every kernel format but BF16
//   [plan]                        only when the call builds it
// A call given a plan needs only the first `planned` bytes.
struct WorkspaceLayout {
  size_t off_pieces, off_pscales, off_qconv, off_kfrag, off_kscale, off_plan, planned, total;
};

inline WorkspaceLayout workspace_layout(const Exec& x, int64_t B, int64_t S_q, int64_t S_k, int H) {
  WorkspaceLayout W{};
  const PlanLayout L = plan_layout(B, S_q, H);
  if (L.total == 0 || S_k <= 0) return W;
  size_t off = 0;
  if (uses_pieces(x.kf, H)) {
    W.off_pieces = off;
    off += align256(size_t(L.n_rows) * kPieceRowBytes);
    W.off_pscales = off;
    off += align256(size_t(L.n_rows) * kPieceSlots * 4);
  }
  if (x.convert) {
    W.off_qconv = off;
    off += align256(size_t(L.n_rows) * size_t(H) * 256);
  }
  W.off_kfrag = off;
  off += align256(size_t(B) * size_t((S_k + 31) / 32) * 32 * row_bytes_of(x.kf));
  if (has_kscale(x.kf)) {
    W.off_kscale = off;
    off += align256(size_t(B) * size_t((S_k + 31) / 32) * 64 * 4);
  }
  W.planned = off;
  W.off_plan = off;
  off += L.total;
  W.total = off;
  return W;
}

// Unsigned 32-bit division by a divisor fixed per launch, as one 64 x 64-bit
// high multiply (Lemire, Kaser and Kurz, "Faster remainder by direct
// computation", 2019: with M = floor((2^64 - 1) / d) + 1, n / d is the high
// word of M * n for every 32-bit n and d >= 2).
struct FastDiv {
  uint64_t M;
  uint32_t d;
  static FastDiv make(uint32_t d) { return FastDiv{d > 1 ? ~uint64_t(0) / d + 1 : 0, d}; }
  __device__ __forceinline__ uint32_t div(uint32_t n) const { return d > 1 ? uint32_t(__umul64hi(M, n)) : n; }
};

// ---------------------------------------------------------------------------
// Fused top-k selection (idx_logits_run_topk)
//
// Scores become 32-bit rank keys whose unsigned order is the ranking of the
// selection: larger scores first, +0 and -0 equal, NaN below every number.
// A call then
//  1. scores a sample first: every kSampleStride-th block of 32 keys (blocks
//     0, R, 2R, ...), as sample columns j' = 32 (j / 32R) + min(j % 32R, 32)
//     of key j (sample_col), so a window [s, e) of keys is the window
//     [sample_col(s), sample_col(e)) of the sample;
//  2. takes a threshold per row, the key of the m-th best sampled score in
//     its window with its low 16 bits cleared, m about 1.25 k / R plus a
//     margin (0, every cell, when the window holds at most k keys or the
//     sample is too small to say);
//  3. scores every cell in select mode: a cell of a row's window whose key
//     is at least the row's threshold is appended, as (score bits, column),
//     to the row's candidate area; the unit of columns [c0, c1) writes its
//     candidates in column order from slot c0 of the row on, and (c0, count)
//     to the row's entry for its chunk;
//  4. selects the top k of every row from its candidates, which are exactly
//     the cells ranked above the threshold; a row with fewer candidates than
//     min(k, window) gets threshold 0 and goes through 3 and 4 once more, so
//     the result never depends on the sample.
// ---------------------------------------------------------------------------
constexpr int kSampleStride = 16;
constexpr uint32_t kTauNone = 0xFFFFFFFFu;  // threshold no key reaches: the row keeps nothing

__host__ __device__ inline int64_t sample_col(int64_t j) {
  const int64_t span = 32 * int64_t(kSampleStride);
  const int64_t r = j % span;
  return (j / span) * 32 + (r < 32 ? r : 32);
}

// Rank key of a score's fp32 bits (bf16 scores widened): negative scores map
// to -bits as an unsigned (so -0 lands on +0's key 0x80000000), others get the
// top bit set, NaN gets 0.
__device__ __forceinline__ uint32_t rank_key(uint32_t u) {
  const uint32_t neg = uint32_t(int32_t(u) >> 31);
  const uint32_t k = ((u ^ neg) - neg) ^ (~neg & 0x80000000u);
  return __builtin_isnan(__uint_as_float(u)) ? 0u : k;
}

// A threshold key (rank_key order) as a float compare: a score reaches key
// tau exactly when it is a number >= tau_value(tau) (rank keys of numbers
// order like the numbers, +0 and -0 alike), or when tau is 0, which keeps NaN
// too; kTauNone gives NaN, which no score reaches.
__device__ __forceinline__ float tau_value(uint32_t tau) {
  if (tau == kTauNone) return __builtin_nanf("");
  if (tau == 0u) return -__builtin_inff();
  return __uint_as_float((tau >> 31) ? (tau & 0x7FFFFFFFu) : (0u - tau));
}

// Extra workspace of a fused top-k call, after the sections of the scoring
// call itself (WorkspaceLayout, plan included), 256-byte aligned:
//   [sampled K in fragment order]   B x ceil(nblk / R) blocks
//   [sampled K scales]              (not BF16)
//   [sample plan]                   plan_layout(B, S_q, H).total
//   [sample scores]                 n_rows x S_ks, fp32 or bf16
//   [thresholds, redo list, big-row list]  n_rows x 4 each
//   [gate]                          256 B: counts of the two lists
//   [chunk entries]                 n_rows x n_chunk_max x (c0, count)
//   [candidates]                    n_rows x S_k x (score bits, column)
struct TopkLayout {
  WorkspaceLayout base;
  size_t off_skfrag, off_skscale, off_splan, off_sscore, off_tau, off_redo, off_big, off_gate, off_meta, off_cand, total;
  int64_t S_ks, nblk_s;
  int32_t n_chunk_max;
};

constexpr int kDynUnitTiles = 256;

// Everything a scoring kernel needs, passed by value.
struct ScoreArgs {
  const void* q;
  const void* q_scale;
  const void* w;
  void* out;
  const unsigned char* plan;
  int64_t ld;  // output row stride in elements
  float sm_scale;
  int32_t B, S_q, S_k, H;
  int32_t n_tiles, tiles_per_batch, tile_rows;
  // Work positions, one per workgroup (blockIdx.x), which the hardware
  // deals out in order:
  //   [0, n_pos_compute)          chunk p % n_chunk of slot p / n_chunk
  //   [n_pos_compute, n_positions) cleanup of tile p - n_pos_compute
  // Slots walk the plan's tiles from the last batch to the first, each
  // batch's sort segments from its last to its first (its last segment
  // holds last_seg_tiles tiles, the others tiles_per_seg), and each segment's
  // tiles in the plan's cost order: costliest first globally under causal
  // windows (later rows see more keys), and in every segment otherwise, so
  // the work dealt out last is short.  A tile's coverage [lo, hi)
  // is cut into n_chunk equal chunks, multiples of 64 columns and at least
  // min_chunk wide.
  int32_t min_chunk, n_chunk;
  int32_t seg_per_batch, tiles_per_seg, last_seg_tiles;
  // 64-head calls with at most two query rows per batch (decode): every
  // wave of a unit scores the tile's two rows over a quarter of its columns,
  // instead of three of its four waves holding padding rows only
  int32_t wave_split;
  // Decode-sized calls of at most kDynUnitTiles tiles (one per batch): the
  // units are not n_chunk per tile but chunks of one width for every tile,
  // the width set in the kernel from the tiles' total coverage so that they
  // number at most n_pos_compute; positions past them are empty
  int32_t dyn_units;
  int32_t n_pos_compute, n_positions;
  uint32_t off_start, off_end, off_slot, off_lo, off_hi, off_order;
  const unsigned char* pieces;   // per row PieceFmt<F>::N pieces of PieceFmt<F>::BYTES (formats with pieces)
  const uint32_t* pscales;       // per row PieceFmt<F>::SLOTS E8M0 words
  const unsigned char* kfrag;    // K in fragment order, [B][ceil(S_k/32)][32 * ROWB]
  const uint32_t* kscale;        // K scales in block order, [B][ceil(S_k/32)][64] (not BF16)
  // Paged keys read straight from the cache (pages of 32 * 2^bpp_shift rows,
  // cache under 2 GiB): block u of request b is rows [32 (u % bpp), +32) of
  // page btable[b][u / bpp], bpp = 2^bpp_shift; kfrag / kscale are then unused.
  const unsigned char* kcache;   // [num_pages][page_size][ROWB]
  const uint32_t* kscache;       // [num_pages][page_size] (not BF16)
  const int32_t* btable;         // [B][max_pages]
  int32_t num_pages, page_size, max_pages, bpp_shift;
  // Select mode (fused top-k) when cand is set: no score is stored (out is
  // unused, no cleanup positions); row r keeps the cells of its window whose
  // rank key is at least tau[r] as (score bits, column) pairs at
  // cand + 8 (r S_k + c0 + i), and writes (c0, count) to meta[2 (r n_chunk +
  // chunk)].  With gate set, the launch does nothing while *gate is 0.
  unsigned char* cand;
  int32_t* meta;
  const uint32_t* tau;
  const int32_t* gate;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_plan(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* offsets,
                       const int32_t* starts, const int32_t* ends, void* plan, hipStream_t stream);
hipError_t launch_copy_windows(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                               int32_t* ws, int32_t* we, hipStream_t stream);
// Plan of packed variable-length rows over ratio-compressed keys (B = 1).
hipError_t launch_plan_thd(int32_t n_seg, const int32_t* cu_q, const int32_t* cu_k, int32_t ratio, int32_t T_q,
                           int32_t m_total, int32_t H, int32_t D, void* plan, hipStream_t stream);

// Plan of paged calls: windows from the requests' context lengths.
hipError_t launch_plan_paged(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* ctx,
                             void* plan, hipStream_t stream);

// What a call that builds its own plan passes to the preparation launch.
struct PlanBuild {
  int32_t B, S_q, S_k, H, D;
  const int32_t* offsets;
  const int32_t* starts;
  const int32_t* ends;
  const int32_t* ctx;  // paged calls: context lengths (offsets / starts / ends then NULL)
  unsigned char* plan;
};

// Where the preparation reads K when it comes from a paged cache.
struct PagedK {
  const unsigned char* k_cache;
  const uint32_t* k_scale_cache;
  const int32_t* block_table;
  const int32_t* ctx;
  int32_t num_pages, page_size, max_pages;
  bool skip_gather;  // the scoring kernel reads the cache itself: no K copy
};

// K in fragment order, K scales in block order (not for BF16), the
// weighted-query pieces when `pieces` is given, and the plan when `build` is
// given, in one launch.
// With convert, Q (n_rows x H heads) is written to qconv as bf16 and K to
// kfrag in the bf16 fragment order, exactly, MX block scales folded in.
hipError_t launch_prepare(idx_in_t fmt, bool convert, int H, idx_fp_t w_dtype, const void* k, const void* k_scale,
                          int64_t B, int64_t S_k, unsigned char* kfrag, uint32_t* kscale, const void* q,
                          const void* q_scale, const void* w, int64_t n_rows, unsigned char* pieces,
                          uint32_t* pscales, uint16_t* qconv, const PlanBuild* build,
                          const PagedK* paged, hipStream_t stream);
// Top-k selection over the scores a call wrote (topk.hip): for each of the
// plan's rows, the k <= kMaxTopK best columns of its window, by column or in
// rank order.
constexpr int kMaxTopK = 2048;
hipError_t launch_topk(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                       const void* logits, bool logits_bf16, int64_t ld, int32_t k, bool by_score,
                       int32_t* out_idx, float* out_val, hipStream_t stream);

// Fused top-k steps (topk_fused.hip), in launch order around the scoring
// launches.  The sample plan, sampled K, thresholds and the rest live in the
// call's workspace at the offsets of T (ws is its base).
// Sample plan from plan, sampled K blocks, gate = 0.
hipError_t launch_fused_setup(const TopkLayout& T, int kf, int32_t B, int32_t S_q, int32_t S_k, int32_t H,
                              const unsigned char* plan, unsigned char* ws, hipStream_t stream);
// Per row: threshold from the sample scores, chunk entries 0.
hipError_t launch_threshold(const TopkLayout& T, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t k,
                            bool scores_bf16, int32_t n_chunk, const unsigned char* plan, unsigned char* ws,
                            hipStream_t stream);
// Per row: the top k of the candidates (pass 1: every row; rows short of
// candidates get threshold 0 and join the redo list, whose length gate[0]
// gates the second scoring launch; pass 2: the rows of the redo list, and
// *n_redo = gate[0] when n_redo is set).
hipError_t launch_select(const TopkLayout& T, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, int32_t k,
                         bool by_score, int32_t n_chunk, int pass, const unsigned char* plan, unsigned char* ws,
                         int32_t* out_idx, float* out_val, int32_t* n_redo, hipStream_t stream);

hipError_t launch_score_bf16(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                             hipStream_t stream);
hipError_t launch_score_fp8(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                            hipStream_t stream);
hipError_t launch_score_mxfp8(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                              hipStream_t stream);
hipError_t launch_score_mxfp4(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                              hipStream_t stream);
hipError_t launch_score_bf16rs(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                               hipStream_t stream);

}  // namespace idx
