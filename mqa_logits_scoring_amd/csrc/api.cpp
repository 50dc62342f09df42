// Host side of the C ABI: argument validation (all of it before any launch),
// plan construction, work decomposition and kernel dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

// Workspace of idx_logits_run_noalloc: one array per device, allocated with
// the library's code object on each device it runs on and held until the
// process ends.  In host code `scratch` names a host-side stand-in, never a
// device address: the device address comes from hipGetSymbolAddress, once per
// device (scratch_on_device below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "no error";

idx_status_t fail(idx_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

idx_status_t check_dims(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D) {
  if (B <= 0 || S_q <= 0 || S_k <= 0 || H <= 0 || D <= 0)
    return fail(IDX_E_INVALID, "dimensions must be positive (B=%d S_q=%d S_k=%d H=%d D=%d)", B, S_q, S_k, H, D);
  if (!idx::supported_heads(H) || D != 128)
    return fail(IDX_E_UNSUPPORTED, "H must be 8, 16, 32 or 64 query heads and D must be 128 (got H=%d D=%d)", H, D);
  const idx::PlanLayout L = idx::plan_layout(B, S_q, H);
  if (L.total == 0) return fail(IDX_E_INVALID, "B*S_q=%lld rows is too large", (long long)B * S_q);
  return IDX_OK;
}

// Work split (ScoreArgs): every tile's coverage is cut on the device into
// n_chunk equal chunks of at least kMinChunk columns, one unit each.  Each
// unit loads its rows' whole Q before its first MFMA, so units should be
// long; but the resident workgroups need enough of them (about four per CU)
// to stay fed, and tiles of very different coverage (irregular windows)
// balance only when no unit is much longer than kChunkCols.
constexpr int64_t kUnitsPerCu = 4;
constexpr int64_t kChunkCols = 16384;
constexpr int64_t kMinChunk = 256;
// CUs the split is sized against in host-side bounds (more than any device has).
constexpr int64_t kMaxCus = 4096;

int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

// S_q and tile_rows: when a batch has fewer query rows than a tile, the waves
// holding only padding rows idle, so more units keep the CUs fed.
// units_per_cu: a sample scoring launch (fused top-k), whose units are short
// anyway, takes one round of units (two workgroups per CU).
int32_t pick_chunks(int64_t S_k, int64_t n_tiles, int64_t S_q, int64_t tile_rows, int64_t cus,
                    int64_t units_per_cu = kUnitsPerCu) {
  const int64_t span = cdiv(S_k, idx::kColAlign) * idx::kColAlign;  // widest tile coverage
  const int64_t rows_per_wave = tile_rows / 4;
  const int64_t rows = S_q < tile_rows ? S_q : tile_rows;
  const int64_t active = cdiv(rows, rows_per_wave);  // waves of a tile with a real row
  const int64_t target = units_per_cu * cus * 4 / active;
  int64_t want = std::max(cdiv(target, n_tiles), cdiv(span, kChunkCols));
  want = std::min(want, cdiv(span, kMinChunk));
  return int32_t(std::max<int64_t>(want, 1));
}

// Work positions: every chunk of every tile, then one cleanup unit per tile
// (the most a launch takes: the FP8-family, one-row BF16 and 8-32-head
// kernels clean their own rows and launch no cleanup units).
int64_t positions_of(const idx::PlanLayout& L, int64_t n_chunk) { return L.n_tiles * (n_chunk + 1); }

// CUs of the current device, looked up once per device.
hipError_t device_cus(int& cus) {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  if (cache[dev] == 0) {
    int c = 0;
    if ((e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    cache[dev] = c > 0 ? c : 1;
  }
  cus = cache[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t idx_abi_version(void) { return IDX_ABI_VERSION; }

const char* idx_last_error(void) { return g_err; }

size_t idx_logits_plan_bytes(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D) {
  if (B <= 0 || S_q <= 0 || S_k <= 0 || H <= 0 || D <= 0) return 0;
  return idx::plan_layout(B, S_q, H).total;
}

idx_status_t idx_logits_plan(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                             const int32_t* q_causal_offsets, const int32_t* row_starts, const int32_t* row_ends,
                             void* plan, size_t plan_bytes, void* stream) {
  idx_status_t st = check_dims(B, S_q, S_k, H, D);
  if (st != IDX_OK) return st;
  if ((row_starts == nullptr) != (row_ends == nullptr))
    return fail(IDX_E_INVALID, "row_starts and row_ends must be given together");
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "plan buffer is NULL");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan buffer must be 256-byte aligned");
  const size_t need = idx::plan_layout(B, S_q, H).total;
  if (plan_bytes < need)
    return fail(IDX_E_WORKSPACE, "plan buffer has %zu bytes, %zu needed", plan_bytes, need);
  hipError_t e = idx::launch_plan(B, S_q, S_k, H, D, q_causal_offsets, row_starts, row_ends, plan,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(IDX_E_HIP, "plan launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

idx_status_t idx_logits_plan_thd(int32_t n_seg, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t ratio, int32_t T_q, int32_t m_total, int32_t H, int32_t D, void* plan,
                                 size_t plan_bytes, void* stream) {
  idx_status_t st = check_dims(1, T_q, m_total, H, D);
  if (st != IDX_OK) return st;
  if (n_seg <= 0) return fail(IDX_E_INVALID, "n_seg must be positive (got %d)", n_seg);
  if (ratio <= 0) return fail(IDX_E_INVALID, "ratio must be positive (got %d)", ratio);
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)
    return fail(IDX_E_INVALID, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "plan buffer is NULL");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan buffer must be 256-byte aligned");
  const size_t need = idx::plan_layout(1, T_q, H).total;
  if (plan_bytes < need) return fail(IDX_E_WORKSPACE, "plan buffer has %zu bytes, %zu needed", plan_bytes, need);
  hipError_t e = idx::launch_plan_thd(n_seg, cu_seqlens_q, cu_seqlens_k, ratio, T_q, m_total, H, D, plan,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(IDX_E_HIP, "plan launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

static idx::WorkspaceLayout layout_of(const idx_logits_args_t* a) {
  if (a == nullptr || a->B <= 0 || a->S_q <= 0 || a->S_k <= 0 || a->H <= 0 || a->D <= 0) return {};
  const idx_in_t f = a->in_dtype;
  if (f != IDX_IN_BF16 && f != IDX_IN_FP8_E4M3 && f != IDX_IN_MXFP8_E4M3 && f != IDX_IN_MXFP4_E2M1) return {};
  if (a->accumulate != IDX_ACCUM_NATIVE && a->accumulate != IDX_ACCUM_FP32) return {};
  return idx::workspace_layout(idx::exec_of(f, a->accumulate), a->B, a->S_q, a->S_k, a->H);
}

size_t idx_logits_workspace_bytes(const idx_logits_args_t* a) { return layout_of(a).total; }

size_t idx_logits_workspace_bytes_planned(const idx_logits_args_t* a) { return layout_of(a).planned; }

idx_status_t idx_logits_plan_windows(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                                     int32_t* win_start, int32_t* win_end, void* stream) {
  idx_status_t st = check_dims(B, S_q, S_k, H, D);
  if (st != IDX_OK) return st;
  if (plan == nullptr || win_start == nullptr || win_end == nullptr)
    return fail(IDX_E_INVALID, "plan, win_start and win_end must be non-NULL");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  if ((reinterpret_cast<uintptr_t>(win_start) & 3u) != 0 || (reinterpret_cast<uintptr_t>(win_end) & 3u) != 0)
    return fail(IDX_E_INVALID, "win_start and win_end must be 4-byte aligned");
  hipError_t e = idx::launch_copy_windows(plan, B, S_q, S_k, H, D, win_start, win_end,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(IDX_E_HIP, "window copy launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

}  // extern "C"

namespace {

// Every check on the call's arguments; nothing is launched before they pass.
// With keys_elsewhere (paged calls, which take their keys from an
// idx_paged_k_t, and scoring from a prepared workspace) a->k and a->k_scale
// are not used.
// With no_out (fused top-k calls) a->out, out_row_stride and clean_logits
// are not used.
idx_status_t check_args(const idx_logits_args_t* a, bool keys_elsewhere = false, bool no_out = false) {
  if (a == nullptr) return fail(IDX_E_INVALID, "args is NULL");
  idx_status_t st = check_dims(a->B, a->S_q, a->S_k, a->H, a->D);
  if (st != IDX_OK) return st;
  const idx_in_t f = a->in_dtype;
  if (f != IDX_IN_BF16 && f != IDX_IN_FP8_E4M3 && f != IDX_IN_MXFP8_E4M3 && f != IDX_IN_MXFP4_E2M1)
    return fail(IDX_E_INVALID, "unknown in_dtype %d", int(f));
  if ((a->w_dtype != IDX_F32 && a->w_dtype != IDX_BF16) || (a->out_dtype != IDX_F32 && a->out_dtype != IDX_BF16))
    return fail(IDX_E_INVALID, "w_dtype and out_dtype must be IDX_F32 or IDX_BF16");
  if (a->accumulate != IDX_ACCUM_NATIVE && a->accumulate != IDX_ACCUM_FP32)
    return fail(IDX_E_INVALID, "accumulate must be IDX_ACCUM_NATIVE or IDX_ACCUM_FP32 (got %d)", int(a->accumulate));
  const bool mx = f == IDX_IN_MXFP8_E4M3 || f == IDX_IN_MXFP4_E2M1;
  if (a->q == nullptr || (!keys_elsewhere && a->k == nullptr) || a->w == nullptr || (!no_out && a->out == nullptr))
    return fail(IDX_E_INVALID, no_out ? "q, k and w must be non-NULL" : "q, k, w and out must be non-NULL");
  if (mx && a->q_scale == nullptr) return fail(IDX_E_INVALID, "MX formats need q_scale");
  if (!keys_elsewhere && (mx || f == IDX_IN_FP8_E4M3) && a->k_scale == nullptr)
    return fail(IDX_E_INVALID, "FP8 and MX formats need k_scale");
  if (!aligned16(a->q) || (!keys_elsewhere && !aligned16(a->k)) || !aligned16(a->w) || (!no_out && !aligned16(a->out)) ||
      (mx && !aligned16(a->q_scale)) || (!keys_elsewhere && (mx || f == IDX_IN_FP8_E4M3) && !aligned16(a->k_scale)))
    return fail(IDX_E_INVALID, "q, k, w, out and scale pointers must be 16-byte aligned");
  const int64_t rows = int64_t(a->B) * a->S_q;
  if (no_out) {
    if (rows * a->S_k > (int64_t(1) << 40))
      return fail(IDX_E_INVALID, "%lld rows x %d keys is too large", (long long)rows, a->S_k);
  } else {
    if (a->out_row_stride < a->S_k)
      return fail(IDX_E_INVALID, "out_row_stride %lld < S_k %d", (long long)a->out_row_stride, a->S_k);
    if (a->out_row_stride > (int64_t(1) << 40) || rows * a->out_row_stride > (int64_t(1) << 40))
      return fail(IDX_E_INVALID, "output of %lld rows x stride %lld elements is too large", (long long)rows,
                  (long long)a->out_row_stride);
  }
  if (!isfinite(a->sm_scale)) return fail(IDX_E_INVALID, "sm_scale must be finite");
  const idx::Exec x = idx::exec_of(f, a->accumulate);
  if ((int64_t(a->S_k) + 31) / 32 * 32 * idx::row_bytes_of(x.kf) > (int64_t(1) << 31) - 1)
    return fail(IDX_E_UNSUPPORTED, "S_k=%d is too long: one batch's K must stay under 2 GiB", a->S_k);
  const idx::PlanLayout L = idx::plan_layout(a->B, a->S_q, a->H);
  if (L.total > 0xFFFFFFFFull) return fail(IDX_E_INVALID, "plan too large");
  // decode-sized calls (at most two rows per batch at 64 heads) cut units of
  // at least kMinChunk columns; the others as pick_chunks
  const int64_t max_chunks = a->H == 64 && a->S_q <= idx::kTileRows / 4
                                 ? cdiv(int64_t(a->S_k) + idx::kColAlign - 1, kMinChunk)
                                 : pick_chunks(a->S_k, L.n_tiles, a->S_q, L.tile_rows, kMaxCus);
  if (positions_of(L, max_chunks) > (int64_t(1) << 31) - 1)
    return fail(IDX_E_INVALID, "problem too large for one grid");
  return IDX_OK;
}

// The paged key descriptor of a call (after check_args(a, true) passed).
idx_status_t check_paged(const idx_logits_args_t* a, const idx_paged_k_t* kv) {
  if (kv == nullptr) return fail(IDX_E_INVALID, "paged key descriptor is NULL");
  const idx_in_t f = a->in_dtype;
  const bool scaled = idx::has_kscale(f);
  if (kv->k_cache == nullptr || kv->block_table == nullptr || kv->context_lens == nullptr ||
      (scaled && kv->k_scale_cache == nullptr))
    return fail(IDX_E_INVALID, "k_cache, block_table, context_lens (and k_scale_cache for FP8 / MX) must be non-NULL");
  if (!aligned16(kv->k_cache) || (scaled && !aligned16(kv->k_scale_cache)))
    return fail(IDX_E_INVALID, "k_cache and k_scale_cache must be 16-byte aligned");
  if (kv->num_pages <= 0 || kv->page_size <= 0 || kv->max_pages <= 0)
    return fail(IDX_E_INVALID, "num_pages, page_size and max_pages must be positive");
  if (int64_t(kv->max_pages) * kv->page_size < a->S_k)
    return fail(IDX_E_INVALID, "S_k=%d exceeds max_pages * page_size = %lld", a->S_k,
                (long long)(int64_t(kv->max_pages) * kv->page_size));
  return IDX_OK;
}

idx::PagedK paged_k(const idx_paged_k_t* kv) {
  return idx::PagedK{static_cast<const unsigned char*>(kv->k_cache), static_cast<const uint32_t*>(kv->k_scale_cache),
                     kv->block_table, kv->context_lens, kv->num_pages, kv->page_size, kv->max_pages, false};
}

// Whether a one-call paged request can score straight from the cache: the
// 64-head kernel, pages of 32 * 2^j keys (whole 32-key blocks, found with a
// shift), and a cache (and scale cache) addressable with 31-bit offsets.
// Other calls gather K first.
// Calls that convert their operands to bf16 read the converted keys.
bool direct_paged(const idx_logits_args_t* a, const idx_paged_k_t* kv) {
  const int64_t rows = int64_t(kv->num_pages) * kv->page_size;
  const int32_t bpp = kv->page_size / 32;
  return a->H == 64 && !idx::exec_of(a->in_dtype, a->accumulate).convert && kv->page_size % 32 == 0 &&
         (bpp & (bpp - 1)) == 0 &&
         rows * idx::row_bytes_of(a->in_dtype) < (int64_t(1) << 31) && rows * 4 < (int64_t(1) << 31);
}

// with_plan: the call builds its plan in the workspace.
idx_status_t check_workspace(const idx::WorkspaceLayout& WL, const void* ws, size_t ws_bytes, bool with_plan) {
  if (WL.total == 0) return fail(IDX_E_INVALID, "workspace size overflows");
  const size_t need = with_plan ? WL.total : WL.planned;
  if (ws == nullptr)
    return fail(IDX_E_WORKSPACE, "this call needs a workspace of %zu bytes (%s)", need,
                with_plan ? "idx_logits_workspace_bytes" : "idx_logits_workspace_bytes_planned");
  if (!aligned256(ws)) return fail(IDX_E_INVALID, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(IDX_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return IDX_OK;
}

idx::WorkspaceLayout layout_checked(const idx_logits_args_t* a) {
  return idx::workspace_layout(idx::exec_of(a->in_dtype, a->accumulate), a->B, a->S_q, a->S_k, a->H);
}

// Per-call preparation: K in MFMA fragment order and, where the call has
// them, the weighted-query pieces or Q converted to bf16.
idx_status_t prepare(const idx_logits_args_t* a, const idx::WorkspaceLayout& WL, unsigned char* ws,
                     const idx::PlanBuild* build, const idx::PagedK* paged, hipStream_t s) {
  const idx::Exec x = idx::exec_of(a->in_dtype, a->accumulate);
  const bool scaled = idx::has_kscale(x.kf), pieces = idx::uses_pieces(x.kf, a->H);
  hipError_t e = idx::launch_prepare(
      a->in_dtype, x.convert, a->H, a->w_dtype, a->k, a->k_scale, a->B, a->S_k, ws + WL.off_kfrag,
      scaled ? reinterpret_cast<uint32_t*>(ws + WL.off_kscale) : nullptr, a->q, a->q_scale, a->w,
      int64_t(a->B) * a->S_q, pieces ? ws + WL.off_pieces : nullptr,
      pieces ? reinterpret_cast<uint32_t*>(ws + WL.off_pscales) : nullptr,
      x.convert ? reinterpret_cast<uint16_t*>(ws + WL.off_qconv) : nullptr, build, paged, s);
  if (e != hipSuccess) return fail(IDX_E_HIP, "preparation launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

// The unit grid of a scoring launch over S_k columns (ScoreArgs).
idx_status_t set_units(idx::ScoreArgs& k, const idx::PlanLayout& L, int64_t S_k, bool cleanup,
                       int64_t units_per_cu = kUnitsPerCu) {
  int cus = 0;
  hipError_t he = device_cus(cus);
  if (he != hipSuccess) return fail(IDX_E_HIP, "device query failed: %s", hipGetErrorString(he));
  k.min_chunk = int32_t(kMinChunk);
  // Decode-sized tiles split a unit over all four waves: few, long units
  // then (one round, two per CU; measured against two rounds and against
  // units of one width for every tile), since each wave's start (its rows'
  // Q, weights and windows) costs about as much as streaming 500 keys.
  const int64_t rows = k.wave_split ? L.tile_rows : k.S_q;
  if (k.wave_split) units_per_cu = std::min<int64_t>(units_per_cu, 2);
  k.n_chunk = pick_chunks(S_k, L.n_tiles, rows, L.tile_rows, std::min<int64_t>(cus, kMaxCus), units_per_cu);
  k.n_pos_compute = int32_t(L.n_tiles * k.n_chunk);  // bounded by check_args
  // Decode-sized tiles of very different coverage (each request's context):
  // chunks of one width, as many as there are places in one round, so the
  // longest is no wider than that width (n equal chunks per tile left the
  // longest requests' chunks about twice the mean)
  k.dyn_units = 0;
  if (k.wave_split && L.n_tiles <= idx::kDynUnitTiles && L.n_tiles == k.B &&
      int64_t(S_k + idx::kColAlign) * L.n_tiles < (int64_t(1) << 31)) {  // the kernel sums widths in 32 bits
    k.dyn_units = 1;
    k.n_pos_compute =
        int32_t(std::max<int64_t>(units_per_cu * std::min<int64_t>(cus, kMaxCus), L.n_tiles + 64));
  }
  k.n_positions = cleanup ? int32_t(k.n_pos_compute + L.n_tiles) : k.n_pos_compute;
  return IDX_OK;
}

// Arguments of a scoring launch of call a with plan p (units set by set_units).
idx::ScoreArgs score_args(const idx_logits_args_t* a, const unsigned char* p, const idx::WorkspaceLayout& WL,
                          unsigned char* ws) {
  const idx::Exec x = idx::exec_of(a->in_dtype, a->accumulate);
  const idx::PlanLayout L = idx::plan_layout(a->B, a->S_q, a->H);
  idx::ScoreArgs k{};
  k.q = x.convert ? static_cast<const void*>(ws + WL.off_qconv) : a->q;
  k.q_scale = x.convert ? nullptr : a->q_scale;
  k.w = a->w;
  k.out = a->out;
  k.plan = p;
  k.ld = a->out_row_stride;
  k.sm_scale = a->sm_scale;
  k.B = a->B;
  k.S_q = a->S_q;
  k.S_k = a->S_k;
  k.n_tiles = int32_t(L.n_tiles);
  k.H = a->H;
  k.tile_rows = L.tile_rows;
  k.tiles_per_batch = int32_t(idx::tiles_per_batch(a->S_q, L.tile_rows));
  k.wave_split = a->H == 64 && a->S_q <= idx::kTileRows / 4 ? 1 : 0;
  k.seg_per_batch = int32_t(L.n_seg / a->B);
  k.tiles_per_seg = L.tiles_per_seg;
  k.last_seg_tiles = int32_t(k.tiles_per_batch - (k.seg_per_batch - 1) * int64_t(L.tiles_per_seg));
  k.off_start = uint32_t(L.off_start);
  k.off_end = uint32_t(L.off_end);
  k.off_slot = uint32_t(L.off_slot);
  k.off_lo = uint32_t(L.off_lo);
  k.off_hi = uint32_t(L.off_hi);
  k.off_order = uint32_t(L.off_order);
  k.pieces = idx::uses_pieces(x.kf, a->H) ? ws + WL.off_pieces : nullptr;
  k.pscales = idx::uses_pieces(x.kf, a->H) ? reinterpret_cast<const uint32_t*>(ws + WL.off_pscales) : nullptr;
  k.kfrag = ws + WL.off_kfrag;
  k.kscale = idx::has_kscale(x.kf) ? reinterpret_cast<const uint32_t*>(ws + WL.off_kscale) : nullptr;
  return k;
}

idx_status_t launch_scoring(int kf, const idx_logits_args_t* a, bool clean, const idx::ScoreArgs& k, hipStream_t s) {
  hipError_t e = hipSuccess;
  switch (kf) {
    case IDX_IN_BF16: e = idx::launch_score_bf16(a->w_dtype, a->out_dtype, clean, k, s); break;
    case IDX_IN_FP8_E4M3: e = idx::launch_score_fp8(a->w_dtype, a->out_dtype, clean, k, s); break;
    case IDX_IN_MXFP8_E4M3: e = idx::launch_score_mxfp8(a->w_dtype, a->out_dtype, clean, k, s); break;
    case IDX_IN_MXFP4_E2M1: e = idx::launch_score_mxfp4(a->w_dtype, a->out_dtype, clean, k, s); break;
    case idx::kInBF16RowScale: e = idx::launch_score_bf16rs(a->w_dtype, a->out_dtype, clean, k, s); break;
    default: return fail(IDX_E_INVALID, "unknown kernel format %d", kf);
  }
  if (e != hipSuccess) return fail(IDX_E_HIP, "scoring launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

// direct: a paged call whose scoring kernel reads the cache itself (see
// direct_paged), else NULL.
idx_status_t score(const idx_logits_args_t* a, const unsigned char* p, const idx::WorkspaceLayout& WL,
                   unsigned char* ws, hipStream_t s, const idx::PagedK* direct = nullptr) {
  idx::ScoreArgs k = score_args(a, p, WL, ws);
  idx_status_t st = set_units(k, idx::plan_layout(a->B, a->S_q, a->H), a->S_k, true);
  if (st != IDX_OK) return st;
  if (direct != nullptr) {
    k.kcache = direct->k_cache;
    k.kscache = direct->k_scale_cache;
    k.btable = direct->block_table;
    k.num_pages = direct->num_pages;
    k.page_size = direct->page_size;
    k.max_pages = direct->max_pages;
    while ((32 << k.bpp_shift) < direct->page_size) ++k.bpp_shift;
  }
  return launch_scoring(idx::exec_of(a->in_dtype, a->accumulate).kf, a, a->clean_logits != 0, k, s);
}

}  // namespace

extern "C" {

idx_status_t idx_logits_run(const idx_logits_args_t* a, const void* plan, const int32_t* q_causal_offsets,
                            const int32_t* row_starts, const int32_t* row_ends, void* workspace,
                            size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a);
  if (st != IDX_OK) return st;
  const unsigned char* p = static_cast<const unsigned char*>(plan);
  if (p == nullptr && (row_starts == nullptr) != (row_ends == nullptr))
    return fail(IDX_E_INVALID, "row_starts and row_ends must be given together");
  if (p != nullptr && !aligned256(p)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, p == nullptr)) != IDX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a plan built here shares the preparation launch
  idx::PlanBuild build{a->B, a->S_q, a->S_k, a->H, a->D, q_causal_offsets, row_starts, row_ends, nullptr,
                       ws + WL.off_plan};
  const bool build_plan = p == nullptr;
  if (build_plan) p = ws + WL.off_plan;
  if ((st = prepare(a, WL, ws, build_plan ? &build : nullptr, nullptr, s)) != IDX_OK) return st;
  return score(a, p, WL, ws, s);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of this device's `scratch`: the stream's device, which
// must be the current one (the symbol is looked up with it current).
idx_status_t scratch_on_device(void* stream, unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(IDX_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(IDX_E_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (int(sdev) != dev)
      return fail(IDX_E_INVALID, "the stream belongs to device %d, the current device is %d", int(sdev), dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(IDX_E_UNSUPPORTED, "device %d is beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(IDX_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch[dev];
  return IDX_OK;
}

}  // namespace

extern "C" {

idx_status_t idx_logits_run_noalloc(const idx_logits_args_t* a, const void* plan, const int32_t* q_causal_offsets,
                                    const int32_t* row_starts, const int32_t* row_ends, void* stream) {
  idx_status_t st = check_args(a);
  if (st != IDX_OK) return st;
  const idx::WorkspaceLayout WL = layout_checked(a);
  const size_t need = plan != nullptr ? WL.planned : WL.total;
  if (WL.total == 0) return fail(IDX_E_INVALID, "workspace size overflows");
  if (need > kScratchBytes)
    return fail(IDX_E_WORKSPACE, "this call needs %zu bytes of workspace; idx_logits_run_noalloc holds %zu",
                need, kScratchBytes);
  unsigned char* ws = nullptr;
  if ((st = scratch_on_device(stream, &ws)) != IDX_OK) return st;
  return idx_logits_run(a, plan, q_causal_offsets, row_starts, row_ends, ws, kScratchBytes, stream);
}

size_t idx_logits_noalloc_scratch_bytes(void) { return kScratchBytes; }

idx_status_t idx_logits_prepare(const idx_logits_args_t* a, void* workspace, size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a);
  if (st != IDX_OK) return st;
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, false)) != IDX_OK) return st;
  return prepare(a, WL, ws, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

idx_status_t idx_logits_plan_paged(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                                   const int32_t* context_lens, void* plan, size_t plan_bytes, void* stream) {
  idx_status_t st = check_dims(B, S_q, S_k, H, D);
  if (st != IDX_OK) return st;
  if (context_lens == nullptr) return fail(IDX_E_INVALID, "context_lens must be non-NULL");
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "plan buffer is NULL");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan buffer must be 256-byte aligned");
  const size_t need = idx::plan_layout(B, S_q, H).total;
  if (plan_bytes < need) return fail(IDX_E_WORKSPACE, "plan buffer has %zu bytes, %zu needed", plan_bytes, need);
  hipError_t e = idx::launch_plan_paged(B, S_q, S_k, H, D, context_lens, plan, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(IDX_E_HIP, "plan launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

idx_status_t idx_logits_prepare_paged(const idx_logits_args_t* a, const idx_paged_k_t* kv, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a, true);
  if (st != IDX_OK) return st;
  if ((st = check_paged(a, kv)) != IDX_OK) return st;
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, false)) != IDX_OK) return st;
  const idx::PagedK pk = paged_k(kv);
  return prepare(a, WL, ws, nullptr, &pk, static_cast<hipStream_t>(stream));
}

idx_status_t idx_logits_run_paged(const idx_logits_args_t* a, const idx_paged_k_t* kv, const void* plan,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a, true);
  if (st != IDX_OK) return st;
  if ((st = check_paged(a, kv)) != IDX_OK) return st;
  const unsigned char* p = static_cast<const unsigned char*>(plan);
  if (p != nullptr && !aligned256(p)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, p == nullptr)) != IDX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  idx::PlanBuild build{a->B, a->S_q, a->S_k, a->H, a->D, nullptr, nullptr, nullptr, kv->context_lens,
                       ws + WL.off_plan};
  const bool build_plan = p == nullptr;
  if (build_plan) p = ws + WL.off_plan;
  idx::PagedK pk = paged_k(kv);
  pk.skip_gather = direct_paged(a, kv);
  if ((st = prepare(a, WL, ws, build_plan ? &build : nullptr, &pk, s)) != IDX_OK) return st;
  return score(a, p, WL, ws, s, pk.skip_gather ? &pk : nullptr);
}

idx_status_t idx_logits_score_paged(const idx_logits_args_t* a, const idx_paged_k_t* kv, const void* plan,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a, true);
  if (st != IDX_OK) return st;
  if ((st = check_paged(a, kv)) != IDX_OK) return st;
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "idx_logits_score_paged needs a plan");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, false)) != IDX_OK) return st;
  idx::PagedK pk = paged_k(kv);
  pk.skip_gather = direct_paged(a, kv);
  return score(a, static_cast<const unsigned char*>(plan), WL, ws, static_cast<hipStream_t>(stream),
               pk.skip_gather ? &pk : nullptr);
}

idx_status_t idx_logits_topk(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                             const void* logits, idx_fp_t logits_dtype, int64_t ld, int32_t k, idx_topk_order_t order,
                             int32_t* topk_idx, float* topk_val, void* stream) {
  idx_status_t st = check_dims(B, S_q, S_k, H, D);
  if (st != IDX_OK) return st;
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "idx_logits_topk needs the plan the scores were made with");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  if (logits_dtype != IDX_F32 && logits_dtype != IDX_BF16)
    return fail(IDX_E_INVALID, "logits_dtype must be IDX_F32 or IDX_BF16");
  const uintptr_t es = logits_dtype == IDX_BF16 ? 2 : 4;
  if (logits == nullptr || topk_idx == nullptr) return fail(IDX_E_INVALID, "logits and topk_idx must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(logits) % es) != 0 || (reinterpret_cast<uintptr_t>(topk_idx) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(topk_val) & 3u) != 0)
    return fail(IDX_E_INVALID, "logits, topk_idx and topk_val must be aligned to their element size");
  if (k < 1 || k > idx::kMaxTopK) return fail(IDX_E_UNSUPPORTED, "k=%d outside [1, %d]", k, idx::kMaxTopK);
  if (order != IDX_TOPK_BY_COLUMN && order != IDX_TOPK_BY_SCORE)
    return fail(IDX_E_INVALID, "order must be IDX_TOPK_BY_COLUMN or IDX_TOPK_BY_SCORE");
  if (ld < S_k) return fail(IDX_E_INVALID, "ld %lld < S_k %d", (long long)ld, S_k);
  const int64_t rows = int64_t(B) * S_q;
  if (ld > (int64_t(1) << 40) || rows * ld > (int64_t(1) << 40))
    return fail(IDX_E_INVALID, "scores of %lld rows x stride %lld elements are too large", (long long)rows,
                (long long)ld);
  hipError_t e = idx::launch_topk(plan, B, S_q, S_k, H, D, logits, logits_dtype == IDX_BF16, ld, k,
                                  order == IDX_TOPK_BY_SCORE, topk_idx, topk_val, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(IDX_E_HIP, "top-k launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

idx_status_t idx_logits_score(const idx_logits_args_t* a, const void* plan, void* workspace, size_t workspace_bytes,
                              void* stream) {
  idx_status_t st = check_args(a, true);  // the keys come from the workspace
  if (st != IDX_OK) return st;
  if (plan == nullptr) return fail(IDX_E_WORKSPACE, "idx_logits_score needs a plan");
  if (!aligned256(plan)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  const idx::WorkspaceLayout WL = layout_checked(a);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if ((st = check_workspace(WL, ws, workspace_bytes, false)) != IDX_OK) return st;
  return score(a, static_cast<const unsigned char*>(plan), WL, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Workspace of a fused top-k call (internal.h, TopkLayout); total == 0 when
// the call's arguments are out of range.
idx::TopkLayout topk_layout_of(const idx_logits_args_t* a) {
  idx::TopkLayout T{};
  T.base = layout_of(a);
  if (T.base.total == 0) return T;
  const idx::Exec x = idx::exec_of(a->in_dtype, a->accumulate);
  const idx::PlanLayout L = idx::plan_layout(a->B, a->S_q, a->H);
  const int64_t rows = L.n_rows, S_k = a->S_k;
  if (rows * S_k > (int64_t(1) << 40)) return T;
  T.S_ks = idx::sample_col(S_k);
  T.nblk_s = cdiv(cdiv(S_k, 32), idx::kSampleStride);
  T.n_chunk_max = pick_chunks(S_k, L.n_tiles, a->S_q, L.tile_rows, kMaxCus);
  size_t off = T.base.total;
  T.off_skfrag = off;
  off += idx::align256(size_t(a->B) * size_t(T.nblk_s) * 32 * idx::row_bytes_of(x.kf));
  T.off_skscale = off;
  if (idx::has_kscale(x.kf)) off += idx::align256(size_t(a->B) * size_t(T.nblk_s) * 256);
  T.off_splan = off;
  off += L.total;
  T.off_sscore = off;
  off += idx::align256(size_t(rows) * size_t(T.S_ks) * 4);
  T.off_tau = off;
  off += idx::align256(size_t(rows) * 4);
  T.off_redo = off;
  off += idx::align256(size_t(rows) * 4);
  T.off_big = off;
  off += idx::align256(size_t(rows) * 4);
  T.off_gate = off;
  off += 256;
  T.off_meta = off;
  off += idx::align256(size_t(rows) * size_t(T.n_chunk_max) * 8);
  T.off_cand = off;
  off += idx::align256(size_t(rows) * size_t(S_k) * 8);
  T.total = off;
  return T;
}

}  // namespace

extern "C" {

size_t idx_logits_topk_workspace_bytes(const idx_logits_args_t* a) { return topk_layout_of(a).total; }

idx_status_t idx_logits_run_topk(const idx_logits_args_t* a, const void* plan, const int32_t* q_causal_offsets,
                                 const int32_t* row_starts, const int32_t* row_ends, int32_t k,
                                 idx_topk_order_t order, int32_t* topk_idx, float* topk_val, int32_t* n_redo,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  idx_status_t st = check_args(a, false, true);
  if (st != IDX_OK) return st;
  const unsigned char* p = static_cast<const unsigned char*>(plan);
  if (p == nullptr && (row_starts == nullptr) != (row_ends == nullptr))
    return fail(IDX_E_INVALID, "row_starts and row_ends must be given together");
  if (p != nullptr && !aligned256(p)) return fail(IDX_E_INVALID, "plan must be 256-byte aligned");
  if (k < 1 || k > idx::kMaxTopK) return fail(IDX_E_UNSUPPORTED, "k=%d outside [1, %d]", k, idx::kMaxTopK);
  if (order != IDX_TOPK_BY_COLUMN && order != IDX_TOPK_BY_SCORE)
    return fail(IDX_E_INVALID, "order must be IDX_TOPK_BY_COLUMN or IDX_TOPK_BY_SCORE");
  if (topk_idx == nullptr) return fail(IDX_E_INVALID, "topk_idx must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(topk_idx) & 3u) != 0 || (reinterpret_cast<uintptr_t>(topk_val) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(n_redo) & 3u) != 0)
    return fail(IDX_E_INVALID, "topk_idx, topk_val and n_redo must be 4-byte aligned");
  const idx::TopkLayout T = topk_layout_of(a);
  if (T.total == 0) return fail(IDX_E_INVALID, "workspace size overflows");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (ws == nullptr)
    return fail(IDX_E_WORKSPACE, "this call needs a workspace of %zu bytes (idx_logits_topk_workspace_bytes)",
                T.total);
  if (!aligned256(ws)) return fail(IDX_E_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < T.total)
    return fail(IDX_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, T.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const idx::Exec x = idx::exec_of(a->in_dtype, a->accumulate);
  const idx::PlanLayout L = idx::plan_layout(a->B, a->S_q, a->H);
  const idx::WorkspaceLayout& WL = T.base;

  // plan (unless given) and preparation, as for idx_logits_run
  idx::PlanBuild build{a->B, a->S_q, a->S_k, a->H, a->D, q_causal_offsets, row_starts, row_ends, nullptr,
                       ws + WL.off_plan};
  const bool build_plan = p == nullptr;
  if (build_plan) p = ws + WL.off_plan;
  if ((st = prepare(a, WL, ws, build_plan ? &build : nullptr, nullptr, s)) != IDX_OK) return st;
  hipError_t e = idx::launch_fused_setup(T, x.kf, a->B, a->S_q, a->S_k, a->H, p, ws, s);
  if (e != hipSuccess) return fail(IDX_E_HIP, "top-k setup launch failed: %s", hipGetErrorString(e));

  // the sample: every kSampleStride-th key block, scores stored unclean
  // (not needed when no window can hold more than k keys: every row then
  // keeps its whole window, and the thresholds read no sample)
  if (a->S_k > k) {
    idx::ScoreArgs ks = score_args(a, ws + T.off_splan, WL, ws);
    ks.S_k = int32_t(T.S_ks);
    ks.kfrag = ws + T.off_skfrag;
    ks.kscale = idx::has_kscale(x.kf) ? reinterpret_cast<const uint32_t*>(ws + T.off_skscale) : nullptr;
    ks.out = ws + T.off_sscore;
    ks.ld = T.S_ks;
    if ((st = set_units(ks, L, T.S_ks, false, 2)) != IDX_OK) return st;
    if ((st = launch_scoring(x.kf, a, false, ks, s)) != IDX_OK) return st;
  }

  // thresholds, then every cell in select mode
  idx::ScoreArgs kc = score_args(a, p, WL, ws);
  kc.out = nullptr;
  kc.cand = ws + T.off_cand;
  kc.meta = reinterpret_cast<int32_t*>(ws + T.off_meta);
  kc.tau = reinterpret_cast<const uint32_t*>(ws + T.off_tau);
  kc.wave_split = 0;  // select mode keeps one unit per (row, chunk) entry
  if ((st = set_units(kc, L, a->S_k, false)) != IDX_OK) return st;
  if (kc.n_chunk > T.n_chunk_max) return fail(IDX_E_HIP, "chunk count %d above the workspace's", kc.n_chunk);
  e = idx::launch_threshold(T, a->B, a->S_q, a->S_k, a->H, k, a->out_dtype == IDX_BF16, kc.n_chunk, p, ws, s);
  if (e != hipSuccess) return fail(IDX_E_HIP, "threshold launch failed: %s", hipGetErrorString(e));
  if ((st = launch_scoring(x.kf, a, false, kc, s)) != IDX_OK) return st;
  const bool by_score = order == IDX_TOPK_BY_SCORE;
  e = idx::launch_select(T, a->B, a->S_q, a->S_k, a->H, a->D, k, by_score, kc.n_chunk, 1, p, ws, topk_idx, topk_val,
                         n_redo, s);
  if (e != hipSuccess) return fail(IDX_E_HIP, "selection launch failed: %s", hipGetErrorString(e));

  // rows the sample misjudged, if any, again with every cell of their window
  kc.gate = reinterpret_cast<const int32_t*>(ws + T.off_gate);
  if ((st = launch_scoring(x.kf, a, false, kc, s)) != IDX_OK) return st;
  e = idx::launch_select(T, a->B, a->S_q, a->S_k, a->H, a->D, k, by_score, kc.n_chunk, 2, p, ws, topk_idx, topk_val,
                         n_redo, s);
  if (e != hipSuccess) return fail(IDX_E_HIP, "selection launch failed: %s", hipGetErrorString(e));
  return IDX_OK;
}

}  // extern "C"
