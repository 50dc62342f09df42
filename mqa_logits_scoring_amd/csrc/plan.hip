// Plan construction: per-row windows and per-tile column coverage.
//
// Window rules follow the per-row [start, end) windows of DeepGEMM pull
// request 435 (Performance section, reproducer: starts, ends, valid columns
// are those before `ends`) and the q_causal_offsets of cudnn-frontend pull
// request 416 (What section: offsets folded into per-row windows in 64-bit
// integers; the legacy kernel it describes adds offset + i + 1).  The offset
// is aligned so that offset 0 lets the last query row see every key.
#include "internal.h"

namespace idx {

namespace {

__global__ void plan_kernel(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* offsets,
                            const int32_t* starts, const int32_t* ends, unsigned char* plan, PlanLayout L) {
  const int64_t tile = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tile == 0) {
    PlanHeader* h = reinterpret_cast<PlanHeader*>(plan);
    h->magic = kPlanMagic;
    h->B = B;
    h->S_q = S_q;
    h->S_k = S_k;
    h->H = H;
    h->D = D;
    h->n_tiles = int32_t(L.n_tiles);
    h->tile_rows = kTileRows;
  }
  if (tile >= L.n_tiles) return;
  int32_t* win_start = reinterpret_cast<int32_t*>(plan + L.off_start);
  int32_t* win_end = reinterpret_cast<int32_t*>(plan + L.off_end);
  int32_t* slot_row = reinterpret_cast<int32_t*>(plan + L.off_slot);
  const int64_t tpb = tiles_per_batch(S_q);
  const int64_t b = tile / tpb;
  const int64_t i0 = (tile % tpb) * kTileRows;
  int64_t lo = S_k, hi = 0;
  for (int r = 0; r < kTileRows; ++r) {
    const int64_t i = i0 + r;
    const int64_t slot = tile * kTileRows + r;
    if (i >= S_q) {
      slot_row[slot] = -1;
      continue;
    }
    const int64_t row = b * S_q + i;
    int64_t s, e;
    if (starts != nullptr && ends != nullptr) {
      s = starts[row];
      e = ends[row];
      s = s < 0 ? 0 : (s > S_k ? S_k : s);
      e = e < s ? s : (e > S_k ? S_k : e);
    } else {
      const int64_t off = offsets != nullptr ? int64_t(offsets[b]) : 0;
      s = 0;
      e = int64_t(S_k) - int64_t(S_q) + off + i + 1;
      e = e < 0 ? 0 : (e > S_k ? S_k : e);
    }
    win_start[row] = int32_t(s);
    win_end[row] = int32_t(e);
    slot_row[slot] = int32_t(row);
    if (e > s) {
      lo = s < lo ? s : lo;
      hi = e > hi ? e : hi;
    }
  }
  int32_t* tile_lo = reinterpret_cast<int32_t*>(plan + L.off_lo);
  int32_t* tile_hi = reinterpret_cast<int32_t*>(plan + L.off_hi);
  if (hi <= lo) {  // every row of the tile is empty: nothing to compute
    lo = 0;
    hi = 0;
  } else {
    lo = lo / kColAlign * kColAlign;
    hi = (hi + kColAlign - 1) / kColAlign * kColAlign;
    hi = hi > S_k ? S_k : hi;
  }
  tile_lo[tile] = int32_t(lo);
  tile_hi[tile] = int32_t(hi);
}

__global__ void copy_windows_kernel(const unsigned char* plan, int64_t n_rows, size_t off_start, size_t off_end,
                                    int32_t* ws, int32_t* we) {
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  ws[r] = reinterpret_cast<const int32_t*>(plan + off_start)[r];
  we[r] = reinterpret_cast<const int32_t*>(plan + off_end)[r];
}

}  // namespace

hipError_t launch_plan(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* offsets,
                       const int32_t* starts, const int32_t* ends, void* plan, hipStream_t stream) {
  const PlanLayout L = plan_layout(B, S_q);
  const int threads = 128;
  const int64_t blocks = (L.n_tiles + threads - 1) / threads;
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream, B, S_q, S_k, H, D, offsets,
                     starts, ends, static_cast<unsigned char*>(plan), L);
  return hipGetLastError();
}

hipError_t launch_copy_windows(const void* plan, int64_t n_rows, int32_t* ws, int32_t* we, hipStream_t stream) {
  const PlanLayout L = plan_layout(1, n_rows);
  const int threads = 256;
  const int64_t blocks = (n_rows + threads - 1) / threads;
  hipLaunchKernelGGL(copy_windows_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                     static_cast<const unsigned char*>(plan), n_rows, L.off_start, L.off_end, ws, we);
  return hipGetLastError();
}

}  // namespace idx
