// Plan construction, one segment per workgroup: per-row windows, row order
// and per-tile column coverage (layout in internal.h).  Used by the plan
// kernel and by the preparation kernel of calls that build their plan.
//
// Window rules follow the per-row [start, end) windows of DeepGEMM pull
// request 435 (Performance section, reproducer: starts, ends, valid columns
// are those before `ends`) and the q_causal_offsets of cudnn-frontend pull
// request 416 (What section: offsets folded into per-row windows in 64-bit
// integers; the legacy kernel it describes adds offset + i + 1).  The offset
// is aligned so that offset 0 lets the last query row see every key.
#pragma once

#include "internal.h"

namespace idx {

// Order of a row inside its sort segment: rows with empty windows last, then
// by which sixteenth of [0, S_k] the window ends in, then by start.  Tiles of
// consecutive slots then hold rows whose windows nearly coincide, so a tile's
// coverage (the union of its rows' windows) adds little masked work.  Windows
// from causal offsets are already in this order.
__device__ inline uint32_t order_key(int64_t s, int64_t e, int64_t S_k, int shift) {
  if (e <= s) return 0x80000000u;
  const uint32_t eb = uint32_t((e * 16) / (S_k + 1));  // 0..15
  return (eb << 27) | uint32_t(s >> shift);
}

struct PlanParams {
  int32_t B, S_q, S_k, H, D;
  const int32_t* offsets;
  const int32_t* starts;
  const int32_t* ends;
  unsigned char* plan;
  PlanLayout L;
  // packed variable-length rows over ratio-compressed keys (B = 1): segment
  // boundaries in rows and in keys, n_seg + 1 each; cu_q == nullptr otherwise
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t n_seg, ratio;
  // paged calls: keys each request holds (the window of token i ends at
  // ctx - S_q + i + 1); nullptr otherwise
  const int32_t* ctx;
};

// Window of packed row i: segment s (the last with cu_q[s] <= i, found by
// binary search), local row t = i - cu_q[s], keys [cu_k[s], cu_k[s] +
// floor((t + 1) / ratio)) cut at cu_k[s+1]; rows outside every segment see
// nothing.  Clamping to [0, S_k] is left to the caller.
__device__ inline void thd_window(const PlanParams& P, int64_t i, int64_t& s, int64_t& e) {
  s = 0;
  e = 0;
  if (P.n_seg <= 0 || i < P.cu_q[0]) return;
  int lo = 0, hi = P.n_seg - 1;  // largest seg with cu_q[seg] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (P.cu_q[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  if (i >= P.cu_q[lo + 1]) return;
  const int64_t t = i - P.cu_q[lo];
  s = P.cu_k[lo];
  e = s + (t + 1) / P.ratio;
  const int64_t lim = P.cu_k[lo + 1];
  if (e > lim) e = lim;
}

// Shared memory one segment needs (8-byte aligned).
struct PlanSmem {
  uint64_t key[kSortRows];
  uint64_t tkey[kSortRows / 8];  // tiles of the segment by cost (tiles hold at least 8 rows)
  int32_t win_s[kSortRows], win_e[kSortRows];
  int unsorted;
};

// Ascending bitonic sort of n = 2^k keys in LDS by a whole workgroup.
__device__ inline void bitonic_sort(uint64_t* key, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < n / 2; t += kSortThreads) {
        const int lo = 2 * stride * (t / stride) + (t % stride);  // bit `stride` of lo is clear
        const int hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const uint64_t x = key[lo], y = key[hi];
        if ((x > y) == ascending) {
          key[lo] = y;
          key[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// One segment of the plan, by one workgroup of kSortThreads threads: the
// segment's kSortRows consecutive rows of a batch (segments hold whole tiles).
// It computes the rows' windows, orders the rows (with explicit windows: a
// bitonic sort by (order_key, row) in LDS), writes the slot rows and then the
// coverage of the segment's tiles from the windows it keeps in LDS, and
// last the segment's tiles ordered by cost (covered columns x rows,
// descending; ties by tile).  Segment 0 also writes the header.
__device__ inline void plan_segment(const PlanParams& P, int64_t segment, PlanSmem& sm) {
  const int32_t B = P.B, S_q = P.S_q, S_k = P.S_k, H = P.H, D = P.D;
  const int32_t *offsets = P.offsets, *starts = P.starts, *ends = P.ends;
  unsigned char* plan = P.plan;
  const PlanLayout& L = P.L;
  uint64_t* key = sm.key;
  int32_t* win_s = sm.win_s;
  int32_t* win_e = sm.win_e;
  int& unsorted = sm.unsorted;
  int32_t* win_start = reinterpret_cast<int32_t*>(plan + L.off_start);
  int32_t* win_end = reinterpret_cast<int32_t*>(plan + L.off_end);
  int32_t* slot_row = reinterpret_cast<int32_t*>(plan + L.off_slot);
  int32_t* tile_lo = reinterpret_cast<int32_t*>(plan + L.off_lo);
  int32_t* tile_hi = reinterpret_cast<int32_t*>(plan + L.off_hi);
  if (segment == 0 && threadIdx.x == 0) {
    PlanHeader* h = reinterpret_cast<PlanHeader*>(plan);
    h->magic = kPlanMagic;
    h->B = B;
    h->S_q = S_q;
    h->S_k = S_k;
    h->H = H;
    h->D = D;
    h->n_tiles = int32_t(L.n_tiles);
    h->tile_rows = L.tile_rows;
  }
  const int TR = L.tile_rows;
  const int64_t tpb = tiles_per_batch(S_q, TR);
  const int64_t spb = (int64_t(S_q) + kSortRows - 1) / kSortRows;
  const int64_t b = segment / spb, seg = segment % spb;
  const int64_t i0 = seg * kSortRows;
  const int n = int(min(int64_t(kSortRows), int64_t(S_q) - i0));
  // Packed variable-length rows keep their order: consecutive rows of a
  // segment see nearly the same keys already, and the first rows of every
  // segment (empty windows) would otherwise force a full sort.
  const bool thd = P.cu_q != nullptr;
  const bool explicit_windows = !thd && starts != nullptr && ends != nullptr;
  int shift = 0;
  while ((int64_t(S_k) >> shift) >= (int64_t(1) << 27)) ++shift;
  const int64_t slot0 = b * tpb * TR;
  for (int r = threadIdx.x; r < kSortRows; r += kSortThreads) {
    uint64_t k = ~uint64_t(0);
    if (r < n) {
      const int64_t i = i0 + r, row = b * S_q + i;
      int64_t s, e;
      if (thd) {
        thd_window(P, i, s, e);
        s = s < 0 ? 0 : (s > S_k ? S_k : s);
        e = e < s ? s : (e > S_k ? S_k : e);
      } else if (explicit_windows) {
        s = starts[row];
        e = ends[row];
        s = s < 0 ? 0 : (s > S_k ? S_k : s);
        e = e < s ? s : (e > S_k ? S_k : e);
      } else {
        int64_t off = offsets != nullptr ? int64_t(offsets[b]) : 0;
        if (P.ctx != nullptr) {  // context length n as the offset n - S_k
          int64_t n = P.ctx[b];
          n = n < 0 ? 0 : (n > S_k ? S_k : n);
          off = n - S_k;
        }
        s = 0;
        e = int64_t(S_k) - int64_t(S_q) + off + i + 1;
        e = e < 0 ? 0 : (e > S_k ? S_k : e);
      }
      win_start[row] = int32_t(s);
      win_end[row] = int32_t(e);
      win_s[r] = int32_t(s);
      win_e[r] = int32_t(e);
      k = (uint64_t(order_key(s, e, S_k, shift)) << 32) | uint32_t(r);
    }
    key[r] = k;
  }
  if (threadIdx.x == 0) unsorted = 0;
  __syncthreads();
  if (explicit_windows) {
    // sort only the smallest power of two holding the segment's rows, and
    // not at all when they are in order already
    int np2 = 2;
    while (np2 < n) np2 <<= 1;
    for (int r = threadIdx.x + 1; r < n; r += kSortThreads)
      if (key[r - 1] > key[r]) unsorted = 1;
    __syncthreads();
    if (unsorted) bitonic_sort(key, np2);
  }
  // slot rows (the key's low word is the row's index in the segment; padding
  // keys are all ones and sort last)
  for (int r = threadIdx.x; r < n; r += kSortThreads) {
    const int local = explicit_windows ? int(uint32_t(key[r])) : r;
    slot_row[slot0 + i0 + r] = int32_t(b * S_q + i0 + local);
  }
  if (seg == spb - 1) {  // padding slots of the batch's last tile
    for (int64_t i = int64_t(S_q) + threadIdx.x; i < tpb * TR; i += kSortThreads) slot_row[slot0 + i] = -1;
  }
  // coverage of the segment's tiles: the union of their rows' windows
  // widened to kColAlign columns (0, 0 when every row is empty)
  const int n_tiles_seg = (n + TR - 1) / TR;
  const int tps = kSortRows / TR;  // tile slots of a full segment, a power of two
  for (int t = threadIdx.x; t < tps; t += kSortThreads) sm.tkey[t] = ~uint64_t(0);
  __syncthreads();
  for (int t = threadIdx.x; t < n_tiles_seg; t += kSortThreads) {
    int64_t lo = S_k, hi = 0;
    const int rows = min(TR, n - t * TR);
    for (int r = t * TR; r < t * TR + TR && r < n; ++r) {
      const int local = explicit_windows ? int(uint32_t(key[r])) : r;
      const int64_t s = win_s[local], e = win_e[local];
      if (e > s) {
        lo = s < lo ? s : lo;
        hi = e > hi ? e : hi;
      }
    }
    if (hi <= lo) {
      lo = 0;
      hi = 0;
    } else {
      lo = lo / kColAlign * kColAlign;
      hi = (hi + kColAlign - 1) / kColAlign * kColAlign;
      hi = hi > S_k ? S_k : hi;
    }
    const int64_t tile = b * tpb + i0 / TR + t;
    tile_lo[tile] = int32_t(lo);
    tile_hi[tile] = int32_t(hi);
    // cost below 2^37 (2^31 columns x 64 rows): the key's top bits order by
    // descending cost, its low bits by tile
    const uint64_t cost = uint64_t(hi - lo) * uint64_t(rows);
    sm.tkey[t] = ((uint64_t(1) << 37) - 1 - cost) << 16 | uint64_t(t);
  }
  __syncthreads();
  bitonic_sort(sm.tkey, tps);
  int32_t* order = reinterpret_cast<int32_t*>(plan + L.off_order) + segment * tps;
  for (int r = threadIdx.x; r < tps; r += kSortThreads)
    order[r] = r < n_tiles_seg ? int32_t(b * tpb + i0 / TR + int64_t(sm.tkey[r] & 0xFFFFu)) : -1;
}

}  // namespace idx
