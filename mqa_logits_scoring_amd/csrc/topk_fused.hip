// Fused top-k selection: the steps that run around the scoring launches of
// idx_logits_run_topk (internal.h, "Fused top-k selection", gives the whole
// sequence).  The selection it computes is that of topk.hip over the scores
// a plain call would store: per row, the k columns of the window with the
// largest scores, equal scores by smaller column, NaN after every number.
// The sparse-attention page (FlashInfer SM120 sparse MLA, Summary and the
// DSv3.2 prefill notes) consumes such a 2048-key list per query token, and
// the DeepGEMM pull request 435 page times "uncompressed" logits (Performance
// section), the full S_q x S_k matrix this path never writes.
//
//  fused_setup_kernel  the sample plan (the call's plan with windows and
//                      coverage mapped to sample columns), the sampled K
//                      blocks in fragment order, the gate cleared
//  threshold_kernel    per row: the threshold key from the sample scores, the
//                      redo flag and the row's chunk entries cleared
//  select_kernel       per row: the top k of its candidates (pass 1), or of
//                      the rows sent through a second scoring pass (pass 2)

#include <algorithm>

#include "select_wave.h"

namespace idx {

namespace {

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kThrStage = 4096;   // sample keys a threshold workgroup keeps in LDS
constexpr int kSelStage = 8192;   // candidates a selection workgroup keeps in LDS
// A selection workgroup works on one row at a time: 16 waves (two
// workgroups per CU fit their LDS) keep its serial steps short.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPieceGroup = 256;  // chunk entries a selection workgroup reads at a time

__device__ __forceinline__ bool plan_matches(const unsigned char* plan, int32_t B, int32_t S_q, int32_t S_k,
                                             int32_t H, int32_t D, const PlanLayout& L) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  return h->magic == kPlanMagic && h->B == B && h->S_q == S_q && h->S_k == S_k && h->H == H && h->D == D &&
         h->n_tiles == int32_t(L.n_tiles) && h->tile_rows == L.tile_rows;
}

// ---------------------------------------------------------------------------
// setup

struct SetupArgs {
  const unsigned char* plan;
  unsigned char* splan;
  PlanLayout L;
  int32_t B, S_q, S_k, H, S_ks;
  const unsigned char* kfrag;
  unsigned char* skfrag;
  const uint32_t* kscale;  // NULL for BF16 keys
  uint32_t* skscale;
  int64_t nblk, nblk_s;
  int32_t blk_bytes;
  int32_t* gate;
};

__global__ void __launch_bounds__(kFThreads) fused_setup_kernel(const SetupArgs a) {
  const int64_t gid = int64_t(blockIdx.x) * kFThreads + threadIdx.x;
  const int64_t gsz = int64_t(gridDim.x) * kFThreads;
  const PlanLayout& L = a.L;
  const bool ok = plan_matches(a.plan, a.B, a.S_q, a.S_k, a.H, 128, L);
  if (gid == 0) {
    // a plan that does not match the call gives a sample plan no kernel accepts
    PlanHeader* sh = reinterpret_cast<PlanHeader*>(a.splan);
    sh->magic = ok ? kPlanMagic : 0u;
    sh->B = a.B;
    sh->S_q = a.S_q;
    sh->S_k = a.S_ks;
    sh->H = a.H;
    sh->D = 128;
    sh->n_tiles = int32_t(L.n_tiles);
    sh->tile_rows = L.tile_rows;
    a.gate[0] = 0;  // rows to score again
    a.gate[1] = 0;  // rows left to the workgroup selection
  }
  if (ok) {
    const int32_t* ws = reinterpret_cast<const int32_t*>(a.plan + L.off_start);
    const int32_t* we = reinterpret_cast<const int32_t*>(a.plan + L.off_end);
    int32_t* sws = reinterpret_cast<int32_t*>(a.splan + L.off_start);
    int32_t* swe = reinterpret_cast<int32_t*>(a.splan + L.off_end);
    for (int64_t i = gid; i < L.n_rows; i += gsz) {
      sws[i] = int32_t(sample_col(ws[i]));
      swe[i] = int32_t(sample_col(we[i]));
    }
    const int32_t* slot = reinterpret_cast<const int32_t*>(a.plan + L.off_slot);
    int32_t* sslot = reinterpret_cast<int32_t*>(a.splan + L.off_slot);
    for (int64_t i = gid; i < L.n_tiles * L.tile_rows; i += gsz) sslot[i] = slot[i];
    // coverage bounds are multiples of 32 (or S_k): mapped, they are the
    // bounds of the mapped windows' union, as a plan built from them has
    const int32_t* lo = reinterpret_cast<const int32_t*>(a.plan + L.off_lo);
    const int32_t* hi = reinterpret_cast<const int32_t*>(a.plan + L.off_hi);
    int32_t* slo = reinterpret_cast<int32_t*>(a.splan + L.off_lo);
    int32_t* shi = reinterpret_cast<int32_t*>(a.splan + L.off_hi);
    for (int64_t i = gid; i < L.n_tiles; i += gsz) {
      slo[i] = int32_t(sample_col(lo[i]));
      shi[i] = int32_t(sample_col(hi[i]));
    }
    const int32_t* ord = reinterpret_cast<const int32_t*>(a.plan + L.off_order);
    int32_t* sord = reinterpret_cast<int32_t*>(a.splan + L.off_order);
    for (int64_t i = gid; i < L.n_seg * L.tiles_per_seg; i += gsz) sord[i] = ord[i];
  }
  // sampled K: block jb of batch b is block jb * kSampleStride of the call's
  const int64_t per_blk = a.blk_bytes / 16;
  const uint4* src = reinterpret_cast<const uint4*>(a.kfrag);
  uint4* dst = reinterpret_cast<uint4*>(a.skfrag);
  for (int64_t i = gid; i < int64_t(a.B) * a.nblk_s * per_blk; i += gsz) {
    const int64_t blk = i / per_blk, w = i - blk * per_blk;
    const int64_t b = blk / a.nblk_s, jb = blk - b * a.nblk_s;
    dst[i] = src[(b * a.nblk + jb * kSampleStride) * per_blk + w];
  }
  if (a.kscale != nullptr) {
    for (int64_t i = gid; i < int64_t(a.B) * a.nblk_s * 64; i += gsz) {
      const int64_t blk = i / 64, w = i - blk * 64;
      const int64_t b = blk / a.nblk_s, jb = blk - b * a.nblk_s;
      a.skscale[i] = a.kscale[(b * a.nblk + jb * kSampleStride) * 64 + w];
    }
  }
}

// ---------------------------------------------------------------------------
// threshold

struct ThrArgs {
  const unsigned char* plan;
  PlanLayout L;
  int32_t B, S_q, S_k, H, S_ks, k, n_chunk;
  const void* sscore;  // [n_rows, S_ks] sample scores
  uint32_t* tau;
  int32_t* meta;
};

template <bool BF>
__global__ void __launch_bounds__(kFThreads) threshold_kernel(const ThrArgs a) {
  __shared__ uint32_t stage[kThrStage];
  __shared__ uint32_t hist[kHistWords];
  __shared__ uint32_t res[4];
  __shared__ uint32_t mm[2 * kFWaves];
  const int t = threadIdx.x;
  const int64_t r = blockIdx.x;
  int32_t* me = a.meta + 2 * r * a.n_chunk;
  for (int j = t; j < 2 * a.n_chunk; j += kFThreads) me[j] = 0;
  const PlanLayout& L = a.L;
  if (!plan_matches(a.plan, a.B, a.S_q, a.S_k, a.H, 128, L)) {
    if (t == 0) a.tau[r] = kTauNone;
    return;
  }
  const int64_t s = reinterpret_cast<const int32_t*>(a.plan + L.off_start)[r];
  const int64_t e = reinterpret_cast<const int32_t*>(a.plan + L.off_end)[r];
  const int64_t n = e > s ? e - s : 0;
  const int64_t n_out = n < a.k ? n : a.k;
  const int64_t ss = sample_col(s), ns = e > s ? sample_col(e) - ss : 0;
  const int64_t m = n > n_out ? sample_rank(n_out, n, ns) : 0;
  if (n == 0 || n == n_out || m >= ns) {  // nothing, or every cell of the window
    if (t == 0) a.tau[r] = n == 0 ? kTauNone : 0u;
    return;
  }
  const int64_t base = r * int64_t(a.S_ks) + ss;
  auto key_at = [&](int64_t i) {
    if constexpr (BF)
      return rank_key(uint32_t(static_cast<const uint16_t*>(a.sscore)[base + i]) << 16);
    else
      return rank_key(static_cast<const uint32_t*>(a.sscore)[base + i]);
  };
  const bool staged = ns <= kThrStage;
  int hi_bit = 32;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (staged) {
    // every load of a thread issued before the first store: their latencies overlap
    constexpr int U = kThrStage / kFThreads;
    uint32_t kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = int64_t(u) * kFThreads + t;
      kv[u] = key_at(i < ns ? i : ns - 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = int64_t(u) * kFThreads + t;
      if (i < ns) {
        stage[i] = kv[u];
        kmin = min(kmin, kv[u]);
        kmax = max(kmax, kv[u]);
      }
    }
    block_min_max<kFWaves>(kmin, kmax, mm);
    hi_bit = varying_bits(kmin, kmax);
  }
  auto for_each = [&](auto fn) {
    if (staged) {
      for (int64_t i = t; i < ns; i += kFThreads) fn(stage[i]);
    } else {
      for (int64_t i = t; i < ns; i += kFThreads) fn(key_at(i));
    }
  };
  // the top 16 key bits of the m-th best sampled score, lower bits 0: at
  // least m sampled cells reach it (a threshold a little below the m-th
  // score takes a few more candidates, in two passes instead of four)
  uint32_t count_eq, left;
  const uint32_t T = radix_select<kFThreads>(for_each, uint32_t(m), hist, res, count_eq, left,
                                             hi_bit > 16 ? hi_bit : 16, 16, kmin);
  if (t == 0) a.tau[r] = T;
}

// ---------------------------------------------------------------------------
// selection

struct SelArgs {
  const unsigned char* plan;
  PlanLayout L;
  int32_t B, S_q, S_k, H, D, k, n_chunk, pass;
  const uint2* cand;   // [n_rows, S_k] (score bits, column)
  int32_t* meta;
  uint32_t* tau;
  int32_t* redo;       // rows scored again, gate[0] of them
  int32_t* big;        // rows left to the workgroup kernel, gate[1] of them
  int32_t* gate;
  const int32_t* list; // workgroup kernel: its rows (redo or big), list_count of them; NULL: row = workgroup
  const int32_t* list_count;
  int32_t* out_idx;
  float* out_val;
  int32_t* n_redo;
};

// Pass 1, a row short of candidates: it is scored again keeping its whole
// window (threshold 0, chunk entries cleared, on the redo list).
__device__ void send_to_redo(const SelArgs& a, int64_t r, int lane_in_group, int group_size) {
  int32_t* mw = a.meta + 2 * r * a.n_chunk;
  for (int j = lane_in_group; j < 2 * a.n_chunk; j += group_size) mw[j] = 0;
  if (lane_in_group == 0) {
    a.tau[r] = 0u;
    a.redo[atomicAdd(&a.gate[0], 1)] = int32_t(r);
  }
}

// ---- a 256-thread workgroup per row (pass 1, by column) ----------------------
//
// Most rows: candidates staged by position (positions follow the columns:
// chunks ascend, and a chunk's candidates are in column order), a radix
// select over them and over the positions of the keys equal to its
// threshold, the selection's positions compacted in place, and the output
// gathered by slot.  About 25 KB of LDS, so six rows per CU are in flight.

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowStage = 4096;   // candidates a row keeps in LDS
constexpr int kRowChunks = 128;   // chunk entries a row keeps
constexpr int kRowPer = kRowStage / kRowThreads;  // positions per thread

struct RowSmem {
  uint32_t key[kRowStage];        // keys by position; then the selection's positions
  uint32_t hist[kHistWords];
  int32_t pc0[kRowChunks];        // chunk entries: first column, first position
  uint32_t pbase[kRowChunks];
  uint32_t res[4];
  uint32_t mm[2 * kRowWaves];
  uint32_t wsum[kRowWaves];
  uint32_t count;
};

// Slots in the row's candidate area of ascending candidate positions: each
// thread keeps the chunk of its last position and moves forward from there
// (the last chunk starting at or before p; chunks with no candidate share
// their base with the next one), so a thread walking positions in order does
// a step or two per position instead of a search.
struct SlotCursor {
  int j = 0;
  __device__ __forceinline__ uint32_t slot(const RowSmem& w, int n_chunk, uint32_t p) {
    while (j + 1 < n_chunk && w.pbase[j + 1] <= p) ++j;
    return uint32_t(w.pc0[j]) + (p - w.pbase[j]);
  }
};

__global__ void __launch_bounds__(kRowThreads) select_rows_kernel(const SelArgs a) {
  __shared__ RowSmem sm;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t r = blockIdx.x;
  const PlanLayout& L = a.L;
  const int k = a.k;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val != nullptr ? a.out_val + r * k : nullptr;
  if (!plan_matches(a.plan, a.B, a.S_q, a.S_k, a.H, a.D, L)) {  // loud, not plausible
    for (int i = t; i < k; i += kRowThreads) {
      oi[i] = -1;
      if (ov) ov[i] = __int_as_float(0x7FC00000);
    }
    if (t == 0) a.tau[r] = kTauNone;
    return;
  }
  auto to_big = [&]() {
    if (t == 0) a.big[atomicAdd(&a.gate[1], 1)] = int32_t(r);
  };
  if (a.n_chunk > kRowChunks) {
    to_big();
    return;
  }
  const int64_t s = reinterpret_cast<const int32_t*>(a.plan + L.off_start)[r];
  const int64_t e = reinterpret_cast<const int32_t*>(a.plan + L.off_end)[r];
  const int64_t n = e > s ? e - s : 0;
  const uint32_t n_out = uint32_t(n < k ? n : k);
  // chunk entries (the first wave, lane l: chunks l and l + 64) and their
  // first positions
  if (wave == 0) {
    const int32_t* me = a.meta + 2 * r * a.n_chunk;
    const int j0 = lane, j1 = lane + 64;
    const int32_t c00 = j0 < a.n_chunk ? me[2 * j0] : 0, c01 = j1 < a.n_chunk ? me[2 * j1] : 0;
    const uint32_t n0 = j0 < a.n_chunk ? uint32_t(me[2 * j0 + 1]) : 0u;
    const uint32_t n1 = j1 < a.n_chunk ? uint32_t(me[2 * j1 + 1]) : 0u;
    const uint32_t i0 = wave_scan(n0), i1 = wave_scan(n1);
    const uint32_t t0 = __builtin_amdgcn_readlane(i0, 63);
    sm.pc0[j0] = c00;
    sm.pbase[j0] = i0 - n0;
    sm.pc0[j1] = c01;
    sm.pbase[j1] = t0 + i1 - n1;
    if (lane == 0) sm.count = t0 + __builtin_amdgcn_readlane(i1, 63);
  }
  __syncthreads();
  const uint32_t C = sm.count;
  if (C < n_out) {
    send_to_redo(a, r, t, kRowThreads);
    return;
  }
  if (t == 0) a.tau[r] = kTauNone;  // done: a second pass keeps nothing of it
  if (C > uint32_t(kRowStage)) {
    to_big();
    return;
  }
  for (int i = int(n_out) + t; i < k; i += kRowThreads) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  if (n_out == 0) return;

  // ---- stage the keys by position (every load of a thread in flight) --------
  const uint2* row = a.cand + r * int64_t(a.S_k);
  const int nc = a.n_chunk;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    SlotCursor cur;
    uint32_t bits[kRowPer];
#pragma unroll
    for (int u = 0; u < kRowPer; ++u) {
      const uint32_t p = uint32_t(kRowThreads * u + t);
      bits[u] = row[p < C ? cur.slot(sm, nc, p) : 0u].x;
    }
#pragma unroll
    for (int u = 0; u < kRowPer; ++u) {
      const uint32_t p = uint32_t(kRowThreads * u + t);
      if (p < C) {
        const uint32_t key = rank_key(bits[u]);
        sm.key[p] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
  block_min_max<kRowWaves>(kmin, kmax, sm.mm);  // its barriers also complete the staging

  // ---- threshold: key T, and for keys equal to T the positions up to P2 ---
  const bool all = C == n_out;
  uint32_t T = 0, P2 = 0xFFFFFFFFu;
  if (!all) {
    uint32_t count_eq, want;
    T = radix_select<kRowThreads>(
        [&](auto fn) {
#pragma unroll 4
          for (uint32_t p = t; p < C; p += kRowThreads) fn(sm.key[p]);
        },
        n_out, sm.hist, sm.res, count_eq, want, varying_bits(kmin, kmax), 0, kmin, true);
    if (want < count_eq) {  // ties at T: the want smallest positions among them
      int nbits = 1;
      while ((uint32_t(1) << nbits) < C) ++nbits;
      const uint32_t top = (1u << nbits) - 1u;
      uint32_t ce2, left2;
      const uint32_t V = radix_select<kRowThreads>(
          [&](auto fn) {
            for (uint32_t p = t; p < C; p += kRowThreads)
              if (sm.key[p] == T) fn(top - p);
          },
          want, sm.hist, sm.res, ce2, left2, nbits, 0, 0u, true);
      P2 = top - V;
    }
  }

  // ---- the selection's positions in column order, in place -----------------
  // thread t: positions [t P, t P + P); the scan's barriers order every read
  // before the first write
  {
    const uint32_t P = (C + kRowThreads - 1) / kRowThreads;  // <= kRowPer
    uint32_t selm = 0;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j) {
      const uint32_t p = uint32_t(t) * P + uint32_t(j);
      if (uint32_t(j) < P && p < C) {
        const uint32_t key = sm.key[p];
        selm |= uint32_t(all || key > T || (key == T && p <= P2)) << j;
      }
    }
    const uint32_t mine = uint32_t(__builtin_popcount(selm));
    uint32_t total;
    uint32_t o = block_scan<kRowWaves>(mine, sm.wsum, total) - mine;
#pragma unroll
    for (int j = 0; j < kRowPer; ++j)
      if ((selm >> j) & 1u) sm.key[o++] = uint32_t(t) * P + uint32_t(j);
  }
  __syncthreads();

  // ---- output: scores and columns read back by slot ---------------------------
  constexpr int UO = kMaxTopK / kRowThreads;
  SlotCursor oc;
  uint2 v[UO];
#pragma unroll
  for (int u = 0; u < UO; ++u) {
    const uint32_t i = uint32_t(kRowThreads * u + t);
    v[u] = row[i < n_out ? oc.slot(sm, nc, sm.key[i]) : 0u];
  }
#pragma unroll
  for (int u = 0; u < UO; ++u) {
    const uint32_t i = uint32_t(kRowThreads * u + t);
    if (i < n_out) {
      oi[i] = int32_t(v[u].y);
      if (ov) ov[i] = __uint_as_float(v[u].x);
    }
  }
}

// ---- one workgroup per row ---------------------------------------------------
struct SelSmem {
  // the candidates as (rank key, slot) by position, slot = index in the
  // row's candidate area; compacted in place to the selection in column
  // order; rank order sorts (key, ~place) pairs held past the selection's
  // kMaxTopK entries
  uint2 cand[kSelStage];
  uint32_t hist[kHistWords];
  int32_t pc0[kPieceGroup];      // a group's chunk entries: first column,
  uint32_t pcnt[kPieceGroup];    // candidates,
  uint32_t pbase[kPieceGroup];   // first position
  uint32_t wsum[kSelWaves];
  uint32_t res[4];
  uint32_t mm[2 * kSelWaves];
};
static_assert(2 * kMaxTopK <= kSelStage, "rank order sorts behind the selection");

// Loads per lane issued before any is used (their latencies overlap).
constexpr int kSelUnroll = 4;

// Reads the row's chunk entries kPieceGroup at a time and, for each group,
// runs body(gsize, gbase) with pc0 / pcnt / pbase filled (pbase relative to
// gbase, the positions of the earlier groups).  Contains barriers.
template <typename Body>
__device__ void for_groups(const SelArgs& a, int64_t r, SelSmem& sm, Body body) {
  const int t = threadIdx.x;
  const int32_t* me = a.meta + 2 * r * a.n_chunk;
  uint32_t gbase = 0;
  for (int g0 = 0; g0 < a.n_chunk; g0 += kPieceGroup) {
    const int j = g0 + t;
    const bool own = t < kPieceGroup && j < a.n_chunk;
    const int32_t c0 = own ? me[2 * j] : 0;
    const uint32_t cnt = own ? uint32_t(me[2 * j + 1]) : 0u;
    uint32_t total;
    const uint32_t incl = block_scan<kSelWaves>(cnt, sm.wsum, total);
    if (t < kPieceGroup) {
      sm.pc0[t] = c0;
      sm.pcnt[t] = cnt;
      sm.pbase[t] = incl - cnt;
    }
    const int gsize = a.n_chunk - g0 < kPieceGroup ? a.n_chunk - g0 : kPieceGroup;
    __syncthreads();
    body(gsize, gbase, total);
    gbase += total;
    __syncthreads();  // the next group rewrites the entries
  }
}

// Every candidate of row r, chunk by chunk (a wave per chunk, its lanes over
// the chunk's candidates): fn(position, slot, score bits) -- positions follow
// the columns, slots index the row's candidate area.  fn must not contain
// barriers (the waves' shares differ).
template <typename Fn>
__device__ void for_candidates(const SelArgs& a, int64_t r, SelSmem& sm, Fn fn) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint2* row = a.cand + r * int64_t(a.S_k);
  for_groups(a, r, sm, [&](int gsize, uint32_t gbase, uint32_t) {
    for (int jj = wave; jj < gsize; jj += kSelWaves) {
      const uint32_t c0 = uint32_t(sm.pc0[jj]), cnt = sm.pcnt[jj], base = gbase + sm.pbase[jj];
      for (uint32_t i0 = 0; i0 < cnt; i0 += 64 * kSelUnroll) {
        uint32_t bits[kSelUnroll];
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
          const uint32_t i = i0 + uint32_t(64 * u + lane);
          bits[u] = row[c0 + (i < cnt ? i : cnt - 1)].x;
        }
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
          const uint32_t i = i0 + uint32_t(64 * u + lane);
          if (i < cnt) fn(base + i, c0 + i, bits[u]);
        }
      }
    }
  });
}

// Every candidate position in order, kSelThreads at a time: fn(valid,
// position, (key, slot)) from every thread the same number of times (fn may
// contain barriers).  For rows whose candidates do not fit in LDS; the
// position's chunk is found by a binary search over the group's entries.
template <typename Fn>
__device__ void walk(const SelArgs& a, int64_t r, SelSmem& sm, Fn fn) {
  const int t = threadIdx.x;
  const uint2* row = a.cand + r * int64_t(a.S_k);
  for_groups(a, r, sm, [&](int gsize, uint32_t gbase, uint32_t total) {
    for (uint32_t q0 = 0; q0 < total; q0 += kSelThreads) {
      const uint32_t q = q0 + uint32_t(t);
      int lo = 0, hi = gsize - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.pbase[mid] <= q)
          lo = mid;
        else
          hi = mid - 1;
      }
      const uint32_t slot = q < total ? uint32_t(sm.pc0[lo]) + (q - sm.pbase[lo]) : 0u;
      fn(q < total, gbase + q, make_uint2(rank_key(row[slot].x), slot));
    }
  });
}

// The selection of row r by the whole workgroup: rows whose candidates do
// not fit one wave's LDS (or whose chunk entries do not), pass 1 by score,
// and pass 2.
template <bool BY_SCORE>
__device__ void select_row(const SelArgs& a, int64_t r, SelSmem& sm) {
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int k = a.k;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val != nullptr ? a.out_val + r * k : nullptr;
  const PlanLayout& L = a.L;
  if (!plan_matches(a.plan, a.B, a.S_q, a.S_k, a.H, a.D, L)) {  // loud, not plausible
    for (int i = t; i < k; i += kSelThreads) {
      oi[i] = -1;
      if (ov) ov[i] = __int_as_float(0x7FC00000);
    }
    if (a.pass == 1 && t == 0) a.tau[r] = kTauNone;
    return;
  }
  const int64_t s = reinterpret_cast<const int32_t*>(a.plan + L.off_start)[r];
  const int64_t e = reinterpret_cast<const int32_t*>(a.plan + L.off_end)[r];
  const int64_t n = e > s ? e - s : 0;
  const uint32_t n_out = uint32_t(n < k ? n : k);
  for (int i = int(n_out) + t; i < k; i += kSelThreads) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  // candidates of the row
  const int32_t* me = a.meta + 2 * r * a.n_chunk;
  uint32_t mine = 0;
  for (int j = t; j < a.n_chunk; j += kSelThreads) mine += uint32_t(me[2 * j + 1]);
  uint32_t C;
  block_scan<kSelWaves>(mine, sm.wsum, C);
  if (C < n_out) {
    // fewer than the selection takes: the threshold was too high for this
    // row (pass 1), which is scored again keeping every cell of its window
    if (a.pass == 1) {
      send_to_redo(a, r, t, kSelThreads);
    } else {  // cannot happen: threshold 0 keeps the whole window
      for (int i = t; i < int(n_out); i += kSelThreads) {
        oi[i] = -1;
        if (ov) ov[i] = __int_as_float(0x7FC00000);
      }
    }
    return;
  }
  if (a.pass == 1 && t == 0) a.tau[r] = kTauNone;  // done: a second pass keeps nothing of it
  if (n_out == 0) return;

  // ---- stage (key, slot) by position when it fits; keys' range -------------
  const bool all = C == n_out;
  const bool staged = C <= uint32_t(kSelStage);
  int hi_bit = 32;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (staged) {
    for_candidates(a, r, sm, [&](uint32_t p, uint32_t slot, uint32_t bits) {
      const uint32_t key = rank_key(bits);
      sm.cand[p] = make_uint2(key, slot);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    });
    block_min_max<kSelWaves>(kmin, kmax, sm.mm);  // its barriers also complete the staging
    hi_bit = varying_bits(kmin, kmax);
  }

  // ---- the threshold among the candidates: key T, and for keys equal to T
  // the positions up to P2 (positions follow the columns) ----------------------
  uint32_t T = 0, P2 = 0xFFFFFFFFu;
  if (!all) {
    // fn(key, position) over every candidate (no barrier in fn)
    auto visit = [&](auto fn) {
      if (staged) {
        for (uint32_t p = t; p < C; p += kSelThreads) {
          const uint2 v = sm.cand[p];
          fn(v.x, p);
        }
      } else {
        for_candidates(a, r, sm, [&](uint32_t p, uint32_t, uint32_t bits) { fn(rank_key(bits), p); });
      }
    };
    uint32_t count_eq, want;
    T = radix_select<kSelThreads>([&](auto fn) { visit([&](uint32_t key, uint32_t) { fn(key); }); }, n_out,
                                  sm.hist, sm.res, count_eq, want, hi_bit, 0, kmin, true);
    if (want < count_eq) {
      // ties at T: the want smallest positions among them, as the want
      // largest of top - position
      int nbits = 1;
      while ((uint64_t(1) << nbits) < uint64_t(C)) ++nbits;
      const uint32_t top = nbits >= 32 ? 0xFFFFFFFFu : (1u << nbits) - 1u;
      uint32_t ce2, left2;
      const uint32_t V = radix_select<kSelThreads>(
          [&](auto fn) {
            visit([&](uint32_t key, uint32_t p) {
              if (key == T) fn(top - p);
            });
          },
          want, sm.hist, sm.res, ce2, left2, nbits, 0, 0u, true);
      P2 = top - V;
    }
  }

  // ---- the selection in column order, compacted to the front of sm.cand ---
  // (in place when staged: a round writes only places below its positions,
  // after every thread has read them)
  if (!all || !staged) {
    uint32_t done = 0;
    auto compact = [&](bool valid, uint32_t p, uint2 v) {
      const bool in = valid && (all || v.x > T || (v.x == T && p <= P2));
      const uint64_t b = __ballot(in);
      if (lane == 0) sm.wsum[wave] = uint32_t(__popcll(b));
      __syncthreads();
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) {
        before += w < wave ? sm.wsum[w] : 0u;
        total += sm.wsum[w];
      }
      if (in) {
        const uint32_t at = done + before + lanes_below(b);
        if (at < n_out) sm.cand[at] = v;  // exactly n_out are selected
      }
      done += total;
      __syncthreads();  // wsum is rewritten by the next round
    };
    if (staged) {
      for (uint32_t p0 = 0; p0 < C; p0 += kSelThreads) {
        const uint32_t p = p0 + uint32_t(t);
        const uint2 v = p < C ? sm.cand[p] : make_uint2(0u, 0u);
        compact(p < C, p, v);
      }
    } else {
      walk(a, r, sm, compact);
    }
  }
  __syncthreads();

  // ---- output: scores and columns read back by slot ---------------------------
  const uint2* row = a.cand + r * int64_t(a.S_k);
  if constexpr (!BY_SCORE) {
    for (int i = t; i < int(n_out); i += kSelThreads) {
      const uint2 v = row[sm.cand[i].y];
      oi[i] = int32_t(v.y);
      if (ov) ov[i] = __uint_as_float(v.x);
    }
  } else {
    // rank order: (key, ~place) pairs sorted descending, place = index in
    // the column order (so equal keys keep the smaller column first); padding
    // 0 sorts below every real pair
    uint64_t* pair = reinterpret_cast<uint64_t*>(&sm.cand[kMaxTopK]);
    int P = 1;
    while (P < int(n_out)) P <<= 1;
    for (int i = t; i < P; i += kSelThreads)
      pair[i] = i < int(n_out) ? (uint64_t(sm.cand[i].x) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(i)) : 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = t; i < P / 2; i += kSelThreads) {
          const int lo = 2 * stride * (i / stride) + (i % stride);
          const int hi = lo + stride;
          const bool descending = (lo & size) == 0;
          const uint64_t x = pair[lo], y = pair[hi];
          if ((x < y) == descending) {
            pair[lo] = y;
            pair[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int i = t; i < int(n_out); i += kSelThreads) {
      const uint2 v = row[sm.cand[0xFFFFFFFFu - uint32_t(pair[i])].y];
      oi[i] = int32_t(v.y);
      if (ov) ov[i] = __uint_as_float(v.x);
    }
  }
}

// LIST: the rows of a.list (a.list_count of them), walked by a fixed grid
// (one workgroup per CU: a row of such a list is long); else one workgroup
// per row, two per CU.
template <bool BY_SCORE, bool LIST>
__global__ void __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(LIST ? 4 : 8, LIST ? 4 : 8)))
select_kernel(const SelArgs a) {
  __shared__ SelSmem sm;
  if constexpr (!LIST) {
    select_row<BY_SCORE>(a, blockIdx.x, sm);
  } else {
    const int32_t count = *a.list_count;
    for (int32_t i = blockIdx.x; i < count; i += int32_t(gridDim.x)) {
      select_row<BY_SCORE>(a, a.list[i], sm);
      __syncthreads();  // the next row reuses sm
    }
    if (a.pass == 2 && blockIdx.x == 0 && threadIdx.x == 0 && a.n_redo != nullptr) *a.n_redo = a.gate[0];
  }
}

}  // namespace

hipError_t launch_fused_setup(const TopkLayout& T, int kf, int32_t B, int32_t S_q, int32_t S_k, int32_t H,
                              const unsigned char* plan, unsigned char* ws, hipStream_t stream) {
  SetupArgs a{};
  a.plan = plan;
  a.splan = ws + T.off_splan;
  a.L = plan_layout(B, S_q, H);
  a.B = B;
  a.S_q = S_q;
  a.S_k = S_k;
  a.H = H;
  a.S_ks = int32_t(T.S_ks);
  a.kfrag = ws + T.base.off_kfrag;
  a.skfrag = ws + T.off_skfrag;
  a.kscale = has_kscale(kf) ? reinterpret_cast<const uint32_t*>(ws + T.base.off_kscale) : nullptr;
  a.skscale = has_kscale(kf) ? reinterpret_cast<uint32_t*>(ws + T.off_skscale) : nullptr;
  a.nblk = (int64_t(S_k) + 31) / 32;
  a.nblk_s = T.nblk_s;
  a.blk_bytes = 32 * row_bytes_of(kf);
  a.gate = reinterpret_cast<int32_t*>(ws + T.off_gate);
  const int64_t work = std::max<int64_t>(a.L.n_rows, int64_t(B) * T.nblk_s * (a.blk_bytes / 16));
  const unsigned grid = unsigned(std::min<int64_t>(std::max<int64_t>((work + kFThreads - 1) / kFThreads, 1), 2048));
  hipLaunchKernelGGL(fused_setup_kernel, dim3(grid), dim3(kFThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_threshold(const TopkLayout& T, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t k,
                            bool scores_bf16, int32_t n_chunk, const unsigned char* plan, unsigned char* ws,
                            hipStream_t stream) {
  ThrArgs a{};
  a.plan = plan;
  a.L = plan_layout(B, S_q, H);
  a.B = B;
  a.S_q = S_q;
  a.S_k = S_k;
  a.H = H;
  a.S_ks = int32_t(T.S_ks);
  a.k = k;
  a.n_chunk = n_chunk;
  a.sscore = ws + T.off_sscore;
  a.tau = reinterpret_cast<uint32_t*>(ws + T.off_tau);
  a.meta = reinterpret_cast<int32_t*>(ws + T.off_meta);
  const dim3 grid(unsigned(a.L.n_rows));
  if (scores_bf16)
    hipLaunchKernelGGL(threshold_kernel<true>, grid, dim3(kFThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(threshold_kernel<false>, grid, dim3(kFThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select(const TopkLayout& T, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, int32_t k,
                         bool by_score, int32_t n_chunk, int pass, const unsigned char* plan, unsigned char* ws,
                         int32_t* out_idx, float* out_val, int32_t* n_redo, hipStream_t stream) {
  SelArgs a{};
  a.plan = plan;
  a.L = plan_layout(B, S_q, H);
  a.B = B;
  a.S_q = S_q;
  a.S_k = S_k;
  a.H = H;
  a.D = D;
  a.k = k;
  a.n_chunk = n_chunk;
  a.pass = pass;
  a.cand = reinterpret_cast<const uint2*>(ws + T.off_cand);
  a.meta = reinterpret_cast<int32_t*>(ws + T.off_meta);
  a.tau = reinterpret_cast<uint32_t*>(ws + T.off_tau);
  a.redo = reinterpret_cast<int32_t*>(ws + T.off_redo);
  a.big = reinterpret_cast<int32_t*>(ws + T.off_big);
  a.gate = reinterpret_cast<int32_t*>(ws + T.off_gate);
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.n_redo = n_redo;
  // rows walked from a list: one workgroup per CU of a 256-CU device at most
  const unsigned list_grid = unsigned(std::min<int64_t>(a.L.n_rows, 256));
  if (pass == 2) {
    a.list = a.redo;
    a.list_count = a.gate;
    if (by_score)
      hipLaunchKernelGGL((select_kernel<true, true>), dim3(list_grid), dim3(kSelThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((select_kernel<false, true>), dim3(list_grid), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (by_score) {
    hipLaunchKernelGGL((select_kernel<true, false>), dim3(unsigned(a.L.n_rows)), dim3(kSelThreads), 0, stream, a);
    return hipGetLastError();
  }
  // by column: a 256-thread workgroup per row, then the rows it leaves to the
  // 1024-thread kernel
  hipLaunchKernelGGL(select_rows_kernel, dim3(unsigned(a.L.n_rows)),
                     dim3(kRowThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.list = a.big;
  a.list_count = a.gate + 1;
  hipLaunchKernelGGL((select_kernel<false, true>), dim3(list_grid), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace idx
