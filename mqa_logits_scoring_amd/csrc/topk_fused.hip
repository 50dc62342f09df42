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

#include "internal.h"

namespace idx {

namespace {

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kThrStage = 4096;   // sample keys a threshold workgroup keeps in LDS
constexpr int kSelStage = 8192;   // candidate keys a selection workgroup keeps in LDS

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ bool plan_matches(const unsigned char* plan, int32_t B, int32_t S_q, int32_t S_k,
                                             int32_t H, int32_t D, const PlanLayout& L) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan);
  return h->magic == kPlanMagic && h->B == B && h->S_q == S_q && h->S_k == S_k && h->H == H && h->D == D &&
         h->n_tiles == int32_t(L.n_tiles) && h->tile_rows == L.tile_rows;
}

// Inclusive prefix sum of v over the workgroup (thread order); `total`
// receives the sum.  Contains barriers.
__device__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    const uint32_t s = wsum[w];
    before += w < wave ? s : 0u;
    all += s;
  }
  __syncthreads();  // wsum is reused by the next scan
  total = all;
  return x + before;
}

// Wave 0 over a 256-bin histogram (bin = digit): the digit whose bin holds
// the want-th largest counted key (1 <= want <= keys counted), the keys in
// higher bins and the keys in its bin, into res[0..2].  Lane l reads bins
// 4l..4l+3; a suffix sum over the lanes gives each lane the count above it.
__device__ void find_bin256(const uint32_t* hist, uint32_t want, uint32_t* res) {
  const int lane = threadIdx.x;
  uint32_t h[4], own = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    h[b] = hist[4 * lane + b];
    own += h[b];
  }
  uint32_t x = own;  // keys in the bins of lanes >= lane
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_down(x, d, 64);
    if (lane + d < 64) x += y;
  }
  const uint32_t above = x - own;
  if (above < want && want <= x) {
    uint32_t cum = above;
    bool found = false;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (!found && cum + h[b] >= want) {
        res[0] = uint32_t(4 * lane + b);
        res[1] = cum;
        res[2] = h[b];
        found = true;
      }
      cum += h[b];
    }
  }
}

// Radix select over keys, 8 bits per pass from the top: the want-th largest
// key (want >= 1) of those `for_each` visits, with how many keys equal it and
// how many of those the want-th still takes (want_left).  for_each(fn) calls
// fn(key) for every key, from every thread, and may contain barriers.
template <typename ForEach>
__device__ uint32_t radix_select(ForEach for_each, uint32_t want, uint32_t* hist, uint32_t* res, uint32_t& count_eq,
                                 uint32_t& want_left, int hi_bit = 32) {
  uint32_t prefix = 0, pmask = 0;
  for (int hi = hi_bit; hi > 0; hi -= 8) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dm = (1u << (hi - lo)) - 1u;
    for (int i = threadIdx.x; i < 256; i += kFThreads) hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> lo) & dm], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 64) find_bin256(hist, want, res);
    __syncthreads();
    const uint32_t d = res[0];
    want -= res[1];
    count_eq = res[2];
    prefix |= d << lo;
    pmask |= dm << lo;
  }
  want_left = want;
  return prefix;
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
    *a.gate = 0;
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
  int32_t* redo;
  int32_t* meta;
};

// Sampled cells a row's threshold ranks: about 1.5 times the share of the
// sample that the selection takes, plus 32.  With the sample's cells spread
// like the window's, the window then holds about 1.5 k + 32 R cells at or
// above the threshold, and fewer than k only when the sample misjudges the
// k-th score's rank by about a third; such a row is scored again.
__device__ __forceinline__ int64_t sample_rank(int64_t n_out, int64_t n, int64_t ns) {
  return (3 * n_out * ns + 2 * n - 1) / (2 * n) + 32;
}

template <bool BF>
__global__ void __launch_bounds__(kFThreads) threshold_kernel(const ThrArgs a) {
  __shared__ uint32_t stage[kThrStage];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t res[4];
  const int t = threadIdx.x;
  const int64_t r = blockIdx.x;
  int32_t* me = a.meta + 2 * r * a.n_chunk;
  for (int j = t; j < 2 * a.n_chunk; j += kFThreads) me[j] = 0;
  if (t == 0) a.redo[r] = 0;
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
  if (staged) {
    for (int64_t i = t; i < ns; i += kFThreads) stage[i] = key_at(i);
    __syncthreads();
  }
  auto for_each = [&](auto fn) {
    if (staged) {
      for (int64_t i = t; i < ns; i += kFThreads) fn(stage[i]);
    } else {
      for (int64_t i = t; i < ns; i += kFThreads) fn(key_at(i));
    }
  };
  uint32_t count_eq, left;
  const uint32_t T = radix_select(for_each, uint32_t(m), hist, res, count_eq, left);
  if (t == 0) a.tau[r] = T;
}

// ---------------------------------------------------------------------------
// selection

struct SelArgs {
  const unsigned char* plan;
  PlanLayout L;
  int32_t B, S_q, S_k, H, D, k, n_chunk, pass;
  const uint2* cand;  // [n_rows, S_k] (score bits, column)
  int32_t* meta;
  uint32_t* tau;
  int32_t* redo;
  int32_t* gate;
  int32_t* out_idx;
  float* out_val;
  int32_t* n_redo;
};

struct SelSmem {
  union {
    uint32_t key[kSelStage];     // the candidates' keys, by position
    uint64_t pair[kMaxTopK];     // rank order: (key, ~slot) of the selection
  };
  uint32_t out_bits[kMaxTopK];   // the selection in column order: score bits
  int32_t out_col[kMaxTopK];     // and columns
  uint32_t hist[256];
  int32_t pc0[kFThreads];        // a group's chunk entries: first column,
  uint32_t pbase[kFThreads];     // first position
  uint32_t wsum[kFWaves];
  uint32_t res[4];
};

// Every candidate position of row r in column order, 256 at a time: calls
// fn(valid, position, candidate index) from every thread the same number of
// times (fn may contain barriers).  The row's chunks are read kFThreads at a
// time; a chunk's candidates are consecutive positions, in column order, and
// the chunks' columns ascend.
template <typename Fn>
__device__ void walk(const SelArgs& a, int64_t r, SelSmem& sm, Fn fn) {
  const int t = threadIdx.x;
  const int32_t* me = a.meta + 2 * r * a.n_chunk;
  uint32_t gbase = 0;
  for (int g0 = 0; g0 < a.n_chunk; g0 += kFThreads) {
    const int j = g0 + t;
    const int32_t c0 = j < a.n_chunk ? me[2 * j] : 0;
    const uint32_t cnt = j < a.n_chunk ? uint32_t(me[2 * j + 1]) : 0u;
    uint32_t total;
    const uint32_t incl = block_scan(cnt, sm.wsum, total);
    sm.pc0[t] = c0;
    sm.pbase[t] = incl - cnt;
    const int gsize = a.n_chunk - g0 < kFThreads ? a.n_chunk - g0 : kFThreads;
    __syncthreads();
    for (uint32_t q0 = 0; q0 < total; q0 += kFThreads) {
      const uint32_t q = q0 + uint32_t(t);
      // the last chunk of the group starting at or before q (chunks with no
      // candidate share their base with the next one)
      int lo = 0, hi = gsize - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.pbase[mid] <= q)
          lo = mid;
        else
          hi = mid - 1;
      }
      fn(q < total, gbase + q, r * int64_t(a.S_k) + sm.pc0[lo] + int64_t(q - sm.pbase[lo]));
    }
    gbase += total;
    __syncthreads();  // the next group rewrites pc0 and pbase
  }
}

template <bool BY_SCORE>
__global__ void __launch_bounds__(kFThreads) select_kernel(const SelArgs a) {
  __shared__ SelSmem sm;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r = blockIdx.x;
  if (a.pass == 2) {
    if (r == 0 && t == 0 && a.n_redo != nullptr) *a.n_redo = *a.gate;
    if (a.redo[r] == 0) return;
  }
  const int k = a.k;
  int32_t* oi = a.out_idx + r * k;
  float* ov = a.out_val != nullptr ? a.out_val + r * k : nullptr;
  const PlanLayout& L = a.L;
  if (!plan_matches(a.plan, a.B, a.S_q, a.S_k, a.H, a.D, L)) {  // loud, not plausible
    for (int i = t; i < k; i += kFThreads) {
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
  for (int i = int(n_out) + t; i < k; i += kFThreads) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  // candidates of the row
  const int32_t* me = a.meta + 2 * r * a.n_chunk;
  uint32_t mine = 0;
  for (int j = t; j < a.n_chunk; j += kFThreads) mine += uint32_t(me[2 * j + 1]);
  uint32_t C;
  block_scan(mine, sm.wsum, C);
  if (C < n_out) {
    // fewer than the selection takes: the threshold was too high for this
    // row (pass 1), which is scored again keeping every cell of its window
    if (a.pass == 1) {
      int32_t* mw = a.meta + 2 * r * a.n_chunk;
      for (int j = t; j < 2 * a.n_chunk; j += kFThreads) mw[j] = 0;
      if (t == 0) {
        a.tau[r] = 0u;
        a.redo[r] = 1;
        atomicAdd(a.gate, 1);
      }
    } else {  // cannot happen: threshold 0 keeps the whole window
      for (int i = t; i < int(n_out); i += kFThreads) {
        oi[i] = -1;
        if (ov) ov[i] = __int_as_float(0x7FC00000);
      }
    }
    return;
  }
  if (a.pass == 1 && t == 0) a.tau[r] = kTauNone;  // done: a second pass keeps nothing of it
  if (n_out == 0) return;

  // ---- the threshold among the candidates: key T, and for keys equal to T
  // the positions up to P2 (positions follow the columns) ----------------------
  const bool all = C == n_out;
  const bool staged = C <= uint32_t(kSelStage);
  uint32_t T = 0, P2 = 0xFFFFFFFFu;
  if (!all) {
    if (staged) {
      walk(a, r, sm, [&](bool valid, uint32_t p, int64_t ci) {
        if (valid) sm.key[p] = rank_key(a.cand[ci].x);
      });
      __syncthreads();
    }
    // fn(key, position) over every candidate
    auto visit = [&](auto fn) {
      if (staged) {
        for (uint32_t p = t; p < C; p += kFThreads) fn(sm.key[p], p);
      } else {
        walk(a, r, sm, [&](bool valid, uint32_t p, int64_t ci) {
          if (valid) fn(rank_key(a.cand[ci].x), p);
        });
      }
    };
    uint32_t count_eq, want;
    T = radix_select([&](auto fn) { visit([&](uint32_t key, uint32_t) { fn(key); }); }, n_out, sm.hist, sm.res,
                     count_eq, want);
    if (want < count_eq) {
      // ties at T: the want smallest positions among them, as the want
      // largest of top - position
      int nbits = 1;
      while ((uint64_t(1) << nbits) < uint64_t(C)) ++nbits;
      const uint32_t top = nbits >= 32 ? 0xFFFFFFFFu : (1u << nbits) - 1u;
      uint32_t ce2, left2;
      const uint32_t V = radix_select(
          [&](auto fn) {
            visit([&](uint32_t key, uint32_t p) {
              if (key == T) fn(top - p);
            });
          },
          want, sm.hist, sm.res, ce2, left2, nbits);
      P2 = top - V;
    }
  }
  auto selected = [&](uint32_t key, uint32_t p) { return all || key > T || (key == T && p <= P2); };

  // ---- the selection in column order, staged in LDS --------------------------
  uint32_t done = 0;
  walk(a, r, sm, [&](bool valid, uint32_t p, int64_t ci) {
    bool in = false;
    if (valid) {
      const uint32_t key = all ? 0u : (staged ? sm.key[p] : rank_key(a.cand[ci].x));
      in = selected(key, p);
    }
    const uint64_t b = __ballot(in);
    if (lane == 0) sm.wsum[wave] = uint32_t(__popcll(b));
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kFWaves; ++w) {
      before += w < wave ? sm.wsum[w] : 0u;
      total += sm.wsum[w];
    }
    if (in) {
      const uint32_t at = done + before + lanes_below(b);
      if (at < n_out) {  // exactly n_out are selected
        const uint2 v = a.cand[ci];
        sm.out_bits[at] = v.x;
        sm.out_col[at] = int32_t(v.y);
      }
    }
    done += total;
    __syncthreads();  // wsum is rewritten by the next round
  });
  __syncthreads();

  if constexpr (!BY_SCORE) {
    for (int i = t; i < int(n_out); i += kFThreads) {
      oi[i] = sm.out_col[i];
      if (ov) ov[i] = __uint_as_float(sm.out_bits[i]);
    }
  } else {
    // rank order: (key, ~slot) pairs sorted descending, slot = place in the
    // column order (so equal keys keep the smaller column first); padding 0
    // sorts below every real pair
    int P = 1;
    while (P < int(n_out)) P <<= 1;
    for (int i = t; i < P; i += kFThreads)
      sm.pair[i] = i < int(n_out) ? (uint64_t(rank_key(sm.out_bits[i])) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(i))
                                  : 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = t; i < P / 2; i += kFThreads) {
          const int lo = 2 * stride * (i / stride) + (i % stride);
          const int hi = lo + stride;
          const bool descending = (lo & size) == 0;
          const uint64_t x = sm.pair[lo], y = sm.pair[hi];
          if ((x < y) == descending) {
            sm.pair[lo] = y;
            sm.pair[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int i = t; i < int(n_out); i += kFThreads) {
      const uint32_t slot = 0xFFFFFFFFu - uint32_t(sm.pair[i]);
      oi[i] = sm.out_col[slot];
      if (ov) ov[i] = __uint_as_float(sm.out_bits[slot]);
    }
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
  a.redo = reinterpret_cast<int32_t*>(ws + T.off_redo);
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
  a.gate = reinterpret_cast<int32_t*>(ws + T.off_gate);
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.n_redo = n_redo;
  const dim3 grid(unsigned(a.L.n_rows));
  if (by_score)
    hipLaunchKernelGGL(select_kernel<true>, grid, dim3(kFThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_kernel<false>, grid, dim3(kFThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace idx
