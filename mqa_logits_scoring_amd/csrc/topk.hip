// Top-k selection over the scores of a scoring call (gfx950).
//
// For each query row, the k columns of its window with the largest scores:
// larger first, equal scores by smaller column, NaN after every number (+0
// and -0 equal); listed by ascending column or in that rank order; columns
// past the window's size are -1 with score -inf.  The sparse-attention page
// (FlashInfer SM120 sparse MLA, Summary and the DSv3.2 prefill notes)
// consumes such a per-query list of 2048 key indices; the pages do not say
// how it is chosen, so the ranking above is the plain one and the algorithm
// is this file's own.
//
// One workgroup of 1024 threads per row.  Scores become 32-bit keys whose
// unsigned order is the ranking (sign-magnitude flipped, -0 folded onto +0,
// NaN to 0).  Thread t holds columns s + ch*kChunk + m*1024 + t (m < 32) of
// chunk ch in registers, so every load instruction of a wave reads 64
// consecutive scores; rows up to kChunk = 32768 columns are read once, longer
// rows once per pass.
//
//  1. A histogram of key bits 31..22 (1024 LDS bins, 8 copies spread over the
//     banks by lane) fixes the bucket b holding the k-th largest key: every
//     key above b is selected.
//  2. When b holds at most kCand keys, they are compacted into LDS with their
//     columns (one block scan of the per-thread counts places them) and the
//     rest of the selection is a radix select over that short list (key bits
//     21..10, 9..0, then the column for keys equal to the threshold).  A flat
//     row (b holding more) runs those passes over the registers instead.
//     Either way the result is a threshold (T, T2): a key is selected when it
//     is above T, or equal to T with a column no larger than the one T2 names.
//  3. The selected keys are written out: by column, each wave ballots its
//     selection per register and one block scan over the (register, wave)
//     counts gives every selected column its place; in rank order they go to
//     LDS as (key, ~column) pairs and a bitonic sort orders them.

#include "select_wave.h"

namespace idx {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kPerThread = 32;
constexpr int kChunk = kTopkThreads * kPerThread;  // 32768 columns
constexpr int kBins1 = 1024;                        // first pass: key bits 31..22
constexpr int kCopies1 = 8;                         // lane-interleaved copies of the first histogram
constexpr int kCopyStride = kBins1 + 1;             // words between copies: bin b of copy c is in bank (b + c) % 32
constexpr int kBins = 4096;                         // later passes: up to 12 bits
constexpr int kCand = 4096;                         // threshold-bucket keys kept in LDS
static_assert(kCopyStride * kCopies1 >= kBins, "the first histogram's storage holds the later ones");
static_assert(kBins % kTopkThreads == 0 && kBins1 % kTopkThreads == 0, "every thread owns whole bins");
constexpr int kCounts = kPerThread * kTopkWaves;  // (register, wave) counts of the column-order output
static_assert(kCounts <= kTopkThreads, "one (register, wave) count per thread at most");
static_assert(kPerThread <= 32, "a thread's registers fit one 32-bit mask");

template <bool BF>
__device__ __forceinline__ uint32_t score_bits(const void* logits, int64_t i) {
  if constexpr (BF)
    return uint32_t(static_cast<const uint16_t*>(logits)[i]) << 16;
  else
    return static_cast<const uint32_t*>(logits)[i];
}

struct TopkSmem {
  uint32_t hist[kCopyStride * kCopies1];  // first pass: bin b, copy c at c * kCopyStride + b
  union {
    struct {
      uint32_t key[kCand];
      uint32_t rel[kCand];
    } cand;                  // the threshold bucket's keys and columns (past s)
    uint64_t sel[kMaxTopK];  // rank order: the selection as (key, ~column) pairs
    struct {
      int32_t idx[kMaxTopK];
      uint32_t bits[kMaxTopK];
    } out;                   // column order: the selection staged for coalesced stores
  };
  uint32_t wcount[kCounts];  // selected per (register m, wave), in column order
  uint32_t wsum[kTopkWaves];
  uint32_t digit, above, count, n_cand, n_sel;
};

// Inclusive prefix sum of v over the workgroup's threads (thread order);
// `total` receives the sum over all threads.  Contains barriers.
__device__ uint32_t scan_1024(uint32_t v, TopkSmem& sm, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm.wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t s = sm.wsum[w];
    before += w < wave ? s : 0u;
    all += s;
  }
  __syncthreads();  // wsum is reused by the next scan
  total = all;
  return x + before;
}

struct PassResult {
  uint32_t digit, above, count;
};

// After a histogram pass over NB bins of C copies each: the digit d whose
// bin holds the want-th largest counted key; `above` = keys counted in higher
// bins, `count` = in bin d.
template <int NB, int C>
__device__ PassResult find_digit(TopkSmem& sm, uint32_t want) {
  constexpr int BPT = NB / kTopkThreads;
  __syncthreads();  // histogram complete
  const int t = threadIdx.x;
  uint32_t h[BPT], local = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) x += sm.hist[c * kCopyStride + t * BPT + b];
    h[b] = x;
    local += x;
  }
  uint32_t total;
  const uint32_t incl = scan_1024(local, sm, total);
  const uint32_t above = total - incl;  // keys in the bins of higher threads
  if (above < want && above + local >= want) {
    uint32_t cum = above;
#pragma unroll
    for (int b = BPT - 1; b >= 0; --b) {
      if (cum < want && cum + h[b] >= want) {
        sm.digit = uint32_t(t * BPT + b);
        sm.above = cum;
        sm.count = h[b];
      }
      cum += h[b];
    }
  }
  __syncthreads();
  PassResult r{sm.digit, sm.above, sm.count};
  __syncthreads();  // the next pass may clear the bins and overwrite the result
  return r;
}

template <int N>
__device__ __forceinline__ void clear_hist(TopkSmem& sm) {
  for (int i = threadIdx.x; i < N; i += kTopkThreads) sm.hist[i] = 0;
  __syncthreads();
}

// Score bits back from a key: exact except for the two keys that several
// bit patterns share (+0 for -0 too, 0 for every NaN), which the caller reads
// again.
__device__ __forceinline__ uint32_t key_bits(uint32_t k) { return (k >> 31) ? (k & 0x7FFFFFFFu) : 0u - k; }
__device__ __forceinline__ bool key_is_shared(uint32_t k) { return k == 0x80000000u || k == 0u; }

// MULTI: rows may span several chunks (S_k > kChunk).  The single-chunk
// kernel reads its row once and has one load site, which keeps the load
// offsets out of the registers the rest of the kernel needs.
template <bool BF, bool BY_SCORE, bool MULTI>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const unsigned char* plan, int32_t B, int32_t S_q,
                                                             int32_t S_k, int32_t H, int32_t D, const void* logits,
                                                             int64_t ld, int32_t k, int32_t* out_idx,
                                                             float* out_val, uint32_t off_start, uint32_t off_end) {
  __shared__ TopkSmem sm;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = blockIdx.x;
  int32_t* oi = out_idx + row * k;
  float* ov = out_val != nullptr ? out_val + row * k : nullptr;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == B && hdr->S_q == S_q && hdr->S_k == S_k &&
                       hdr->H == H && hdr->D == D;
  if (!plan_ok) {  // a plan for other dimensions: loud, not plausible
    for (int i = t; i < k; i += kTopkThreads) {
      oi[i] = -1;
      if (ov) ov[i] = __int_as_float(0x7FC00000);
    }
    return;
  }
  const int64_t s = reinterpret_cast<const int32_t*>(plan + off_start)[row];
  const int64_t e = reinterpret_cast<const int32_t*>(plan + off_end)[row];
  const int64_t n = e > s ? e - s : 0;
  const int64_t base = row * ld + s;
  const int n_out = int(n < k ? n : k);  // entries that name a column
  for (int i = n_out + t; i < k; i += kTopkThreads) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  if (n == 0) return;
  if (!BY_SCORE && n <= k) {  // the whole window, in column order
    for (int i = t; i < n_out; i += kTopkThreads) {
      oi[i] = int32_t(s + i);
      if (ov) ov[i] = __uint_as_float(score_bits<BF>(logits, base + i));
    }
    return;
  }
  const int nch = MULTI ? int((n + kChunk - 1) / kChunk) : 1;
  auto value_of = [&](uint32_t kk, uint32_t rel) {  // the score's exact bits
    return key_is_shared(kk) ? score_bits<BF>(logits, base + rel) : key_bits(kk);
  };

  // A chunk is read through a buffer resource based at its first column
  // (num_records = its width in bytes): the lane offset is the thread's, the
  // per-register offset a scalar constant, so addresses take no registers.
  // Registers hold keys; columns past the window get key 0, the NaN key, and
  // lose every tie to the window's own NaN (larger column), so when n > k
  // they can never be selected and need no check.
  constexpr int ES = BF ? 2 : 4;
  uint32_t key[kPerThread];
  auto load = [&](int ch) {
    const int64_t c0 = int64_t(ch) * kChunk;
    const int64_t w = n - c0 < kChunk ? n - c0 : kChunk;
    const int wc = int(w);  // <= kChunk
    const int mv = wc > t ? (wc - t + kTopkThreads - 1) / kTopkThreads : 0;  // registers inside the window
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(static_cast<const unsigned char*>(logits)) + (base + c0) * ES, 0, int(w * ES),
        0x00020000);
#pragma unroll
    for (int m = 0; m < kPerThread; ++m) {
      uint32_t bits;
      if constexpr (BF)
        bits = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rs, t * ES, m * kTopkThreads * ES, 0)) << 16;
      else
        bits = __builtin_amdgcn_raw_buffer_load_b32(rs, t * ES, m * kTopkThreads * ES, 0);
      // masked, not selected: a select on m < mv gets the load sunk into a
      // branch of its own, which then waits for it alone
      key[m] = rank_key(bits) & (0u - uint32_t(m < mv));
    }
  };
  if (!MULTI) load(0);

  // ---- the threshold ---------------------------------------------------------
  // selected: column inside the window and (key > T, or key == T and
  // (nbits == 0 or top - rel >= T2)); rel counts columns past s, up to the
  // padded width nch * kChunk, so the secondary key top - rel never wraps.
  uint32_t T = 0, T2 = 0, top = 0;
  int nbits = 0;
  // One histogram pass over the registers: count digit (v >> shift) & dmask
  // of every key with (key & msk) == pre, or in a tie pass (v = top - rel)
  // of every key equal to T with (v & msk) == pre.
  auto reg_pass = [&](bool tie, int shift, uint32_t dmask, uint32_t pre, uint32_t msk) {
    for (int ch = 0; ch < nch; ++ch) {
      if (MULTI) load(ch);
      uint32_t v0 = top - uint32_t(ch) * kChunk - uint32_t(t);  // tie key of register 0
      // opaque to the optimiser: the 64 tie keys v0 - m * 512 are then formed
      // inside the pass, not hoisted out of the passes into 64 live registers
      asm volatile("" : "+v"(v0));
#pragma unroll
      for (int m = 0; m < kPerThread; ++m) {
        const uint32_t kk = key[m];
        const uint32_t v = tie ? v0 - uint32_t(m * kTopkThreads) : kk;
        const bool c = tie ? (kk == T && (v & msk) == pre) : ((kk & msk) == pre);
        if (c) atomicAdd(&sm.hist[(v >> shift) & dmask], 1u);
      }
    }
  };
  // The same over the candidates in LDS.
  auto cand_pass = [&](int nc, bool tie, int shift, uint32_t dmask, uint32_t pre, uint32_t msk) {
    for (int i = t; i < nc; i += kTopkThreads) {
      const uint32_t kk = sm.cand.key[i];
      const uint32_t v = tie ? top - sm.cand.rel[i] : kk;
      const bool c = tie ? (kk == T && (v & msk) == pre) : ((kk & msk) == pre);
      if (c) atomicAdd(&sm.hist[(v >> shift) & dmask], 1u);
    }
  };
  if (n > k) {
    uint32_t want = uint32_t(k);
    while ((int64_t(1) << nbits) < int64_t(nch) * kChunk) ++nbits;
    top = nbits == 32 ? 0xFFFFFFFFu : (1u << nbits) - 1u;
    // 1. key bits 31..22 over the whole row, into lane-interleaved copies so
    //    that lanes counting the same bin rarely touch the same word
    clear_hist<kCopyStride * kCopies1>(sm);
    if (t == 0) sm.n_cand = 0;
    {  // every key counts: no condition, fixed digit and copies
      const uint32_t copy = (uint32_t(lane) & (kCopies1 - 1u)) * kCopyStride;
      for (int ch = 0; ch < nch; ++ch) {
        if (MULTI) load(ch);
#pragma unroll
        for (int m = 0; m < kPerThread; ++m) atomicAdd(&sm.hist[(key[m] >> 22) + copy], 1u);
      }
    }
    const PassResult r1 = find_digit<kBins1, kCopies1>(sm, want);
    want -= r1.above;
    uint32_t prefix = r1.digit << 22, mask = 0xFFC00000u, count_eq = r1.count;
    // 2. the bucket's keys and columns into LDS when they fit (the passes
    //    below then read the short list), else the passes read the registers
    const bool listed = r1.count <= uint32_t(kCand);
    if (listed) {
      // each thread's candidates at its place from one block scan of the
      // per-thread counts (thread-major order; the selection below does not
      // depend on the list's order)
      uint32_t done = 0;  // candidates of the earlier chunks
      for (int ch = 0; ch < nch; ++ch) {
        if (MULTI) load(ch);
        uint32_t rel0 = uint32_t(ch) * kChunk + uint32_t(t);
        asm volatile("" : "+v"(rel0));  // per-register columns formed here, not hoisted
        uint32_t cm = 0;  // bit m: register m is a candidate
#pragma unroll
        for (int m = 0; m < kPerThread; ++m) cm |= uint32_t((key[m] & mask) == prefix) << m;
        const uint32_t mine = uint32_t(__builtin_popcount(cm));
        uint32_t total;
        uint32_t pos = done + scan_1024(mine, sm, total) - mine;
#pragma unroll
        for (int m = 0; m < kPerThread; ++m) {
          if ((cm >> m) & 1u) {
            if (pos < uint32_t(kCand)) {
              sm.cand.key[pos] = key[m];
              sm.cand.rel[pos] = rel0 + uint32_t(m * kTopkThreads);
            }
            ++pos;
          }
        }
        done += total;
      }
      __syncthreads();
    }
    const int nc = int(r1.count);  // == n_cand when listed
    for (int p = 0; p < 2; ++p) {  // key bits [21:10], [9:0]
      const int shift = p == 0 ? 10 : 0;
      const uint32_t dmask = p == 0 ? 0xFFFu : 0x3FFu;
      clear_hist<kBins>(sm);
      if (listed)
        cand_pass(nc, false, shift, dmask, prefix, mask);
      else
        reg_pass(false, shift, dmask, prefix, mask);
      const PassResult r = find_digit<kBins, 1>(sm, want);
      want -= r.above;
      prefix |= r.digit << shift;
      mask |= dmask << shift;
      count_eq = r.count;
    }
    T = prefix;
    if (want < count_eq) {  // ties at T: the smallest columns among them
      uint32_t prefix2 = 0, mask2 = 0;
      for (int hi = nbits; hi > 0; hi -= 12) {
        const int lo = hi > 12 ? hi - 12 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        clear_hist<kBins>(sm);
        if (listed)
          cand_pass(nc, true, lo, dmask, prefix2, mask2);
        else
          reg_pass(true, lo, dmask, prefix2, mask2);
        const PassResult r = find_digit<kBins, 1>(sm, want);
        want -= r.above;
        prefix2 |= r.digit << lo;
        mask2 |= dmask << lo;
      }
      T2 = prefix2;
    } else {
      nbits = 0;  // every key equal to T is selected
    }
  }
  // n <= k (rank order only) selects every column of the window: T = 0, nbits = 0
  const uint32_t n_rel = uint32_t(n);
  auto selected = [&](uint32_t kk, uint32_t rel) {
    return rel < n_rel && (kk > T || (kk == T && (nbits == 0 || top - rel >= T2)));
  };

  // ---- the output ------------------------------------------------------------
  if constexpr (!BY_SCORE) {
    // by column: per chunk, every (register, wave) count in column order, one
    // block scan, each selected column staged at its place in LDS, then
    // written out with coalesced stores
    uint32_t done = 0;  // selected columns of the earlier chunks
    for (int ch = 0; ch < nch; ++ch) {
      if (MULTI) load(ch);
      uint32_t rel0 = uint32_t(ch) * kChunk + uint32_t(t);
      asm volatile("" : "+v"(rel0));  // per-register columns formed here, not hoisted
      uint32_t selm = 0;  // bit m: register m is selected
#pragma unroll
      for (int m = 0; m < kPerThread; ++m) selm |= uint32_t(selected(key[m], rel0 + uint32_t(m * kTopkThreads))) << m;
      // this wave's count per register, gathered into lane m, written at once
      uint32_t cnt = 0;
#pragma unroll
      for (int m = 0; m < kPerThread; ++m) {
        const uint32_t c_m = uint32_t(__popcll(__ballot((selm >> m) & 1u)));  // wave-uniform
        cnt = lane == m ? c_m : cnt;
      }
      if (lane < kPerThread) sm.wcount[lane * kTopkWaves + wave] = cnt;
      __syncthreads();
      uint32_t total;
      const uint32_t mine = t < kCounts ? sm.wcount[t] : 0u;
      const uint32_t excl = scan_1024(mine, sm, total) - mine;
      if (t < kCounts) sm.wcount[t] = excl;  // entry t = (m, wave) in column order: its first place
      __syncthreads();
      const uint32_t bases = lane < kPerThread ? sm.wcount[lane * kTopkWaves + wave] : 0u;
#pragma unroll
      for (int m = 0; m < kPerThread; ++m) {
        const bool in = (selm >> m) & 1u;
        const uint64_t b = __ballot(in);
        const uint32_t base_m = __builtin_amdgcn_readlane(bases, m);
        if (in) {
          const uint32_t pos = done + base_m + lanes_below(b);
          if (pos < uint32_t(n_out)) {  // exactly n_out are selected
            sm.out.idx[pos] = int32_t(rel0 + uint32_t(m * kTopkThreads));
            sm.out.bits[pos] = key[m];
          }
        }
      }
      done += total;
      __syncthreads();  // wcount is rewritten by the next chunk; the staging is complete
    }
    for (int i = t; i < n_out; i += kTopkThreads) {
      const uint32_t rel = uint32_t(sm.out.idx[i]);
      oi[i] = int32_t(s + rel);
      if (ov) ov[i] = __uint_as_float(value_of(sm.out.bits[i], rel));
    }
  } else {
    // rank order: the selection as (key, ~column) pairs into LDS, bitonic sort
    if (t == 0) sm.n_sel = 0;
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
      if (MULTI) load(ch);
      uint32_t rel0 = uint32_t(ch) * kChunk + uint32_t(t);
      asm volatile("" : "+v"(rel0));  // per-register columns formed here, not hoisted
#pragma unroll
      for (int m = 0; m < kPerThread; ++m) {
        const uint32_t rel = rel0 + uint32_t(m * kTopkThreads);
        const bool in = selected(key[m], rel);
        const uint64_t b = __ballot(in);
        if (b != 0) {
          uint32_t pos = 0;
          if (lane == 0) pos = atomicAdd(&sm.n_sel, uint32_t(__popcll(b)));
          pos = __shfl(pos, 0, 64) + lanes_below(b);
          if (in && pos < uint32_t(kMaxTopK)) sm.sel[pos] = (uint64_t(key[m]) << 32) | uint64_t(0xFFFFFFFFu - rel);
        }
      }
    }
    __syncthreads();
    // pad to a power of two with 0 (below every real pair) and sort
    // descending.  Wave w owns pairs [128w, 128w + 128), so stages with a
    // stride below 256 elements stay inside its own 256 elements and need no
    // workgroup barrier: a wave's LDS accesses are performed in order.
    int P = 1, logP = 0;
    while (P < k) {
      P <<= 1;
      ++logP;
    }
    for (int i = n_out + t; i < P; i += kTopkThreads) sm.sel[i] = 0;
    __syncthreads();
    for (int lsize = 1; lsize <= logP; ++lsize) {
      for (int lstride = lsize - 1; lstride >= 0; --lstride) {
        const int stride = 1 << lstride;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 128 * wave + 64 * h + lane;
          if (i < P / 2) {
            const int lo = ((i >> lstride) << (lstride + 1)) | (i & (stride - 1));
            const int hi = lo + stride;
            const bool descending = ((lo >> lsize) & 1) == 0;
            const uint64_t x = sm.sel[lo], y = sm.sel[hi];
            if ((x < y) == descending) {
              sm.sel[lo] = y;
              sm.sel[hi] = x;
            }
          }
        }
        if (stride >= 256 || (lstride == 0 && lsize >= 8))
          __syncthreads();  // the next stage reads other waves' elements
        else
          __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    for (int i = t; i < n_out; i += kTopkThreads) {
      const uint64_t c = sm.sel[i];
      const uint32_t rel = 0xFFFFFFFFu - uint32_t(c);
      oi[i] = int32_t(s + rel);
      if (ov) ov[i] = __uint_as_float(value_of(uint32_t(c >> 32), rel));
    }
  }
}

// ---------------------------------------------------------------------------
// Column order, one 256-thread workgroup per row
//
// The kernel above holds a whole CU for one row, all of it in registers.
// Rows selected by column run here instead, four workgroups per CU, each
// with about 37 KB of LDS:
//  - A window of at most kTbStage columns is staged whole: the score of
//    column s + p at p.
//  - A wider one is thresholded first, as the fused selection is: the key of
//    the m-th best of a sample of its columns (the first 32 of every 512),
//    its low 16 bits cleared, m = sample_rank.  The four waves then stream a
//    quarter of the window each and stage the scores that reach it, with
//    their columns, in any order: about 1.25 k + 512 of them.
//  - A radix select over the staged keys, then over the columns of the keys
//    equal to its threshold, gives the selection; its columns are marked in
//    a bitmap of the window, whose word counts give each selected column its
//    place in column order, and its score is written there from the stage
//    (no second read of the row).
//  - A row whose threshold keeps more keys than the stage holds (many equal
//    scores) or fewer than it must select, or whose sample does not fit, is
//    selected from memory by its first wave: the same radix selects, every
//    pass streaming the window, then one more pass writing the selection in
//    column order.

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTbThreads = 256;
constexpr int kTbWaves = kTbThreads / 64;
constexpr int kTbStage = 4096;                // keys a row keeps in LDS
constexpr int kTbMaxBitmapCols = 65536;       // windows the bitmap covers (thresholded rows)
// Rows the workgroup kernel takes: byte offsets of a row's columns fit 31 bits.
constexpr int64_t kTkMaxCols = int64_t(1) << 28;

struct TbSmem {
  uint32_t key[kTbStage];  // staged scores' bits (fp32; bf16 widened), by position
  uint16_t col[kTbStage];  // window column (past s) of each position of a thresholded row
  union {
    uint32_t hist[kHistWords];                 // radix-select histograms
    uint32_t bits[kTbMaxBitmapCols / 32];      // the selection's columns
  };
  uint16_t wpre[kTbMaxBitmapCols / 32];        // selected columns in the bitmap's words before each
  uint32_t res[4];
  uint32_t mm[2 * kTbWaves];
  uint32_t wsum[kTbWaves];
  uint32_t count;
};
static_assert(kTbMaxBitmapCols / 32 <= kHistWords, "the bitmap shares the histograms' words");
static_assert(kMaxTopK <= 65535, "places in the output fit the 16-bit word prefixes");

// Streams a row's columns [s, e): body(key, bits, c, valid) runs for the V
// columns c, c + 1, ... of each lane's share, lanes in order and shares in
// column order, and returns false to stop (the same in every lane).  The
// columns from the first 16-byte boundary at or past s to the last one at or
// before e are read in 16-byte loads, two batches of U per lane in flight,
// through a resource that ends at that last boundary (a load past it reads
// zeros, none is cut by it); the few columns before and after, in lane 0,
// one by one through rs, which covers the row's columns [0, e) from its
// first (rowp).
template <bool BF, typename Body>
__device__ __forceinline__ void stream_window(__amdgpu_buffer_rsrc_t rs, const unsigned char* rowp, int64_t s,
                                              int64_t e, Body body) {
  constexpr int ES = BF ? 2 : 4, V = 16 / ES, U = 4;
  constexpr int64_t kStep = 64 * V * U;
  const int lane = threadIdx.x & 63;
  // columns [c, c_end) in lane 0, one load each
  auto few = [&](int64_t c, int64_t c_end) {
    uint32_t bits[V], key[V];
    bool valid[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      valid[j] = lane == 0 && c + j < c_end;
      const int64_t cj = valid[j] ? c + j : c;
      bits[j] = BF ? uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rs, int(cj * 2), 0, 0)) << 16
                   : __builtin_amdgcn_raw_buffer_load_b32(rs, int(cj * 4), 0, 0);
      key[j] = rank_key(bits[j]);
    }
    return body(key, bits, c, valid);
  };
  const int64_t mis = int64_t(((reinterpret_cast<uintptr_t>(rowp) + uint64_t(s) * ES) & 15u) / ES);
  const int64_t h = mis == 0 ? s : (s + V - mis < e ? s + V - mis : e);  // first aligned column
  const int64_t t = h + (e - h) / V * V;                                  // last aligned column
  if (h > s && !few(s, h)) return;
  if (t > h) {
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rowp), 0, int(t * ES), 0x00020000);
    u32x4 b0[U], b1[U];
    auto issue = [&](u32x4 (&b)[U], int64_t cb) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, int((cb + int64_t(64 * u + lane) * V) * ES), 0, 0);
    };
    const uint32_t n = uint32_t(t - h);
    auto consume = [&](const u32x4 (&b)[U], int64_t cb) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c0 = cb + int64_t(64 * u + lane) * V;
        const uint32_t r0 = uint32_t(c0 - h);
        uint32_t bits[V], key[V];
        bool valid[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const uint32_t d = b[u][j * ES / 4];
          bits[j] = BF ? ((j & 1) ? (d & 0xFFFF0000u) : (d << 16)) : d;
          key[j] = rank_key(bits[j]);
          valid[j] = r0 + uint32_t(j) < n;
        }
        if (!body(key, bits, c0, valid)) return false;
      }
      return true;
    };
    int64_t cb = h;
    issue(b0, cb);
    for (;;) {
      issue(b1, cb + kStep);
      if (!consume(b0, cb)) return;
      if (cb + kStep >= t) break;
      issue(b0, cb + 2 * kStep);
      if (!consume(b1, cb + kStep)) return;
      if (cb + 2 * kStep >= t) break;
      cb += 2 * kStep;
    }
  }
  if (e > t && t >= h) few(t, e);
}

// A wave's share of a thresholded row: the aligned columns [h, t) (16-byte
// boundaries of the row), read as stream_window reads them, and every score
// that reaches tf (a number >= tf: the rank keys of numbers order like the
// numbers) appended to the stage with its window column, raw bits for now,
// in any order.  Places are reserved once per batch of U loads: a prefix
// sum of the lanes' counts and one LDS atomic.  A batch that would run past
// the stage is counted and not written (the row is then selected from
// memory).
template <bool BF>
__device__ __forceinline__ void stream_keep(const unsigned char* rowp, int64_t s, int64_t h, int64_t t, float tf,
                                            TbSmem& sm) {
  constexpr int ES = BF ? 2 : 4, V = 16 / ES, U = 4;
  constexpr int64_t kStep = 64 * V * U;
  const int lane = threadIdx.x & 63;
  if (t <= h) return;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rowp), 0, int(t * ES), 0x00020000);
  u32x4 b0[U], b1[U];
  auto issue = [&](u32x4 (&b)[U], int64_t cb) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      b[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, int((cb + int64_t(64 * u + lane) * V) * ES), 0, 0);
  };
  auto consume = [&](const u32x4 (&b)[U], int64_t cb) {
    uint32_t bits[U][V];
    bool keep[U][V];
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = cb + int64_t(64 * u + lane) * V < t;  // t is a vector boundary: whole vectors in or out
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const uint32_t d = b[u][j * ES / 4];
        bits[u][j] = BF ? ((j & 1) ? (d & 0xFFFF0000u) : (d << 16)) : d;
        keep[u][j] = in && __uint_as_float(bits[u][j]) >= tf;
        cnt += keep[u][j] ? 1u : 0u;
      }
    }
    const uint32_t incl = wave_scan(cnt);
    const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
    if (tot == 0) return;
    uint32_t base = 0;
    if (lane == 63) base = atomicAdd(&sm.count, tot);
    base = __builtin_amdgcn_readlane(base, 63);
    if (base + tot > uint32_t(kTbStage)) return;
    uint32_t pos = base + incl - cnt;
    const uint32_t c_lane = uint32_t(cb - s) + uint32_t(lane * V);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        if (keep[u][j]) {
          sm.key[pos] = bits[u][j];
          sm.col[pos] = uint16_t(c_lane + uint32_t(64 * u * V + j));
          ++pos;
        }
      }
    }
  };
  int64_t cb = h;
  issue(b0, cb);
  for (;;) {
    issue(b1, cb + kStep);
    consume(b0, cb);
    if (cb + kStep >= t) break;
    issue(b0, cb + 2 * kStep);
    consume(b1, cb + kStep);
    if (cb + 2 * kStep >= t) break;
    cb += 2 * kStep;
  }
}

template <bool BF>
__global__ void __launch_bounds__(kTbThreads) topk_rows_kernel(const unsigned char* plan, int32_t B, int32_t S_q,
                                                               int32_t S_k, int32_t H, int32_t D, const void* logits,
                                                               int64_t ld, int32_t k, int32_t* out_idx,
                                                               float* out_val, uint32_t off_start, uint32_t off_end) {
  __shared__ TbSmem sm;
  constexpr int ES = BF ? 2 : 4, V = 16 / ES;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = blockIdx.x;
  int32_t* oi = out_idx + row * k;
  float* ov = out_val != nullptr ? out_val + row * k : nullptr;
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(plan);
  if (!(hdr->magic == kPlanMagic && hdr->B == B && hdr->S_q == S_q && hdr->S_k == S_k && hdr->H == H &&
        hdr->D == D)) {  // a plan for other dimensions: loud, not plausible
    for (int i = t; i < k; i += kTbThreads) {
      oi[i] = -1;
      if (ov) ov[i] = __int_as_float(0x7FC00000);
    }
    return;
  }
  const int64_t s = reinterpret_cast<const int32_t*>(plan + off_start)[row];
  const int64_t e = reinterpret_cast<const int32_t*>(plan + off_end)[row];
  const int64_t n = e > s ? e - s : 0;
  const uint32_t n_out = uint32_t(n < k ? n : k);
  for (int i = int(n_out) + t; i < k; i += kTbThreads) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  if (n == 0) return;
  const unsigned char* rowp = static_cast<const unsigned char*>(logits) + row * ld * ES;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rowp), 0, int(e * ES), 0x00020000);
  auto bits_at = [&](int64_t c) -> uint32_t {  // score bits of column c < e
    if constexpr (BF)
      return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rs, int(c * 2), 0, 0)) << 16;
    else
      return __builtin_amdgcn_raw_buffer_load_b32(rs, int(c * 4), 0, 0);
  };
  constexpr int U = kTbStage / kTbThreads;  // 16 loads per thread in flight while staging
  if (n <= int64_t(k)) {  // the whole window
    for (int64_t i0 = 0; i0 < n; i0 += kTbThreads * U) {
      uint32_t b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + kTbThreads * u + t;
        b[u] = bits_at(s + (i < n ? i : n - 1));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + kTbThreads * u + t;
        if (i < n) {
          oi[i] = int32_t(s + i);
          if (ov) ov[i] = __uint_as_float(b[u]);
        }
      }
    }
    return;
  }
  const bool direct = n <= kTbStage;
  bool exact = false;
  uint32_t C = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
  if (direct) {  // every key of the window, key p = column s + p
    uint32_t b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = kTbThreads * u + t;
      b[u] = bits_at(s + (p < n ? p : n - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = kTbThreads * u + t;
      if (p < n) {
        const uint32_t key = rank_key(b[u]);
        sm.key[p] = b[u];
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
    C = uint32_t(n);
  } else {
    // the sample: the first 32 columns of every 512 of the window
    const int64_t ns = 32 * (n / 512) + (n % 512 < 32 ? n % 512 : 32);
    const int64_t m = sample_rank(n_out, n, ns);
    exact = ns > kTbStage || m >= ns;
    if (!exact) {
      uint32_t smin = 0xFFFFFFFFu, smax = 0u;
      uint32_t b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = kTbThreads * u + t < ns ? kTbThreads * u + t : ns - 1;
        b[u] = bits_at(s + 512 * (i / 32) + i % 32);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = kTbThreads * u + t;
        if (i < ns) {
          const uint32_t key = rank_key(b[u]);
          sm.key[i] = key;
          smin = min(smin, key);
          smax = max(smax, key);
        }
      }
      block_min_max<kTbWaves>(smin, smax, sm.mm);  // its barriers also complete the staging
      uint32_t ce, wl;
      const int hb = varying_bits(smin, smax);
      const uint32_t tau = radix_select<kTbThreads>(
          [&](auto fn) {
            for (int64_t i = t; i < ns; i += kTbThreads) fn(sm.key[i]);
          },
          uint32_t(m), sm.hist, sm.res, ce, wl, hb > 16 ? hb : 16, 16, smin);
      if (t == 0) sm.count = 0;
      __syncthreads();  // the sample is read; the candidates overwrite it
      // each wave a quarter of the window's aligned columns (the first wave
      // also the columns before them, the last the columns after), appending
      // the scores that reach tau.  tau = 0 keeps every score, NaN included:
      // that row is selected from memory
      const float tf = tau_value(tau);
      const int64_t mis = int64_t(((reinterpret_cast<uintptr_t>(rowp) + uint64_t(s) * ES) & 15u) / ES);
      const int64_t h = mis == 0 ? s : (s + V - mis < e ? s + V - mis : e);  // first aligned column
      const int64_t nv = (e - h) / V;                                         // aligned vectors
      const int64_t q0 = h + nv * wave / kTbWaves * V, q1 = h + nv * (wave + 1) / kTbWaves * V;
      // the unaligned columns before h and after the last vector: lane 0 of
      // the first and last waves, one by one
      auto few = [&](int64_t c, int64_t c_end) {
        if (lane == 0) {
          for (int64_t cc = c; cc < c_end; ++cc) {
            const uint32_t b = bits_at(cc);
            if (__uint_as_float(b) >= tf) {
              const uint32_t p = atomicAdd(&sm.count, 1u);
              if (p < uint32_t(kTbStage)) {
                sm.key[p] = b;
                sm.col[p] = uint16_t(cc - s);
              }
            }
          }
        }
      };
      if (tau != 0u) {
        if (wave == 0 && h > s) few(s, h);
        stream_keep<BF>(rowp, s, q0, q1, tf, sm);
        if (wave == kTbWaves - 1 && h + nv * V < e) few(h + nv * V, e);
      }
      __syncthreads();
      C = sm.count;
      exact = tau == 0u || C > uint32_t(kTbStage) || C < n_out;
      if (!exact) {  // the staged scores' key range
        for (uint32_t p = uint32_t(t); p < C; p += kTbThreads) {
          const uint32_t key = rank_key(sm.key[p]);
          kmin = min(kmin, key);
          kmax = max(kmax, key);
        }
      }
    }
  }

  int nbits = 1;
  while ((int64_t(1) << nbits) < n) ++nbits;
  const uint32_t top = (1u << nbits) - 1u;  // n <= 2^28
  if (!exact) {
    block_min_max<kTbWaves>(kmin, kmax, sm.mm);  // its barriers also complete the staging
    auto col_of = [&](uint32_t p) -> uint32_t { return direct ? p : uint32_t(sm.col[p]); };
    uint32_t T = 0, P2 = 0xFFFFFFFFu;  // selected: key > T, or key == T at column <= P2
    if (C > n_out) {
      uint32_t count_eq, want;
      T = radix_select<kTbThreads>(
          [&](auto fn) {
#pragma unroll 4
            for (uint32_t p = t; p < C; p += kTbThreads) fn(rank_key(sm.key[p]));
          },
          n_out, sm.hist, sm.res, count_eq, want, varying_bits(kmin, kmax), 0, kmin, true);
      if (want < count_eq) {  // ties at T: the want smallest columns among them
        uint32_t ce2, left2;
        const uint32_t Vs = radix_select<kTbThreads>(
            [&](auto fn) {
              for (uint32_t p = t; p < C; p += kTbThreads)
                if (rank_key(sm.key[p]) == T) fn(top - col_of(p));
            },
            want, sm.hist, sm.res, ce2, left2, nbits, 0, 0u, true);
        P2 = top - Vs;
      }
    }
    // the selection's columns, marked in a bitmap of the window; a column's
    // place in the output is the number of marked columns before it: the
    // selected columns of the words before its own (thread t sums words
    // [t W, t W + W), a prefix sum over the threads) and those below it in
    // its own word.  A thresholded row's selected scores are written there
    // from the stage, each with its column; a staged window (score of column
    // p at p) is listed in column order and written in order.
    const int words = int((n + 31) / 32);
    for (int i = t; i < words; i += kTbThreads) sm.bits[i] = 0;
    __syncthreads();
    auto selected = [&](uint32_t raw, uint32_t c) {
      const uint32_t key = rank_key(raw);
      return key > T || (key == T && c <= P2);
    };
#pragma unroll 4
    for (uint32_t p = t; p < C; p += kTbThreads) {
      const uint32_t c = col_of(p);
      if (selected(sm.key[p], c)) atomicOr(&sm.bits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    const int W = (words + kTbThreads - 1) / kTbThreads;
    uint32_t mine = 0;
    for (int j = 0; j < W; ++j) {
      const int wd = t * W + j;
      if (wd < words) mine += uint32_t(__builtin_popcount(sm.bits[wd]));
    }
    uint32_t total;
    uint32_t pos = block_scan<kTbWaves>(mine, sm.wsum, total) - mine;
    if (direct) {
      // column p's score is staged at p: list the selected columns in order
      // (in the unused column stage), then write the output in order
      for (int j = 0; j < W; ++j) {
        const int wd = t * W + j;
        uint32_t bw = wd < words ? sm.bits[wd] : 0u;
        while (bw != 0) {
          const int b = __builtin_ctz(bw);
          bw &= bw - 1u;
          if (pos < n_out) sm.col[pos] = uint16_t(32 * wd + b);
          ++pos;
        }
      }
      __syncthreads();
      for (uint32_t i = t; i < n_out; i += kTbThreads) {
        const uint32_t c = sm.col[i];
        oi[i] = int32_t(s + int64_t(c));
        if (ov) ov[i] = __uint_as_float(sm.key[c]);
      }
      return;
    }
    for (int j = 0; j < W; ++j) {
      const int wd = t * W + j;
      if (wd < words) {
        sm.wpre[wd] = uint16_t(pos);
        pos += uint32_t(__builtin_popcount(sm.bits[wd]));
      }
    }
    __syncthreads();
#pragma unroll 4
    for (uint32_t p = t; p < C; p += kTbThreads) {
      const uint32_t raw = sm.key[p], c = col_of(p);
      if (selected(raw, c)) {
        const uint32_t w = c >> 5;
        const uint32_t r = uint32_t(sm.wpre[w]) + uint32_t(__builtin_popcount(sm.bits[w] & ((1u << (c & 31)) - 1u)));
        if (r < n_out) {
          oi[r] = int32_t(s + int64_t(c));
          if (ov) ov[r] = __uint_as_float(raw);
        }
      }
    }
    return;
  }

  // ---- from memory, by the first wave: every pass streams the window ---------
  if (wave != 0) return;
  uint32_t* hist = sm.hist;  // two copies' worth, as a wave's radix select uses
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
  stream_window<BF>(rs, rowp, s, e, [&](const uint32_t* key, const uint32_t*, int64_t, const bool* valid) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (valid[j]) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
    }
    return true;
  });
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  uint32_t T, P2 = 0xFFFFFFFFu;
  {
    uint32_t count_eq, want;
    T = wave_radix_select(
        [&](auto fn) {
          stream_window<BF>(rs, rowp, s, e, [&](const uint32_t* key, const uint32_t*, int64_t, const bool* valid) {
#pragma unroll
            for (int j = 0; j < V; ++j)
              if (valid[j]) fn(key[j]);
            return true;
          });
        },
        n_out, hist, count_eq, want, varying_bits(kmin, kmax), 0, kmin, true);
    if (want < count_eq) {  // ties at T: the want smallest columns among them
      uint32_t ce2, left2;
      const uint32_t Vs = wave_radix_select(
          [&](auto fn) {
            stream_window<BF>(rs, rowp, s, e,
                              [&](const uint32_t* key, const uint32_t*, int64_t c0, const bool* valid) {
#pragma unroll
                                for (int j = 0; j < V; ++j)
                                  if (valid[j] && key[j] == T) fn(top - uint32_t(c0 + j - s));
                                return true;
                              });
          },
          want, hist, ce2, left2, nbits, 0, 0u, true);
      P2 = top - Vs;
    }
  }
  uint32_t done = 0;
  stream_window<BF>(rs, rowp, s, e, [&](const uint32_t* key, const uint32_t* bits, int64_t c0, const bool* valid) {
    uint32_t sel = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      sel |= uint32_t(valid[j] && (key[j] > T || (key[j] == T && uint32_t(c0 + j - s) <= P2))) << j;
    const uint32_t cnt = uint32_t(__builtin_popcount(sel));
    const uint32_t incl = wave_scan(cnt);
    uint32_t pos = done + incl - cnt;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      if (((sel >> j) & 1u) && pos < n_out) {
        oi[pos] = int32_t(c0 + j);
        if (ov) ov[pos] = __uint_as_float(bits[j]);
        ++pos;
      }
    }
    done += __builtin_amdgcn_readlane(incl, 63);
    return done < n_out;
  });
}

template <bool BF, bool BY_SCORE>
void launch_t(dim3 grid, const unsigned char* p, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
              const void* logits, int64_t ld, int32_t k, int32_t* out_idx, float* out_val, const PlanLayout& L,
              hipStream_t stream) {
  if (S_k > kChunk)
    hipLaunchKernelGGL((topk_kernel<BF, BY_SCORE, true>), grid, dim3(kTopkThreads), 0, stream, p, B, S_q, S_k, H, D,
                       logits, ld, k, out_idx, out_val, uint32_t(L.off_start), uint32_t(L.off_end));
  else
    hipLaunchKernelGGL((topk_kernel<BF, BY_SCORE, false>), grid, dim3(kTopkThreads), 0, stream, p, B, S_q, S_k, H, D,
                       logits, ld, k, out_idx, out_val, uint32_t(L.off_start), uint32_t(L.off_end));
}

}  // namespace

hipError_t launch_topk(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                       const void* logits, bool logits_bf16, int64_t ld, int32_t k, bool by_score,
                       int32_t* out_idx, float* out_val, hipStream_t stream) {
  const PlanLayout L = plan_layout(B, S_q, H);
  const unsigned char* p = static_cast<const unsigned char*>(plan);
  if (!by_score && int64_t(S_k) <= kTkMaxCols) {
    const dim3 g(unsigned(L.n_rows));
    if (logits_bf16)
      hipLaunchKernelGGL(topk_rows_kernel<true>, g, dim3(kTbThreads), 0, stream, p, B, S_q, S_k, H, D, logits, ld,
                         k, out_idx, out_val, uint32_t(L.off_start), uint32_t(L.off_end));
    else
      hipLaunchKernelGGL(topk_rows_kernel<false>, g, dim3(kTbThreads), 0, stream, p, B, S_q, S_k, H, D, logits, ld,
                         k, out_idx, out_val, uint32_t(L.off_start), uint32_t(L.off_end));
    return hipGetLastError();
  }
  const dim3 grid(unsigned(L.n_rows));
  if (logits_bf16) {
    if (by_score)
      launch_t<true, true>(grid, p, B, S_q, S_k, H, D, logits, ld, k, out_idx, out_val, L, stream);
    else
      launch_t<true, false>(grid, p, B, S_q, S_k, H, D, logits, ld, k, out_idx, out_val, L, stream);
  } else {
    if (by_score)
      launch_t<false, true>(grid, p, B, S_q, S_k, H, D, logits, ld, k, out_idx, out_val, L, stream);
    else
      launch_t<false, false>(grid, p, B, S_q, S_k, H, D, logits, ld, k, out_idx, out_val, L, stream);
  }
  return hipGetLastError();
}

}  // namespace idx
