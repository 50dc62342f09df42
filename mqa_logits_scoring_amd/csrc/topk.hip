// Top-k selection over the scores of a scoring call (gfx950).
//
// For each query row, the k columns of its window with the largest scores,
// larger first, equal scores by smaller column, NaN after every number
// (+0 and -0 equal); columns past the window's size are -1 with score -inf.
// The sparse-attention page (FlashInfer SM120 sparse MLA, Summary and the
// DSv3.2 prefill notes) consumes such a per-query list of 2048 key indices;
// the pages do not say how it is chosen, so the ranking above is the plain
// one and the algorithm is this file's own.
//
// One workgroup per row.  Scores become 32-bit keys whose unsigned order is
// the ranking (sign-magnitude flipped to two's-complement-like order, -0
// folded onto +0, NaN to 0).  A radix select finds the k-th largest key T in
// three histogram passes over 12 + 12 + 8 key bits (4096 LDS bins, one atomic
// per candidate; each pass only counts keys that match the digits fixed so
// far).  When more keys equal T than the selection still needs, the same
// select runs on the column (smaller column = larger secondary key) among
// the keys equal to T.  The selected k are written to LDS as 64-bit (key,
// ~column) pairs and put in rank order by a bitonic sort.
//
// Layout: thread t of the workgroup holds columns s + ch*kChunk + m*kTopkThreads
// + t (m < kPerThread) of chunk ch, so every load instruction of a wave reads
// 64 consecutive scores.  Rows up to kChunk columns keep their keys in
// registers across the passes; longer rows read their chunks again in every
// pass (from L2).
#include "internal.h"

namespace idx {

namespace {

constexpr int kTopkThreads = 512;
constexpr int kPerThread = 64;
constexpr int kChunk = kTopkThreads * kPerThread;  // 32768 columns
constexpr int kBins = 4096;
constexpr int kTopkWaves = kTopkThreads / 64;
static_assert(kBins % kTopkThreads == 0, "every thread owns whole bins");
constexpr int kBinsPerThread = kBins / kTopkThreads;

// Unsigned order of the result = the ranking of the scores (NaN lowest).
__device__ __forceinline__ uint32_t rank_key(uint32_t u) {
  u = u == 0x80000000u ? 0u : u;                       // -0 ranks as +0
  const uint32_t k = (u >> 31) ? ~u : (u | 0x80000000u);
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0u : k;      // NaN
}

template <bool BF>
__device__ __forceinline__ uint32_t score_bits(const void* logits, int64_t i) {
  if constexpr (BF)
    return uint32_t(static_cast<const uint16_t*>(logits)[i]) << 16;
  else
    return static_cast<const uint32_t*>(logits)[i];
}

struct TopkSmem {
  uint32_t hist[kBins];
  uint64_t sel[kMaxTopK];
  uint32_t wsum[kTopkWaves];
  uint32_t digit, above, count, n_sel;
};

// Inclusive prefix sum of v over the workgroup's threads (thread order);
// `total` receives the sum over all threads.  Contains barriers.
__device__ uint32_t block_scan(uint32_t v, TopkSmem& sm, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

// One radix-select pass: among the candidates (cand(key2, ...) true), count the
// digit (key >> shift) & dmask, then find the digit d holding the want-th
// largest candidate.  Returns d; `above` = candidates with a larger digit,
// `count` = candidates with digit d.
struct PassResult {
  uint32_t digit, above, count;
};

__device__ PassResult find_digit(TopkSmem& sm, uint32_t want) {
  __syncthreads();  // histogram complete
  const int t = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int b = 0; b < kBinsPerThread; ++b) local += sm.hist[t * kBinsPerThread + b];
  uint32_t total;
  const uint32_t incl = block_scan(local, sm, total);
  const uint32_t above = total - incl;  // candidates in the bins of higher threads
  if (above < want && above + local >= want) {
    uint32_t cum = above;
    for (int b = kBinsPerThread - 1; b >= 0; --b) {
      const uint32_t h = sm.hist[t * kBinsPerThread + b];
      if (cum + h >= want) {
        sm.digit = uint32_t(t * kBinsPerThread + b);
        sm.above = cum;
        sm.count = h;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
  PassResult r{sm.digit, sm.above, sm.count};
  __syncthreads();  // the next pass may clear the bins and overwrite the result
  return r;
}

__device__ __forceinline__ void clear_hist(TopkSmem& sm) {
  for (int i = threadIdx.x; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
  __syncthreads();
}

template <bool BF>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const unsigned char* plan, int32_t B, int32_t S_q,
                                                             int32_t S_k, int32_t H, int32_t D, const void* logits,
                                                             int64_t ld, int32_t k, int32_t* out_idx,
                                                             float* out_val, uint32_t off_start, uint32_t off_end) {
  __shared__ TopkSmem sm;
  const int t = threadIdx.x;
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
  const int nch = int((n + kChunk - 1) / kChunk);

  // A chunk is read through a buffer resource based at its first column
  // (num_records = its width in bytes): the lane offset is the thread's, the
  // per-element offset a scalar constant, so addresses take no registers.
  constexpr int ES = BF ? 2 : 4;
  uint32_t key[kPerThread];
  auto load = [&](int ch) {
    const int64_t c0 = int64_t(ch) * kChunk;
    const int64_t w = n - c0 < kChunk ? n - c0 : kChunk;
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
      key[m] = rank_key(bits);  // past the chunk's width: never a candidate (m >= valid(ch))
    }
  };
  // elements m < valid(ch) of this thread lie inside the window (32-bit
  // arithmetic: a chunk is at most kChunk columns)
  auto valid = [&](int ch) {
    const int64_t w = n - int64_t(ch) * kChunk;
    const int wc = w < kChunk ? int(w) : kChunk;
    return wc > t ? (wc - t + kTopkThreads - 1) / kTopkThreads : 0;
  };

  // threshold: select key > T, and key == T with secondary key >= T2, where the
  // secondary key of column s + rel is (2^nbits - 1) - rel
  uint32_t T = 0, T2 = 0;
  int nbits = 0;
  if (n > k) {
    if (nch == 1) load(0);
    uint32_t want = uint32_t(k), prefix = 0, mask = 0, count_eq = 0;
#pragma unroll
    for (int p = 0; p < 3; ++p) {  // key bits [31:20], [19:8], [7:0]
      const int shift = p == 0 ? 20 : (p == 1 ? 8 : 0);
      const uint32_t dmask = p == 2 ? 0xFFu : 0xFFFu;
      clear_hist(sm);
      for (int ch = 0; ch < nch; ++ch) {
        if (nch > 1) load(ch);
        const int mv = valid(ch);
#pragma unroll
        for (int m = 0; m < kPerThread; ++m)
          if (m < mv && (key[m] & mask) == prefix) atomicAdd(&sm.hist[(key[m] >> shift) & dmask], 1u);
      }
      const PassResult r = find_digit(sm, want);
      want -= r.above;
      prefix |= r.digit << shift;
      mask |= dmask << shift;
      count_eq = r.count;
    }
    T = prefix;
    if (want < count_eq) {  // ties at T: the smallest columns among them
      while ((int64_t(1) << nbits) < n) ++nbits;
      const uint32_t top = nbits == 32 ? 0xFFFFFFFFu : (1u << nbits) - 1u;
      uint32_t prefix2 = 0, mask2 = 0;
      for (int hi = nbits; hi > 0; hi -= 12) {
        const int lo = hi > 12 ? hi - 12 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        clear_hist(sm);
        for (int ch = 0; ch < nch; ++ch) {
          if (nch > 1) load(ch);
          const int mv = valid(ch);
          const uint32_t k2c = top - uint32_t(ch) * kChunk - uint32_t(t);  // secondary key of element 0
#pragma unroll
          for (int m = 0; m < kPerThread; ++m) {
            const uint32_t k2 = k2c - uint32_t(m * kTopkThreads);
            if (m < mv && key[m] == T && (k2 & mask2) == prefix2) atomicAdd(&sm.hist[(k2 >> lo) & dmask], 1u);
          }
        }
        const PassResult r = find_digit(sm, want);
        want -= r.above;
        prefix2 |= r.digit << lo;
        mask2 |= dmask << lo;
      }
      T2 = prefix2;
    }
  }

  // gather the selection (exactly min(k, n) entries) as (key, ~column) pairs
  if (t == 0) sm.n_sel = 0;
  __syncthreads();
  const uint32_t top = nbits == 0 ? 0u : (nbits == 32 ? 0xFFFFFFFFu : (1u << nbits) - 1u);
  for (int ch = 0; ch < nch; ++ch) {
    if (nch > 1 || n <= k) load(ch);
    const int mv = valid(ch);
    const uint32_t rel0 = uint32_t(ch) * kChunk + uint32_t(t);  // column of element 0, past s
#pragma unroll
    for (int m = 0; m < kPerThread; ++m) {
      const uint32_t rel = rel0 + uint32_t(m * kTopkThreads);
      const bool take =
          m < mv && (n <= k || key[m] > T || (key[m] == T && (nbits == 0 || top - rel >= T2)));
      if (take) {
        const uint32_t pos = atomicAdd(&sm.n_sel, 1u);
        if (pos < uint32_t(kMaxTopK))  // exactly min(k, n) <= kMaxTopK by construction
          sm.sel[pos] = (uint64_t(key[m]) << 32) | uint64_t(0xFFFFFFFFu - rel);
      }
    }
  }
  __syncthreads();
  // pad to a power of two with 0 (below every real pair) and sort descending
  int P = 1;
  while (P < k) P <<= 1;
  const int n_sel = int(min(sm.n_sel, uint32_t(kMaxTopK)));
  for (int i = n_sel + t; i < P; i += kTopkThreads) sm.sel[i] = 0;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < P / 2; i += kTopkThreads) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool descending = (lo & size) == 0;
        const uint64_t x = sm.sel[lo], y = sm.sel[hi];
        if ((x < y) == descending) {
          sm.sel[lo] = y;
          sm.sel[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < k; i += kTopkThreads) {
    const uint64_t c = sm.sel[i];
    if (c == 0) {
      oi[i] = -1;
      if (ov) ov[i] = -__builtin_inff();
    } else {
      const int64_t col = s + int64_t(0xFFFFFFFFu - uint32_t(c));
      oi[i] = int32_t(col);
      if (ov) ov[i] = __uint_as_float(score_bits<BF>(logits, row * ld + col));
    }
  }
}

}  // namespace

hipError_t launch_topk(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                       const void* logits, bool logits_bf16, int64_t ld, int32_t k, int32_t* out_idx,
                       float* out_val, hipStream_t stream) {
  const PlanLayout L = plan_layout(B, S_q, H);
  const unsigned char* p = static_cast<const unsigned char*>(plan);
  const dim3 grid(unsigned(L.n_rows)), block(kTopkThreads);
  if (logits_bf16)
    hipLaunchKernelGGL(topk_kernel<true>, grid, block, 0, stream, p, B, S_q, S_k, H, D, logits, ld, k, out_idx,
                       out_val, uint32_t(L.off_start), uint32_t(L.off_end));
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, block, 0, stream, p, B, S_q, S_k, H, D, logits, ld, k, out_idx,
                       out_val, uint32_t(L.off_start), uint32_t(L.off_end));
  return hipGetLastError();
}

}  // namespace idx
