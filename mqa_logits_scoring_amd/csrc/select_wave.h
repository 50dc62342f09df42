// Selection helpers shared by the top-k kernels (gfx950): radix selects over
// LDS histograms for one wave and for a workgroup, prefix sums and
// reductions over a wave's lanes or a workgroup's threads, and the sample
// rank of the thresholded selections.
#pragma once

#include "internal.h"

namespace idx {

// Lanes of the wave below this one whose bit is set in mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// Radix-select histograms of a wave: 256 bins in two lane-interleaved copies.
// Copy c of bin b is word c * kHistStride + b, so a bin's copies sit in
// different banks.
constexpr int kHistStride = 257;
constexpr int kWaveHistWords = 2 * kHistStride;

// Bits a radix select must look at when every key lies in [lo, hi]: those
// below the highest bit where lo and hi differ (keys that share their top
// bits would all land in one histogram bin, and LDS atomics on one address
// serialize).
__device__ __forceinline__ int varying_bits(uint32_t lo, uint32_t hi) {
  return lo == hi ? 8 : 32 - __builtin_clz(lo ^ hi);
}

// LDS written by some lanes of a wave and read by others: a wave's LDS
// accesses complete in order; the fence keeps the compiler from moving them
// across and waits for those outstanding.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = min(x, uint32_t(__shfl_xor(x, d, 64)));
  return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = max(x, uint32_t(__shfl_xor(x, d, 64)));
  return x;
}

// Inclusive prefix sum over the wave's lanes, in data-parallel moves between
// lanes (no LDS): within each row of 16 lanes by shifts of 1, 2, 4 and 8,
// then the last lane of row 0 added to row 1 and of row 2 to row 3, and the
// last lane of row 1 (by then the sum of rows 0 and 1) to rows 2 and 3.  A
// lane whose source is outside its row, or whose row the row mask leaves
// out, adds the 0 it starts from.
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xF, 0xF, false));  // row_shr:1
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xF, 0xF, false));  // row_shr:2
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xF, 0xF, false));  // row_shr:4
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xF, 0xF, false));  // row_shr:8
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xA, 0xF, false));  // row_bcast:15
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return x;
}

// A wave's radix select (as radix_select, over the wave's own histogram):
// for_each(fn) calls fn(key) for every key, from every lane.
template <typename ForEach>
__device__ __forceinline__ uint32_t wave_radix_select(ForEach for_each, uint32_t want, uint32_t* hist,
                                                      uint32_t& count_eq, uint32_t& want_left, int hi_bit,
                                                      int stop_bit, uint32_t prefix0, bool take_whole = false) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = hi_bit >= 32 ? 0u : prefix0 & ~((1u << hi_bit) - 1u);
  uint32_t pmask = hi_bit >= 32 ? 0u : ~((1u << hi_bit) - 1u);
  for (int hi = hi_bit; hi > stop_bit; hi -= 8) {
    const int lo = hi - 8 > stop_bit ? hi - 8 : stop_bit;
    const uint32_t dm = (1u << (hi - lo)) - 1u;
    for (int i = lane; i < kWaveHistWords; i += 64) hist[i] = 0;
    wave_sync();
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(lane & 1) * kHistStride + ((key >> lo) & dm)], 1u);
    });
    wave_sync();
    // lane l: bins 4l..4l+3; the lane whose bins hold the want-th key reports
    uint32_t h[4], own = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h[b] = hist[4 * lane + b] + hist[kHistStride + 4 * lane + b];
      own += h[b];
    }
    uint32_t x = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_down(x, d, 64);
      if (lane + d < 64) x += y;
    }
    const uint32_t above = x - own;
    const bool here = above < want && want <= x;
    uint32_t dig = 0, abv = 0, cnt = 0, cum = above;
    bool found = false;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (!found && cum + h[b] >= want) {
        dig = uint32_t(4 * lane + b);
        abv = cum;
        cnt = h[b];
        found = true;
      }
      cum += h[b];
    }
    const uint64_t who = __ballot(here);
    const int src = __builtin_ctzll(who);  // exactly one lane holds it
    const uint32_t d = __builtin_amdgcn_readlane(dig, src);
    want -= __builtin_amdgcn_readlane(abv, src);
    count_eq = __builtin_amdgcn_readlane(cnt, src);
    prefix |= d << lo;
    pmask |= dm << lo;
    wave_sync();  // the next pass clears the bins read here
    if (take_whole && want == count_eq) break;
  }
  want_left = want;
  return prefix;
}

// Sampled cells a row's threshold ranks: 1.25 times the share of the sample
// that the selection takes, plus 32.  With the sample's cells spread like the
// window's, the window then holds about 1.25 k + 32 R cells at or above the
// threshold (3072 for k = 2048, R = 16), with a spread of about R sqrt(m): it
// holds fewer than k (the row is scored again) or more than one wave keeps
// in LDS (the workgroup selection takes it) each about 4.6 spreads away.
__device__ __forceinline__ int64_t sample_rank(int64_t n_out, int64_t n, int64_t ns) {
  return (5 * n_out * ns + 4 * n - 1) / (4 * n) + 32;
}

// ---- workgroup-level ---------------------------------------------------------

// Inclusive prefix sum of v over a workgroup of NW waves (thread order);
// `total` receives the sum.  Contains barriers.
template <int NW>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  for (int w = 0; w < NW; ++w) {
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
// Minimum and maximum of per-thread values over a workgroup of NW waves
// (mm[0..2 NW) is scratch).  Contains barriers.
template <int NW>
__device__ __forceinline__ void block_min_max(uint32_t& lo, uint32_t& hi, uint32_t* mm) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    lo = min(lo, uint32_t(__shfl_xor(lo, d, 64)));
    hi = max(hi, uint32_t(__shfl_xor(hi, d, 64)));
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0) {
    mm[wave] = lo;
    mm[NW + wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, mm[w]);
    hi = max(hi, mm[NW + w]);
  }
  __syncthreads();
}

// Radix-select histograms: 256 bins in kHistCopies copies, lane l counting
// into copy l % kHistCopies, so that the lanes of one instruction that count
// the same digit mostly hit different words (LDS atomics on one word
// serialize).  Copy c of bin b is word c * kHistStride + b, which also puts a
// bin's copies in different banks.
constexpr int kHistCopies = 8;
constexpr int kHistWords = kHistCopies * kHistStride;

__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin) {
  atomicAdd(&hist[(threadIdx.x & (kHistCopies - 1)) * kHistStride + bin], 1u);
}

// Wave 0 over the histogram (bin = digit): the digit whose bin holds the
// want-th largest counted key (1 <= want <= keys counted), the keys in higher
// bins and the keys in its bin, into res[0..2].  Lane l reads bins 4l..4l+3;
// a suffix sum over the lanes gives each lane the count above it.
__device__ inline void find_bin256(const uint32_t* hist, uint32_t want, uint32_t* res) {
  const int lane = threadIdx.x;
  uint32_t h[4], own = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) x += hist[c * kHistStride + 4 * lane + b];
    h[b] = x;
    own += x;
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

// Radix select over keys, 8 bits per pass from bit hi_bit down to bit
// stop_bit: the want-th largest key (want >= 1) of those `for_each` visits,
// its bits below stop_bit cleared, with how many keys share its bits above
// and how many of those the want-th still takes (want_left).  for_each(fn)
// calls fn(key) for every key, from every thread, and may contain barriers.
// Bits above hi_bit are taken as given (prefix0, the same for every key).
// take_whole: stop after the pass whose digit's keys all belong to the want
// largest (want_left == count_eq); the result then has zeros below that
// digit, and the want largest keys are exactly those at or above it.
// NT: threads of the workgroup.
template <int NT, typename ForEach>
__device__ __forceinline__ uint32_t radix_select(ForEach for_each, uint32_t want, uint32_t* hist, uint32_t* res,
                                                 uint32_t& count_eq, uint32_t& want_left, int hi_bit = 32,
                                                 int stop_bit = 0, uint32_t prefix0 = 0, bool take_whole = false) {
  uint32_t prefix = hi_bit >= 32 ? 0u : prefix0 & ~((1u << hi_bit) - 1u);
  uint32_t pmask = hi_bit >= 32 ? 0u : ~((1u << hi_bit) - 1u);
  for (int hi = hi_bit; hi > stop_bit; hi -= 8) {
    const int lo = hi - 8 > stop_bit ? hi - 8 : stop_bit;
    const uint32_t dm = (1u << (hi - lo)) - 1u;
    for (int i = threadIdx.x; i < kHistWords; i += NT) hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) hist_add(hist, (key >> lo) & dm);
    });
    __syncthreads();
    if (threadIdx.x < 64) find_bin256(hist, want, res);
    __syncthreads();
    const uint32_t d = res[0];
    want -= res[1];
    count_eq = res[2];
    prefix |= d << lo;
    pmask |= dm << lo;
    if (take_whole && want == count_eq) break;
  }
  want_left = want;
  return prefix;
}

}  // namespace idx
