// Scoring kernel template for 8, 16 and 32 query heads per row (gfx950).
//
// Same score and same work decomposition as the 64-head kernel
// (score_kernel.h): a workgroup of 4 waves runs one tile and one chunk of key
// columns, K comes in fragment order one 32-column block ahead, and every
// 32-column block costs each wave four 32x32 MFMA blocks over d.  What
// changes with H is how the M dimension of those blocks is filled: a block
// covers 32 (row, head) pairs, that is 32/H rows of H heads, so a wave holds
// WR = 128/H rows and a tile 512/H.  The cudnn-frontend indexer page lists
// qhead_per_kv_head = 32 among its configurations and the DeepGEMM pull
// request 435 screen covers H = 8, 32 and 64 (Performance section); both
// share one K head across the H query heads as here.
//
// Epilogue: ReLU as a signed-integer max of the float's bits and one FMA per
// head (the weighted-query pieces of the 64-head kernels need four to eight
// extra A rows per query row, a whole extra MFMA block per wave at these H).
// Lane (c, g) of a 32x32 accumulator holds column c and the block's M rows
// 8(r/4) + 4g + r%4 in register r; with H <= 32 those rows belong to query
// row r / (16 / RPB) of the block whatever g is, so each lane keeps one
// partial sum per query row of its wave, and one permlane32 swap per pair of
// rows joins the lane halves' head sets and leaves row 2i + g in lane half g.
//
// Cleaning: when the call cleans, each wave writes -inf to its rows outside
// the tile's coverage after its last score store (the first chunk left of
// the coverage, the last chunk right of it), and the launch has no cleanup
// units.
#pragma once

#include "score_kernel.h"

namespace idx {

template <int H>
struct HeadTiling {
  static_assert(H == 8 || H == 16 || H == 32, "the 64-head kernel is score_kernel");
  static constexpr int RPB = 32 / H;     // query rows per 32x32 MFMA block
  static constexpr int NBLK = 4;         // MFMA blocks per wave per 32 key columns
  static constexpr int WR = NBLK * RPB;  // query rows per wave
  static constexpr int TR = 4 * WR;      // query rows per tile
  static constexpr int REGS = 16 / RPB;  // accumulator registers of one query row, per lane
  static_assert(TR == 512 / H, "a tile holds 512 (row, head) pairs");
};

// SEL: select mode (ScoreArgs::cand), as in the 64-head kernels.  At 8 heads
// a wave's 16 rows each carry a threshold and a count besides their windows,
// more than fits beside two waves per SIMD: that variant runs one.
template <int F, int H, bool SEL>
constexpr int gh_waves_per_eu() {
  return SEL && H == 8 ? 1 : waves_per_eu<F>();
}

template <int F, int H, bool WBF, bool OBF, bool CLEAN, bool SEL = false>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(gh_waves_per_eu<F, H, SEL>(), gh_waves_per_eu<F, H, SEL>())))
    score_kernel_gh(const ScoreArgs a) {
  static_assert(!SEL || !CLEAN, "select mode stores no scores");
  if constexpr (SEL) {
    if (a.gate != nullptr && *a.gate == 0) return;  // a second pass with no row to redo
  }
  using T = Fmt<F>;
  using HT = HeadTiling<H>;
  constexpr int WR = HT::WR, TR = HT::TR, RPB = HT::RPB, REGS = HT::REGS, NBLK = HT::NBLK;
  constexpr bool HAS_KS = T::MX || T::ROWSCALE;
  constexpr int QD = T::LB / 4;  // dwords per lane per (row, head)
  constexpr int KD = T::KB / 4;  // dwords per lane per k-step

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5, c = lane & 31;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == a.B && hdr->S_q == a.S_q && hdr->S_k == a.S_k &&
                       hdr->H == H && hdr->D == 128 && hdr->tile_rows == TR && hdr->n_tiles == a.n_tiles;
  // one work position per workgroup, dealt in order by the hardware
  const int pos = int(blockIdx.x);
  if (pos >= a.n_pos_compute) {
    cleanup_unit<OBF, CLEAN, TR>(a, pos - a.n_pos_compute, plan_ok);
    return;
  }
  // with no cleanup units in the launch, each wave cleans its own rows
  const bool own_clean = CLEAN && !SEL && units_clean_own_rows(a);
  if (!plan_ok) {
    if (own_clean && pos % a.n_chunk == 0) cleanup_unit<OBF, CLEAN, TR>(a, pos / a.n_chunk, false);
    return;
  }
  const Unit u = decode_unit(a, pos);
  if (u.kind != kUnitCompute) {
    if (own_clean && u.tile >= 0 && u.cl1 < a.S_k) {  // a tile whose rows all see nothing
      const int32_t* srow = reinterpret_cast<const int32_t*>(a.plan + a.off_slot) + int64_t(u.tile) * TR;
      for (int t = 0; t < WR; ++t) {
        const int r = __builtin_amdgcn_readfirstlane(srow[wave * WR + t]);
        if (r >= 0) clean_row_outside<OBF>(a, r, 0, 0, lane);
      }
    }
    return;
  }
  const int tile = u.tile, c0 = u.c0, c1 = u.c1;  // columns [c0, c1) of the tile are this unit's
  const int n_pairs = (c1 - c0 + 63) / 64;
  const int b = tile / a.tiles_per_batch;

  // ---- the wave's query rows (padding slots borrow the tile's first row and
  // store nothing) --------------------------------------------------------------
  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot) + int64_t(tile) * TR;
  const int32_t first_row = slot_row[0];
  int rows[WR];
  bool rvalid[WR];
#pragma unroll
  for (int t = 0; t < WR; ++t) {
    const int r = slot_row[wave * WR + t];
    rvalid[t] = r >= 0;
    rows[t] = r >= 0 ? r : first_row;
  }
  bool any_row = false;
#pragma unroll
  for (int t = 0; t < WR; ++t) any_row = any_row || rvalid[t];
  if (!any_row) return;  // padding rows only: nothing to store in this unit
  // select mode: the rows' thresholds; a wave whose rows keep nothing is done
  uint32_t tau_r[WR];
#pragma unroll
  for (int t = 0; t < WR; ++t) tau_r[t] = kTauNone;
  if constexpr (SEL) {
    bool any_sel = false;
#pragma unroll
    for (int t = 0; t < WR; ++t) {
      tau_r[t] = rvalid[t] ? a.tau[rows[t]] : kTauNone;
      any_sel = any_sel || tau_r[t] != kTauNone;
    }
    if (!any_sel) return;
  }

  // Q fragments: block j, M row c = (query row j*RPB + c/H, head c%H); the
  // row differs between lanes when H < 32, so its index is read per lane
  uint32_t qf[NBLK][QD];
  uint32_t sa[NBLK];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) {
    const int r = slot_row[wave * WR + j * RPB + c / H];
    const int64_t qrow = int64_t(r >= 0 ? r : first_row) * H + c % H;
    const unsigned char* src = static_cast<const unsigned char*>(a.q) + qrow * T::ROWB + g * T::CBASE;
#pragma unroll
    for (int v = 0; v < QD / 4; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + v * T::CSTRIDE);
      qf[j][4 * v + 0] = x.x;
      qf[j][4 * v + 1] = x.y;
      qf[j][4 * v + 2] = x.z;
      qf[j][4 * v + 3] = x.w;
    }
    if constexpr (T::MX) {
      const uint32_t word = static_cast<const uint32_t*>(a.q_scale)[qrow];
      sa[j] = g ? (word >> T::SCALE_SHIFT) : word;
    } else {
      sa[j] = 0;
    }
  }

  // weights: register r of block j is head (8(r/4) + 4g + r%4) % H of query
  // row j*RPB + r/REGS; four consecutive registers are four consecutive heads
  float wv[NBLK][16];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int t = j * RPB + (4 * q4) / REGS;
      const int64_t off = int64_t(rows[t]) * H + (8 * q4 + 4 * g) % H;
      if constexpr (WBF) {
        const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.w) + off);
        wv[j][4 * q4 + 0] = __uint_as_float(x.x << 16);
        wv[j][4 * q4 + 1] = __uint_as_float(x.x & 0xFFFF0000u);
        wv[j][4 * q4 + 2] = __uint_as_float(x.y << 16);
        wv[j][4 * q4 + 3] = __uint_as_float(x.y & 0xFFFF0000u);
      } else {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.w) + off);
        wv[j][4 * q4 + 0] = x.x;
        wv[j][4 * q4 + 1] = x.y;
        wv[j][4 * q4 + 2] = x.z;
        wv[j][4 * q4 + 3] = x.w;
      }
    }
  }

  // K fragments and scales, as in the 64-head kernel: buffer loads with the
  // block offset in a scalar register; blocks past the end of K are clamped
  // to the last one (in bounds, and the columns they feed are never stored)
  const int nblk = (a.S_k + 31) >> 5;
  const int kb0 = c0 >> 5;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(a.kfrag) + int64_t(b) * nblk * (32 * T::ROWB), 0, nblk * (32 * T::ROWB), kBufWord3);
  const __amdgpu_buffer_rsrc_t srs =
      HAS_KS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.kscale) + int64_t(b) * nblk * 64, 0,
                                                 nblk * 256, kBufWord3)
             : krs;
  auto kload = [&](int u, uint32_t (&bf)[QD], uint32_t& kword) {
    const int blk = min(kb0 + u, nblk - 1);
#pragma unroll
    for (int v = 0; v < QD / 4; ++v) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, lane * 16 + v * 1024, blk * (32 * T::ROWB), 0);
      bf[4 * v + 0] = x[0];
      bf[4 * v + 1] = x[1];
      bf[4 * v + 2] = x[2];
      bf[4 * v + 3] = x[3];
    }
    if constexpr (HAS_KS) kword = __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, blk * 256, 0);
  };

  // one 32x32 block over all of d: acc = Q(block j) x K(32 columns)^T
  auto mfma_block = [&](f32x16& acc, const uint32_t (&q)[QD], uint32_t sA, const uint32_t (&bf)[QD],
                        uint32_t sB) {
    f32x16 d = {};
#pragma unroll
    for (int s = 0; s < T::KSTEPS; ++s) {
      if constexpr (bf16_operands(F)) {
        bf16x8 av, bv;
        __builtin_memcpy(&av, &q[s * KD], 16);
        __builtin_memcpy(&bv, &bf[s * KD], 16);
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, d, 0, 0, 0);
      } else {
        i32x8 av = {}, bv = {};
#pragma unroll
        for (int e = 0; e < KD; ++e) {
          av[e] = int(q[s * KD + e]);
          bv[e] = int(bf[s * KD + e]);
        }
        if constexpr (T::MX) {
          constexpr int OS = T::OPSEL_STEP;
          if (s == 0)
            d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, 0, sA, 0, sB);
          else
            d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, OS, sA, OS, sB);
        } else {
          d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, 0, 127, 0, 127);
        }
      }
    }
    acc = d;
  };

  // Stores: round i writes row 2i + g from lane half g, through one buffer
  // resource per row based at the unit's first column (num_records = the
  // unit's width, 0 for a padding row), the other half's lanes dropped by an
  // offset with the top bit set; -inf picked byte-wise by v_perm_b32, never by
  // a branch (see the 64-head kernel for why).
  // (select mode: in columns, with the pair's threshold and candidate count)
  constexpr int ES = OBF ? 2 : 4;
  constexpr int EW = SEL ? 1 : ES;
  constexpr uint32_t kDrop = 0x80000000u;
  const uint32_t half0 = g ? kDrop : 0u, half1 = g ? 0u : kDrop;
  uint32_t s_rel[WR / 2], w_len[WR / 2], sel_cnt[WR];
#pragma unroll
  for (int i = 0; i < WR / 2; ++i) {
    const int my_row = g ? rows[2 * i + 1] : rows[2 * i];
    const int my_s = reinterpret_cast<const int32_t*>(a.plan + a.off_start)[my_row];
    const int my_e = reinterpret_cast<const int32_t*>(a.plan + a.off_end)[my_row];
    if constexpr (SEL) {
      sel_window(my_s, my_e, c0, c1, s_rel[i], w_len[i]);
    } else {
      s_rel[i] = uint32_t(my_s - c0) * EW;
      w_len[i] = uint32_t(max(my_e - my_s, 0)) * EW;
    }
  }
#pragma unroll
  for (int t = 0; t < WR; ++t) sel_cnt[t] = 0;
  auto out_rsrc = [&](int t) {
    return __builtin_amdgcn_make_buffer_rsrc(static_cast<unsigned char*>(a.out) + (int64_t(rows[t]) * a.ld + c0) * ES,
                                             0, rvalid[t] ? (c1 - c0) * ES : 0, kBufWord3);
  };
  auto store_pair = [&](float v, int u, int i) {
    if constexpr (SEL) {
      sel_emit<OBF>(v, u, c, g, uint32_t(c0), s_rel[i], w_len[i], sel_tau(tau_r[2 * i], tau_r[2 * i + 1]),
                    sel_cnt[2 * i], sel_cnt[2 * i + 1], sel_rsrc(a, rows[2 * i], rvalid[2 * i], c0, c1 - c0),
                    sel_rsrc(a, rows[2 * i + 1], rvalid[2 * i + 1], c0, c1 - c0));
      return;
    }
    const uint32_t off = uint32_t(32 * u + c) * ES;  // u = -1 wraps to a huge offset: dropped
    const bool inwin = off - s_rel[i] < w_len[i];
    uint32_t o0 = off | half0, o1 = off | half1;
    if constexpr (!CLEAN) {
      o0 = inwin ? o0 : kDrop;
      o1 = inwin ? o1 : kDrop;
    }
    float val = v;
    if constexpr (CLEAN)
      val = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(v), 0xFF800000u,
                                                  inwin ? 0x07060504u : 0x03020100u));
    if constexpr (OBF) {
      const uint16_t h = __builtin_bit_cast(uint16_t, static_cast<__bf16>(val));  // round to nearest even
      // cached, as in score_kernel: the line's other half comes with the next block
      __builtin_amdgcn_raw_buffer_store_b16(h, out_rsrc(2 * i), int(o0), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(h, out_rsrc(2 * i + 1), int(o1), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), out_rsrc(2 * i), int(o0), 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), out_rsrc(2 * i + 1), int(o1), 0, kNonTemporal);
    }
  };

  // With H <= 16 every block holds whole rows of its own (RPB of them), with
  // H = 32 two consecutive blocks hold a row pair: rows are finished and
  // stored as soon as the blocks holding them are summed, so a lane keeps
  // only PR partial sums.
  constexpr int PR = RPB >= 2 ? RPB : 2;
  float p[PR];
#pragma unroll
  for (int t = 0; t < PR; ++t) p[t] = 0.f;
  // weighted ReLU of block j's registers into the partial sums of their rows
  auto epi = [&](const f32x16& acc, const float (&w)[16], int j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = RPB >= 2 ? r / REGS : j % 2;
      p[t] = __builtin_fmaf(w[r], __int_as_float(max(__float_as_int(acc[r]), 0)), p[t]);
    }
  };
  // after block j: join the lane halves of each finished row pair, scale,
  // store it at column block u, restart its sums
  auto finish = [&](int j, int u, float kscl) {
    if (RPB == 1 && j % 2 == 0) return;
    float scale = a.sm_scale;
    if constexpr (T::ROWSCALE) scale *= kscl;
#pragma unroll
    for (int i = 0; i < PR / 2; ++i) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[2 * i]), __float_as_uint(p[2 * i + 1]),
                                                       false, false);
      store_pair((__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * scale, u, (j * RPB) / 2 + i);
    }
#pragma unroll
    for (int t = 0; t < PR; ++t) p[t] = 0.f;
  };

  // Pipelined as in the 64-head kernel: each MFMA block runs while the
  // epilogue of the previous one executes, two accumulators alternating; block
  // 3 of column block u - 1 is summed and stored under block 0 of u.
  f32x16 accA = {}, accB = {};
  float kprev = 1.f;
  auto block = [&](const uint32_t (&bf)[QD], uint32_t kword, int u) {
    const float kcur = __uint_as_float(kword);
    mfma_block(accA, qf[0], sa[0], bf, kword);  // block 0 of u     ||
    epi(accB, wv[3], 3);                         //   block 3 of u-1
    finish(3, u - 1, kprev);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(accB, qf[1], sa[1], bf, kword);  // block 1          ||
    epi(accA, wv[0], 0);                         //   block 0
    finish(0, u, kcur);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(accA, qf[2], sa[2], bf, kword);  // block 2          ||
    epi(accB, wv[1], 1);                         //   block 1
    finish(1, u, kcur);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(accB, qf[3], sa[3], bf, kword);  // block 3          ||
    epi(accA, wv[2], 2);                         //   block 2
    finish(2, u, kcur);
    __builtin_amdgcn_sched_barrier(0);
    kprev = kcur;
  };
  constexpr int NB = kfrag_ring<F>();
  uint32_t bfs[NB][QD];
  uint32_t kws[NB] = {};
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) kload(i, bfs[i], kws[i]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const int n_iter = (2 * n_pairs + NB - 1) / NB;
  for (int s = 0; s < n_iter; ++s) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = NB * s + i;
      kload(u + NB - 1, bfs[(i + NB - 1) % NB], kws[(i + NB - 1) % NB]);
      block(bfs[i], kws[i], u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  epi(accB, wv[3], 3);
  finish(3, NB * n_iter - 1, kprev);
  if constexpr (SEL) {
#pragma unroll
    for (int i = 0; i < WR / 2; ++i)
      if (c == 0 && (g ? rvalid[2 * i + 1] : rvalid[2 * i]))
        sel_finish(a, g ? rows[2 * i + 1] : rows[2 * i], u.chunk, c0, g ? sel_cnt[2 * i + 1] : sel_cnt[2 * i]);
  }
  if (own_clean) {
#pragma unroll
    for (int t = 0; t < WR; ++t)
      if (rvalid[t]) clean_row_outside<OBF>(a, rows[t], u.cl0, u.cl1, lane);
  }
}

template <int F, int H, bool WBF, bool OBF, bool CLEAN>
hipError_t launch_score_gh_t(const ScoreArgs& a, hipStream_t stream) {
  if (a.cand != nullptr) {  // select mode: launched without cleaning
    if constexpr (CLEAN)
      return hipErrorInvalidValue;
    else
      return launch_units(score_kernel_gh<F, H, WBF, OBF, false, true>, a, stream);
  }
  // each wave cleans its own rows: no cleanup units
  ScoreArgs own = a;
  if (CLEAN) own.n_positions = a.n_pos_compute;
  return launch_units(score_kernel_gh<F, H, WBF, OBF, CLEAN>, own, stream);
}

// Every weight type x output type x clean flag of one format and head count.
template <int F, int H>
hipError_t launch_score_heads(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                              hipStream_t stream) {
  const bool wb = w_dtype == IDX_BF16, ob = out_dtype == IDX_BF16;
  if constexpr (H == 64) {
    if (wb) {
      if (ob) return clean ? launch_score_t<F, true, true, true>(a, stream) : launch_score_t<F, true, true, false>(a, stream);
      return clean ? launch_score_t<F, true, false, true>(a, stream) : launch_score_t<F, true, false, false>(a, stream);
    }
    if (ob) return clean ? launch_score_t<F, false, true, true>(a, stream) : launch_score_t<F, false, true, false>(a, stream);
    return clean ? launch_score_t<F, false, false, true>(a, stream) : launch_score_t<F, false, false, false>(a, stream);
  } else {
    if (wb) {
      if (ob) return clean ? launch_score_gh_t<F, H, true, true, true>(a, stream)
                           : launch_score_gh_t<F, H, true, true, false>(a, stream);
      return clean ? launch_score_gh_t<F, H, true, false, true>(a, stream)
                   : launch_score_gh_t<F, H, true, false, false>(a, stream);
    }
    if (ob) return clean ? launch_score_gh_t<F, H, false, true, true>(a, stream)
                         : launch_score_gh_t<F, H, false, true, false>(a, stream);
    return clean ? launch_score_gh_t<F, H, false, false, true>(a, stream)
                 : launch_score_gh_t<F, H, false, false, false>(a, stream);
  }
}

// Dispatch on the head count of the call (checked by the host API).
template <int F>
hipError_t launch_score_fmt(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                            hipStream_t stream) {
  switch (a.H) {
    case 64: return launch_score_heads<F, 64>(w_dtype, out_dtype, clean, a, stream);
    case 32: return launch_score_heads<F, 32>(w_dtype, out_dtype, clean, a, stream);
    case 16: return launch_score_heads<F, 16>(w_dtype, out_dtype, clean, a, stream);
    case 8: return launch_score_heads<F, 8>(w_dtype, out_dtype, clean, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace idx
