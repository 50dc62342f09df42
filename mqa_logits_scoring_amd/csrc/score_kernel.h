// Scoring kernel template for gfx950 (CDNA4).
//
// Computes, for the rows of one tile and one chunk of key columns,
//   out[i, j] = sm_scale * sum_h w[i,h] * max(0, q[i,h,:] . k[j,:])
// (the lightning-indexer score; see include/idx_logits.h for where the pages
// define it) and writes -inf to the tile's in-coverage cells outside a row's
// window when cleaning.  Cells outside the tile's coverage are written by
// cleanup units that run after the compute units in the same grid, so cleanup
// never competes with the matrix work of a compute unit (the placement lesson
// of DeepGEMM pull request 435, Investigation notes).
//
// Work decomposition
//   workgroup = 4 waves = one tile of kTileRows query rows x one key chunk
//   wave      = TW query rows; for each row its Q (64 heads x 128 d) sits in
//               registers for the whole chunk, as A operands of 32x32 MFMAs
//               (heads on the M dimension)
//   key chunk = stages of 64 columns, staged through LDS (double buffered) and
//               shared by the four waves; each stage is two 32-column blocks
//               that are the B operands (key columns on N)
//   epilogue  = in registers: lane l of the 32x32 accumulator holds column
//               l%32 and 16 heads per M block; ReLU, weight and sum its 32
//               heads, then one permlane32 swap joins the two lane halves
//               (heads differ between halves, the column does not) and leaves
//               one row's 32 consecutive columns per half-wave, stored
//               coalesced.  The epilogue of one 32-column block is issued
//               between the MFMAs of the next, so vector ALU and matrix
//               pipes overlap (cudnn-frontend pull request 416 keeps its
//               head-sum register-resident for the same reason, Why section).
//
// Operand layout inside a lane: any permutation of d applied alike to Q and K
// leaves every dot product unchanged, so each format places d where loads are
// wide and where the MFMA's block scales line up with the E8M0 bytes.  Lane
// (c = l%32, g = l/32) holds LB bytes of its Q row (head c) and K row (column
// c) as 16-byte chunks; Fmt<> gives their offsets, the k-steps that use them,
// and how the scale word is shifted per lane half so that op_sel picks the
// right E8M0 byte (the placement of the scaled f8f6f4 MFMA differs between
// e4m3 and e2m1 operands, see Fmt<>).
#pragma once

#include "internal.h"

namespace idx {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int F>
struct Fmt;
// ROWB: bytes per Q/K row of 128 elements; LB: bytes one lane holds of a row,
// as LB/16 chunks of 16 bytes, chunk t at row byte CBASE*g + CSTRIDE*t;
// KSTEPS: MFMA k-steps per 32x32 block over d; KB: bytes per lane per k-step
// (k-step s uses chunks [s*KB/16, (s+1)*KB/16)).
// MX: SCALE_SHIFT is the right shift of the scale word for lane half g = 1,
// OPSEL_STEP the op_sel byte step per k-step.
template <>
struct Fmt<IDX_IN_BF16> {
  static constexpr int ROWB = 256, LB = 128, KSTEPS = 8, KB = 16, CBASE = 128, CSTRIDE = 16;
  static constexpr bool MX = false, ROWSCALE = false;
};
// e4m3 in the 32x32x64 f8f6f4 MFMA: bytes 0-15 of both lane halves form one
// 32-element block (scaled by lane half 0's scale), bytes 16-31 the other
// (lane half 1's scale).  Lane half g therefore holds 16-byte chunks at
// 16*g + 32*t: k-step s pairs block 2s (chunk 2s) with block 2s+1 (chunk 2s+1).
template <>
struct Fmt<IDX_IN_FP8_E4M3> {
  static constexpr int ROWB = 128, LB = 64, KSTEPS = 2, KB = 32, CBASE = 16, CSTRIDE = 32;
  static constexpr bool MX = false, ROWSCALE = true;
  static constexpr int CODE = 0;  // f8f6f4 operand format: e4m3
};
template <>
struct Fmt<IDX_IN_MXFP8_E4M3> {
  static constexpr int ROWB = 128, LB = 64, KSTEPS = 2, KB = 32, CBASE = 16, CSTRIDE = 32;
  static constexpr bool MX = true, ROWSCALE = false;
  static constexpr int CODE = 0;
  // lane half g scales block 2s+g at k-step s: byte 2s of (word >> 8g)
  static constexpr int SCALE_SHIFT = 8, OPSEL_STEP = 2;
};
// e2m1 in the same MFMA: each lane half's 16 bytes are one whole 32-element
// block scaled by its own lane's scale, so lane half g holds bytes
// [32g, 32g+32) and k-step s is block 2g+s: byte s of (word >> 16g).
template <>
struct Fmt<IDX_IN_MXFP4_E2M1> {
  static constexpr int ROWB = 64, LB = 32, KSTEPS = 2, KB = 16, CBASE = 32, CSTRIDE = 16;
  static constexpr bool MX = true, ROWSCALE = false;
  static constexpr int CODE = 4;  // f8f6f4 operand format: e2m1
  static constexpr int SCALE_SHIFT = 16, OPSEL_STEP = 1;
};

constexpr int kStageCols = 64;
constexpr int kThreads = 256;

template <bool OBF>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OBF) {
    // round to nearest even, NaN kept quiet
    uint32_t u = __float_as_uint(v);
    uint32_t r = ((u >> 16) & 1u) + 0x7FFFu;
    uint16_t h = (u & 0x7FFFFFFFu) > 0x7F800000u ? uint16_t((u >> 16) | 0x40u) : uint16_t((u + r) >> 16);
    static_cast<uint16_t*>(out)[idx] = h;
  } else {
    static_cast<float*>(out)[idx] = v;
  }
}

// Cells of a tile's rows outside its computed coverage: -inf when cleaning.
// With a plan that does not match the call, every row of the tile is filled
// with quiet NaN instead, so the mismatch cannot pass unnoticed.
template <bool OBF, bool CLEAN>
__device__ void cleanup_unit(const ScoreArgs& a, int tile, bool plan_ok) {
  if (plan_ok && !CLEAN) return;
  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
  int lo = 0, hi = 0;
  float fill = __int_as_float(0x7FC00000);
  if (plan_ok) {
    lo = reinterpret_cast<const int32_t*>(a.plan + a.off_lo)[tile];
    hi = reinterpret_cast<const int32_t*>(a.plan + a.off_hi)[tile];
    fill = -__builtin_inff();
  }
  const int tpb = a.tiles_per_batch;
  for (int r = 0; r < kTileRows; ++r) {
    int64_t row;
    if (plan_ok) {
      row = slot_row[int64_t(tile) * kTileRows + r];
      if (row < 0) continue;
    } else {
      const int64_t i = int64_t(tile % tpb) * kTileRows + r;
      if (i >= a.S_q) continue;
      row = int64_t(tile / tpb) * a.S_q + i;
    }
    const int64_t base = row * a.ld;
    for (int j = threadIdx.x; j < lo; j += kThreads) store_out<OBF>(a.out, base + j, fill);
    for (int j = hi + threadIdx.x; j < a.S_k; j += kThreads) store_out<OBF>(a.out, base + j, fill);
  }
}

template <int F, bool WBF, bool OBF, bool CLEAN, int TW>
__global__ void __launch_bounds__(kThreads, 1) score_kernel(const ScoreArgs a) {
  using T = Fmt<F>;
  static_assert(TW == 1 || TW == 2, "one or two query rows per wave");
  static_assert(4 * TW == kTileRows, "four waves cover one tile");
  constexpr int STRIDE = T::ROWB + 16;  // padded LDS row: conflict-free 16-byte lane reads
  constexpr bool HAS_KS = T::MX || T::ROWSCALE;
  constexpr int STAGE_BYTES = kStageCols * STRIDE + kStageCols * 4;
  constexpr int CPR = T::ROWB / 16;                  // 16-byte chunks per K row
  constexpr int NCH = kStageCols * CPR / kThreads;   // chunks per thread per stage
  constexpr int QD = T::LB / 4;                      // dwords per lane per row
  constexpr int KD = T::KB / 4;                      // dwords per lane per k-step
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, c = lane & 31;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == a.B && hdr->S_q == a.S_q && hdr->S_k == a.S_k &&
                       hdr->H == 64 && hdr->D == 128 && hdr->tile_rows == kTileRows && hdr->n_tiles == a.n_tiles;
  const int bid = blockIdx.x;
  if (bid >= a.n_compute) {
    cleanup_unit<OBF, CLEAN>(a, bid - a.n_compute, plan_ok);
    return;
  }
  if (!plan_ok) return;

  // longest tiles first for causal windows: the last rows see the most keys
  const int tile = a.n_tiles - 1 - bid / a.n_chunks;
  const int chunk = bid % a.n_chunks;
  const int lo = reinterpret_cast<const int32_t*>(a.plan + a.off_lo)[tile];
  const int hi = reinterpret_cast<const int32_t*>(a.plan + a.off_hi)[tile];
  const int c0 = lo + chunk * a.chunk_cols;
  if (c0 >= hi) return;
  const int c1 = min(hi, c0 + a.chunk_cols);
  const int n_stages = (c1 - c0 + kStageCols - 1) / kStageCols;
  const int b = tile / a.tiles_per_batch;

  // ---- the wave's query rows ----------------------------------------------
  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
  const int32_t first_row = slot_row[int64_t(tile) * kTileRows];
  int rows[TW];
  bool rvalid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int r = slot_row[int64_t(tile) * kTileRows + wave * TW + t];
    rvalid[t] = r >= 0;
    rows[t] = r >= 0 ? r : first_row;
  }

  // Q fragments: qf[t][mb] = lane's LB bytes of head 32*mb + c, from byte g*LB
  uint32_t qf[TW][2][QD];
  uint32_t sa[TW][2];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int64_t qrow = int64_t(rows[t]) * 64 + 32 * mb + c;
      const unsigned char* src = static_cast<const unsigned char*>(a.q) + qrow * T::ROWB + g * T::CBASE;
#pragma unroll
      for (int v = 0; v < QD / 4; ++v) {
        const uint4 x = *reinterpret_cast<const uint4*>(src + v * T::CSTRIDE);
        qf[t][mb][4 * v + 0] = x.x;
        qf[t][mb][4 * v + 1] = x.y;
        qf[t][mb][4 * v + 2] = x.z;
        qf[t][mb][4 * v + 3] = x.w;
      }
      if constexpr (T::MX) {
        const uint32_t word = static_cast<const uint32_t*>(a.q_scale)[qrow];
        sa[t][mb] = g ? (word >> T::SCALE_SHIFT) : word;
      } else {
        sa[t][mb] = 0;
      }
    }
  }

  // weights of the lane's 32 heads: head 32*mb + 8*(r/4) + 4*g + r%4 for reg r
  float wv[TW][2][16];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int64_t off = int64_t(rows[t]) * 64 + 32 * mb + 8 * q4 + 4 * g;
        if constexpr (WBF) {
          const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.w) + off);
          wv[t][mb][4 * q4 + 0] = __uint_as_float(x.x << 16);
          wv[t][mb][4 * q4 + 1] = __uint_as_float(x.x & 0xFFFF0000u);
          wv[t][mb][4 * q4 + 2] = __uint_as_float(x.y << 16);
          wv[t][mb][4 * q4 + 3] = __uint_as_float(x.y & 0xFFFF0000u);
        } else {
          const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.w) + off);
          wv[t][mb][4 * q4 + 0] = x.x;
          wv[t][mb][4 * q4 + 1] = x.y;
          wv[t][mb][4 * q4 + 2] = x.z;
          wv[t][mb][4 * q4 + 3] = x.w;
        }
      }
    }
  }

  // the row this lane stores: half-wave g stores row t = g (TW = 2); with one
  // row per wave only the low half stores
  const int my_t = (TW == 2) ? g : 0;
  const bool my_valid = (TW == 2) ? (g ? rvalid[TW - 1] : rvalid[0]) : (rvalid[0] && g == 0);
  const int my_row = (TW == 2) ? (g ? rows[TW - 1] : rows[0]) : rows[0];
  (void)my_t;
  const int my_s = reinterpret_cast<const int32_t*>(a.plan + a.off_start)[my_row];
  const int my_e = reinterpret_cast<const int32_t*>(a.plan + a.off_end)[my_row];
  const int64_t obase = int64_t(my_row) * a.ld;

  const unsigned char* kb = static_cast<const unsigned char*>(a.k) + int64_t(b) * a.S_k * T::ROWB;
  const uint32_t* ksb = HAS_KS ? static_cast<const uint32_t*>(a.k_scale) + int64_t(b) * a.S_k : nullptr;

  // ---- stage staging: global -> registers -> LDS -----------------------------
  uint4 stg[NCH];
  uint32_t stg_s = 0;
  auto gload = [&](int s) {
    const int jb = c0 + s * kStageCols;
#pragma unroll
    for (int v = 0; v < NCH; ++v) {
      const int qq = tid + kThreads * v;
      const int j = jb + qq / CPR;
      stg[v] = j < a.S_k ? reinterpret_cast<const uint4*>(kb + int64_t(j) * T::ROWB)[qq % CPR]
                         : make_uint4(0, 0, 0, 0);
    }
    if constexpr (HAS_KS) {
      if (tid < kStageCols) {
        const int j = jb + tid;
        stg_s = j < a.S_k ? ksb[j] : 0u;
      }
    }
  };
  auto swrite = [&](int buf) {
    unsigned char* base = lds + buf * STAGE_BYTES;
#pragma unroll
    for (int v = 0; v < NCH; ++v) {
      const int qq = tid + kThreads * v;
      *reinterpret_cast<uint4*>(base + (qq / CPR) * STRIDE + (qq % CPR) * 16) = stg[v];
    }
    if constexpr (HAS_KS) {
      if (tid < kStageCols) *reinterpret_cast<uint32_t*>(base + kStageCols * STRIDE + tid * 4) = stg_s;
    }
  };

  // B operand of 32-column block u of a stage, plus the column's scale word
  auto bread = [&](int buf, int u, uint32_t (&bf)[QD], uint32_t& sb, float& kscl) {
    const unsigned char* base = lds + buf * STAGE_BYTES;
    const unsigned char* p = base + (32 * u + c) * STRIDE + g * T::CBASE;
#pragma unroll
    for (int v = 0; v < QD / 4; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + v * T::CSTRIDE);
      bf[4 * v + 0] = x.x;
      bf[4 * v + 1] = x.y;
      bf[4 * v + 2] = x.z;
      bf[4 * v + 3] = x.w;
    }
    if constexpr (HAS_KS) {
      const uint32_t word = *reinterpret_cast<const uint32_t*>(base + kStageCols * STRIDE + (32 * u + c) * 4);
      if constexpr (T::MX) sb = g ? (word >> T::SCALE_SHIFT) : word;
      if constexpr (T::ROWSCALE) kscl = __uint_as_float(word);
    }
  };

  auto mma = [&](f32x16 (&acc)[TW][2], const uint32_t (&bf)[QD], uint32_t sb) {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 d = {};
#pragma unroll
        for (int s = 0; s < T::KSTEPS; ++s) {
          if constexpr (F == IDX_IN_BF16) {
            bf16x8 av, bv;
            __builtin_memcpy(&av, &qf[t][mb][s * KD], 16);
            __builtin_memcpy(&bv, &bf[s * KD], 16);
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, d, 0, 0, 0);
          } else {
            i32x8 av = {}, bv = {};
#pragma unroll
            for (int e = 0; e < KD; ++e) {
              av[e] = int(qf[t][mb][s * KD + e]);
              bv[e] = int(bf[s * KD + e]);
            }
            if constexpr (T::MX) {
              constexpr int OS = T::OPSEL_STEP;
              if (s == 0)
                d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, 0, sa[t][mb], 0, sb);
              else
                d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, OS, sa[t][mb], OS,
                                                                    sb);
            } else {
              d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, d, T::CODE, T::CODE, 0, 127, 0, 127);
            }
          }
        }
        acc[t][mb] = d;
      }
    }
  };

  auto epi = [&](const f32x16 (&acc)[TW][2], int jbase, float kscl) {
    float p[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      float s = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s = __builtin_fmaf(wv[t][mb][r], __builtin_fmaxf(acc[t][mb][r], 0.f), s);
      }
      p[t] = s;
    }
    // lanes c and c+32 hold the same column for different heads: swap the
    // upper half of row 0's partial with the lower half of row 1's
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[TW - 1]), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    float scale = a.sm_scale;
    if constexpr (T::ROWSCALE) scale = a.sm_scale * kscl;
    const float v = tot * scale;
    const int j = jbase + c;
    if (my_valid && j < c1) {
      const bool inwin = j >= my_s && j < my_e;
      if constexpr (CLEAN) {
        store_out<OBF>(a.out, obase + j, inwin ? v : -__builtin_inff());
      } else {
        if (inwin) store_out<OBF>(a.out, obase + j, v);
      }
    }
  };

  // ---- main loop: stage s holds columns [c0 + 64 s, c0 + 64 s + 64) --------
  f32x16 acc0[TW][2], acc1[TW][2];
  gload(0);
  swrite(0);
  __syncthreads();
  float kprev = 1.f;
  for (int s = 0; s < n_stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < n_stages) gload(s + 1);
    uint32_t bf[QD];
    uint32_t sb = 0;
    float k0 = 1.f, k1 = 1.f;
    bread(buf, 0, bf, sb, k0);
    mma(acc0, bf, sb);
    if (s > 0) epi(acc1, c0 + kStageCols * (s - 1) + 32, kprev);
    bread(buf, 1, bf, sb, k1);
    mma(acc1, bf, sb);
    epi(acc0, c0 + kStageCols * s, k0);
    kprev = k1;
    if (s + 1 < n_stages) swrite(buf ^ 1);
    __syncthreads();
  }
  epi(acc1, c0 + kStageCols * (n_stages - 1) + 32, kprev);
}

template <int F, bool WBF, bool OBF, bool CLEAN>
hipError_t launch_score_t(const ScoreArgs& a, hipStream_t stream) {
  const int64_t grid = int64_t(a.n_compute) + a.n_tiles;
  hipLaunchKernelGGL((score_kernel<F, WBF, OBF, CLEAN, 2>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace idx
