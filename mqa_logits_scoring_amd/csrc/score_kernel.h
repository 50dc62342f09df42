// Scoring kernel template for gfx950 (CDNA4).
//
// Computes, for the rows of one tile and one chunk of key columns,
//   out[i, j] = sm_scale * sum_h w[i,h] * max(0, q[i,h,:] . k[j,:])
// (the lightning-indexer score; include/idx_logits.h says where the pages
// define it) and writes -inf to the tile's in-coverage cells outside a row's
// window when cleaning.  Cells outside the tile's coverage are written, in
// this kernel, by cleanup units that run after the compute units in the same
// grid, so cleanup never competes with the matrix work of a compute unit (the
// placement lesson of DeepGEMM pull request 435, Investigation notes).  The
// FP8-family kernel and the one-row BF16 kernel below, and the 8-32-head
// kernel (score_kernel_gh.h), instead clean each row in the compute unit that
// scores it, after its last score store: with two workgroups per CU the
// other's MFMAs cover those stores, and the launch has no tail of cleanup
// units.
//
// Work decomposition
//   workgroup = 4 waves = one tile of kTileRows query rows x one key chunk
//   wave      = 2 query rows; each row's Q (64 heads x 128 d) sits in
//               registers for the whole chunk as A operands of 32x32 MFMAs
//               (heads on the M dimension)
//   32-column block u of the chunk = the B operand (key columns on N).  Every
//               wave loads its own B fragments straight from global memory
//               one block ahead; the four waves of a workgroup walk the same
//               columns, so the key rows come from L1/L2 and no LDS staging,
//               barrier or bank traffic sits on the critical path.
//   epilogue  = in registers: lane l of the 32x32 accumulator holds column
//               l%32 and 16 heads per M block; weight and sum its heads, then
//               one permlane32 swap joins the two lane halves (heads differ
//               between halves, the column does not) and leaves one row's 32
//               consecutive columns per half-wave, stored coalesced.  The
//               epilogue of one MFMA block is issued between the MFMAs of the
//               next, so the vector ALU and matrix pipes overlap (cudnn-frontend
//               pull request 416 keeps its head-sum register-resident for the
//               same reason, Why section).
//
// FP8, MXFP8 and MXFP4 inputs use ReLU(x) = (x + |x|) / 2: the epilogue is one
// FMA per head with |.| as a free source modifier, and the linear half
// qt . k (qt = sum_h w_h q_h) comes from one more MFMA block fed by the
// weighted-query pieces (internal.h).  On gfx950 two waves per SIMD can hide
// about 12 vector instructions under each 64-cycle e4m3 MFMA; the plain
// max + FMA epilogue needs about 19, the split form about 8.  BF16 inputs are
// MFMA-bound with either form and keep max + FMA.
//
// FP8 and MXFP8 keys at 64 heads go to score_kernel_x16 below instead: the
// same units and epilogue on 16x16x128 MFMAs, which make the linear term half
// as expensive.  score_kernel serves BF16 and MXFP4.
//
// Operand layout inside a lane: any permutation of d applied alike to Q and K
// leaves every dot product unchanged, so each format places d where loads are
// wide and where the MFMA's block scales line up with the E8M0 bytes.  Lane
// (c = l%32, g = l/32) holds LB bytes of its Q row (head c) and K row (column
// c) as 16-byte chunks; Fmt<> gives their offsets, the k-steps that use them,
// and how the scale word is shifted per lane half so that op_sel picks the
// right E8M0 byte (the scaled f8f6f4 MFMA places e4m3 and e2m1 operands
// differently, see Fmt<>).
#pragma once

#include <type_traits>

#include "internal.h"

namespace idx {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle): offsets past num_records read zero and drop writes.
constexpr int kBufWord3 = 0x00020000;
// cache policy of the output stores: non-temporal
constexpr int kNonTemporal = 2;
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt not waited for (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0x0F70;

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
// FP8 inputs converted exactly to bf16 (exact accumulation): the BF16 kernel,
// with the per-row K scale multiplying after the head-sum as for FP8
template <>
struct Fmt<kInBF16RowScale> {
  static constexpr int ROWB = 256, LB = 128, KSTEPS = 8, KB = 16, CBASE = 128, CSTRIDE = 16;
  static constexpr bool MX = false, ROWSCALE = true;
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

template <int F>
constexpr bool placement_matches() {
  return Fmt<F>::ROWB == KLayout<F>::ROWB && Fmt<F>::CBASE == KLayout<F>::CBASE &&
         Fmt<F>::CSTRIDE == KLayout<F>::CSTRIDE;
}
static_assert(placement_matches<IDX_IN_BF16>() && placement_matches<IDX_IN_FP8_E4M3>() &&
                  placement_matches<IDX_IN_MXFP8_E4M3>() && placement_matches<IDX_IN_MXFP4_E2M1>() &&
                  placement_matches<kInBF16RowScale>(),
              "K is reordered in the placement the MFMA operands use");
static_assert(Fmt<IDX_IN_MXFP8_E4M3>::SCALE_SHIFT == KLayout<IDX_IN_MXFP8_E4M3>::SHIFT &&
                  Fmt<IDX_IN_MXFP4_E2M1>::SCALE_SHIFT == KLayout<IDX_IN_MXFP4_E2M1>::SHIFT,
              "K scales are pre-shifted as the MFMA scale operands use them");

constexpr int kThreads = 256;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Select mode (fused top-k, ScoreArgs::cand): a lane keeps its cell as a
// candidate instead of storing it.
//
// Thresholds of a row pair, as the select-mode epilogue uses them (the same
// in every lane, so they stay in scalar registers).
struct SelTau {
  float v0, v1;
  bool all0, all1;
};
__device__ __forceinline__ SelTau sel_tau(uint32_t tau0, uint32_t tau1) {
  return SelTau{tau_value(tau0), tau_value(tau1), tau0 == 0u, tau1 == 0u};
}

// One 32-column block u of a row pair: lane half g holds row g's cell at
// column c0 + 32u + c.  A cell is kept when its column lies in [lo, lo + len)
// past c0 (its row's window cut to the unit's columns) and its score, as the
// call would store it (bf16 rounded to nearest even with OBF), reaches its
// row's threshold.  Row g's kept cells go, in column order, to slots cnt_g,
// cnt_g + 1, ... of its candidate area (rs0 / rs1, based at column c0); the
// other half's lanes and the lanes not kept write at an offset with the top
// bit set, which the buffer drops.  Counts, like thresholds, are the same in
// every lane.
template <bool OBF>
__device__ __forceinline__ void sel_emit(float v, int u, int c, int g, uint32_t c0, uint32_t lo, uint32_t len,
                                         const SelTau& tau, uint32_t& cnt0, uint32_t& cnt1,
                                         __amdgpu_buffer_rsrc_t rs0, __amdgpu_buffer_rsrc_t rs1) {
  constexpr uint32_t kDrop = 0x80000000u;
  const uint32_t col = uint32_t(32 * u + c);  // u = -1 wraps far past every window
  uint32_t bits = __float_as_uint(v);
  if constexpr (OBF) bits = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v))) << 16;
  const bool reach = __uint_as_float(bits) >= (g ? tau.v1 : tau.v0) || (g ? tau.all1 : tau.all0);
  const bool keep = col - lo < len && reach;
  const uint64_t m = __ballot(keep);
  const uint32_t n0 = uint32_t(__builtin_popcount(uint32_t(m))), n1 = uint32_t(__builtin_popcount(uint32_t(m >> 32)));
  const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
  const uint32_t off = keep ? ((g ? cnt1 - n0 : cnt0) + below) * 8u : kDrop;
  const u32x2 pair = {bits, c0 + col};
  __builtin_amdgcn_raw_buffer_store_b64(pair, rs0, int(off | (g ? kDrop : 0u)), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b64(pair, rs1, int(off | (g ? 0u : kDrop)), 0, 0);
  cnt0 += n0;
  cnt1 += n1;
}

// A row's window cut to the unit's columns [c0, c1), relative to c0: start
// and width (0 when they do not meet).
__device__ __forceinline__ void sel_window(int s, int e, int c0, int c1, uint32_t& lo, uint32_t& len) {
  const int a = max(s, c0), b = min(e, c1);
  lo = uint32_t(a - c0);
  len = uint32_t(max(b - a, 0));
}

// A row's candidate area from column c0 on, ncols pairs (none for a padding row).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sel_rsrc(const ScoreArgs& a, int row, bool valid, int c0,
                                                          int ncols) {
  return __builtin_amdgcn_make_buffer_rsrc(a.cand + (int64_t(row) * a.S_k + c0) * 8, 0, valid ? ncols * 8 : 0,
                                           0x00020000);
}

// The unit's entry of a row: (first column, candidates kept).
__device__ __forceinline__ void sel_finish(const ScoreArgs& a, int row, int chunk, int c0, uint32_t cnt) {
  int32_t* e = a.meta + 2 * (int64_t(row) * a.n_chunk + chunk);
  e[0] = c0;
  e[1] = int32_t(cnt);
}

template <bool OBF>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OBF) {
    // round to nearest even, NaN kept quiet
    uint32_t u = __float_as_uint(v);
    uint32_t r = ((u >> 16) & 1u) + 0x7FFFu;
    uint16_t h = (u & 0x7FFFFFFFu) > 0x7F800000u ? uint16_t((u >> 16) | 0x40u) : uint16_t((u + r) >> 16);
    __builtin_nontemporal_store(h, static_cast<uint16_t*>(out) + idx);
  } else {
    __builtin_nontemporal_store(v, static_cast<float*>(out) + idx);
  }
}

// Cells of a tile's TR rows outside its computed coverage: -inf when cleaning.
// With a plan that does not match the call, every row of the tile is filled
// with quiet NaN instead, so the mismatch cannot pass unnoticed.
template <bool OBF, bool CLEAN, int TR>
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
  for (int r = 0; r < TR; ++r) {
    int64_t row;
    if (plan_ok) {
      row = slot_row[int64_t(tile) * TR + r];
      if (row < 0) continue;
    } else {
      const int64_t i = int64_t(tile % tpb) * TR + r;
      if (i >= a.S_q) continue;
      row = int64_t(tile / tpb) * a.S_q + i;
    }
    const int64_t base = row * a.ld;
    for (int j = threadIdx.x; j < lo; j += kThreads) store_out<OBF>(a.out, base + j, fill);
    for (int j = hi + threadIdx.x; j < a.S_k; j += kThreads) store_out<OBF>(a.out, base + j, fill);
  }
}

// -inf over [0, lo) and [hi, S_k) of one output row, by one wave (lane =
// its lane): wave-uniform loops whose buffer ranges drop what lies past each
// part, so no lane branches.  Compute units that clean their own rows call
// it after their last store; nothing waits on these stores.
template <bool OBF>
__device__ __forceinline__ void clean_row_outside(const ScoreArgs& a, int row, int lo, int hi, int lane) {
  constexpr int ES = OBF ? 2 : 4;
  unsigned char* base = static_cast<unsigned char*>(a.out) + int64_t(row) * a.ld * ES;
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc(base, 0, lo * ES, kBufWord3);
  const __amdgpu_buffer_rsrc_t r1 =
      __builtin_amdgcn_make_buffer_rsrc(base + int64_t(hi) * ES, 0, (a.S_k - hi) * ES, kBufWord3);
  for (int j = 0; j < lo; j += 64) {
    if constexpr (OBF) __builtin_amdgcn_raw_buffer_store_b16(uint16_t(0xFF80u), r0, (j + lane) * ES, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(0xFF800000u, r0, (j + lane) * ES, 0, kNonTemporal);
  }
  for (int j = 0; j < a.S_k - hi; j += 64) {
    if constexpr (OBF) __builtin_amdgcn_raw_buffer_store_b16(uint16_t(0xFF80u), r1, (j + lane) * ES, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(0xFF800000u, r1, (j + lane) * ES, 0, kNonTemporal);
  }
}

// Compute units clean their own rows when the launch has no cleanup units
// (the launchers drop them for the plain, non-paged, non-decode FP8-family,
// one-row BF16 and 8-32-head kernels when cleaning).
__device__ __forceinline__ bool units_clean_own_rows(const ScoreArgs& a) {
  return a.n_positions == a.n_pos_compute && !a.wave_split && !a.dyn_units;
}

// A unit of work: compute (a tile's columns [c0, c1)), cleanup (a tile's
// cells outside its coverage) or nothing (a missing tile of a partial
// segment, or a chunk past the tile's coverage).  [0, cl0) and [cl1, S_k) are
// the cells outside the coverage that the unit cleans when compute units
// clean their own rows: the first chunk takes the cells left of the
// coverage, the last the cells right of it; chunk 0 of a tile whose rows all
// see nothing (kind none, tile >= 0) takes whole rows.
enum { kUnitNone = 0, kUnitCompute = 1, kUnitCleanup = 2 };
struct Unit {
  int kind, tile, c0, c1, chunk, cl0, cl1;
};

// dyn_units: compute position p -> unit.  Every wave reads every tile's
// coverage (tiles are batches here), sums the widths, takes a chunk width w
// that keeps the chunks (ceil(width / w) per tile) within the positions,
// and finds the tile whose chunks hold position p by a scan over the tiles
// in order.  All 64 lanes take part.
__device__ __forceinline__ Unit decode_dyn_unit(const ScoreArgs& a, int p) {
  const int lane = int(threadIdx.x & 63);
  const int32_t* lo = reinterpret_cast<const int32_t*>(a.plan + a.off_lo);
  const int32_t* hi = reinterpret_cast<const int32_t*>(a.plan + a.off_hi);
  constexpr int K = kDynUnitTiles / 64;
  int tlo[K], span[K];
  uint32_t tot = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int t = lane + 64 * k, tc = min(t, a.n_tiles - 1);  // loads in bounds, issued together
    const int l = lo[tc], h = hi[tc];
    tlo[k] = l;
    span[k] = t < a.n_tiles ? max(h - l, 0) : 0;
    tot += uint32_t(span[k]);
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) tot += uint32_t(__shfl_xor(int(tot), d, 64));
  // the same in every lane: read as such, so that what follows stays scalar
  tot = __builtin_amdgcn_readfirstlane(tot);
  // a width that surely fits (each tile rounds up by less than one chunk),
  // or, when it also fits, the narrower one that counts half a chunk per tile
  auto width_for = [&](uint32_t room) {
    return max(a.min_chunk, int((((tot + room - 1) / room) + 63u) & ~63u));
  };
  const int w_sure = width_for(uint32_t(a.n_pos_compute - a.n_tiles));
  const int w_try = width_for(uint32_t(a.n_pos_compute - (a.n_tiles + 1) / 2));
  uint32_t need = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) need += uint32_t((span[k] + w_try - 1) / w_try);
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) need += uint32_t(__shfl_xor(int(need), d, 64));
  need = __builtin_amdgcn_readfirstlane(need);
  const int w = need <= uint32_t(a.n_pos_compute) ? w_try : w_sure;
  // no branch on the result (the kernels' MFMAs must not sit under a saved
  // exec mask): every step runs, the hit is kept by selects
  uint32_t carry = 0;
  int tile = -1, c0 = 0, c1 = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const uint32_t cnt = uint32_t((span[k] + w - 1) / w);
    uint32_t incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = uint32_t(__shfl_up(int(incl), d, 64));
      incl += lane >= d ? y : 0u;
    }
    const uint32_t first = carry + incl - cnt;
    const uint64_t here = __ballot(cnt != 0 && first <= uint32_t(p) && uint32_t(p) < first + cnt);
    const int src = here != 0 ? __builtin_ctzll(here) : 0;
    const int lo_s = __builtin_amdgcn_readlane(tlo[k], src);
    const int end_s = __builtin_amdgcn_readlane(tlo[k] + span[k], src);
    const int first_s = __builtin_amdgcn_readlane(int(first), src);
    const int a0 = lo_s + (p - first_s) * w;
    tile = here != 0 ? src + 64 * k : tile;
    c0 = here != 0 ? a0 : c0;
    c1 = here != 0 ? min(a0 + w, end_s) : c1;
    carry += uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
  }
  return Unit{tile >= 0 ? int(kUnitCompute) : int(kUnitNone), max(tile, 0), c0, c1, 0, 0, a.S_k};
}

// Work position p (ScoreArgs) -> unit.
__device__ __forceinline__ Unit decode_unit(const ScoreArgs& a, int p) {
  if (p >= a.n_pos_compute) return Unit{kUnitCleanup, p - a.n_pos_compute, 0, 0, 0, 0, a.S_k};
  if (a.dyn_units) return decode_dyn_unit(a, p);
  const int slot = p / a.n_chunk, chunk = p - slot * a.n_chunk;
  // slot -> (batch, segment, rank): batches and segments from the last
  const int tpb = a.tiles_per_batch, spb = a.seg_per_batch, tps = a.tiles_per_seg, last = a.last_seg_tiles;
  const int j = slot / tpb, r = slot - j * tpb;
  const int b = a.B - 1 - j;
  int seg, rank;
  if (r < last) {
    seg = spb - 1;
    rank = r;
  } else {
    const int r2 = r - last;
    seg = spb - 2 - r2 / tps;
    rank = r2 - (r2 / tps) * tps;
  }
  const int tile =
      reinterpret_cast<const int32_t*>(a.plan + a.off_order)[(int64_t(b) * spb + seg) * tps + rank];
  if (tile < 0) return Unit{kUnitNone, -1, 0, 0, 0, 0, a.S_k};
  const int lo = reinterpret_cast<const int32_t*>(a.plan + a.off_lo)[tile];
  const int hi = reinterpret_cast<const int32_t*>(a.plan + a.off_hi)[tile];
  const int w = max(a.min_chunk, ((hi - lo + a.n_chunk - 1) / a.n_chunk + 63) & ~63);
  const int c0 = lo + chunk * w, c1 = min(hi, c0 + w);
  if (c0 >= c1) return Unit{kUnitNone, tile, c0, c0, chunk, 0, chunk == 0 ? 0 : a.S_k};
  return Unit{kUnitCompute, tile, c0, c1, chunk, chunk == 0 ? c0 : 0, c1 == hi ? c1 : a.S_k};
}

// Waves per SIMD the kernel is built for: the FP8-family and FP4 kernels fit in
// 256 registers and run two workgroups per CU so one wave's epilogue overlaps
// the other's MFMAs; the BF16 kernel holds twice the Q bytes and runs one.
template <int F>
constexpr int waves_per_eu() {
  return bf16_operands(F) ? 1 : 2;
}

// K fragment buffers per wave (even): the load of a block is issued
// kfrag_ring - 1 blocks before its MFMAs.  One block ahead covers the L2
// latency; deeper rings only cost registers (measured, all formats).
template <int F>
constexpr int kfrag_ring() {
  return 2;
}

// PD: keys straight from a paged cache (ScoreArgs::kcache) instead of the
// fragment-order copy.  SEL: select mode (ScoreArgs::cand).
template <int F, bool WBF, bool OBF, bool CLEAN, bool PD = false, bool SEL = false>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(waves_per_eu<F>(), waves_per_eu<F>()))) score_kernel(const ScoreArgs a) {
  static_assert(!SEL || (!CLEAN && !PD), "select mode stores no scores and reads contiguous keys");
  if constexpr (SEL) {
    if (a.gate != nullptr && *a.gate == 0) return;  // a second pass with no row to redo
  }
  using T = Fmt<F>;
  constexpr int TW = 2;  // query rows per wave
  static_assert(4 * TW == kTileRows, "four waves cover one tile");
  constexpr bool HAS_KS = T::MX || T::ROWSCALE;
  constexpr int QD = T::LB / 4;  // dwords per lane per row
  constexpr int KD = T::KB / 4;  // dwords per lane per k-step

  const int tid = threadIdx.x;
  // the wave index is wave-uniform; saying so lets everything derived from it
  // (rows, their windows, the output resources) live in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5, c = lane & 31;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == a.B && hdr->S_q == a.S_q && hdr->S_k == a.S_k &&
                       hdr->H == 64 && hdr->D == 128 && hdr->tile_rows == kTileRows && hdr->n_tiles == a.n_tiles;
  // one work position per workgroup, dealt in order by the hardware
  const int pos = int(blockIdx.x);
  if (pos >= a.n_pos_compute) {
    cleanup_unit<OBF, CLEAN, kTileRows>(a, pos - a.n_pos_compute, plan_ok);
    return;
  }
  if (!plan_ok) return;
  const Unit u = decode_unit(a, pos);
  if (u.kind != kUnitCompute) return;
  const int tile = u.tile;
  int c0 = u.c0, c1 = u.c1;  // columns [c0, c1) of the tile are this unit's
  // the wave whose tile slots hold this wave's rows: its own, or with
  // decode-sized tiles (wave_split: at most two rows per batch) slots 0 and 1
  // for every wave, each wave taking a quarter of the unit's columns
  int slot_wave = wave;
  if (!SEL && a.wave_split) {
    const int per = (((c1 - c0 + 63) / 64) + 3) / 4;  // 64-column pairs per wave
    const int w0 = c0 + 64 * per * wave;
    c1 = min(c1, w0 + 64 * per);
    c0 = w0;
    if (c0 >= c1) return;
    slot_wave = 0;
  }
  const int n_pairs = (c1 - c0 + 63) / 64;  // pairs of 32-column blocks
  const int b = tile / a.tiles_per_batch;

  // ---- the wave's query rows ----------------------------------------------
  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
  const int32_t first_row = slot_row[int64_t(tile) * kTileRows];
  int rows[TW];
  bool rvalid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int r = slot_row[int64_t(tile) * kTileRows + slot_wave * TW + t];
    rvalid[t] = r >= 0;
    rows[t] = r >= 0 ? r : first_row;
  }
  // a wave with padding rows only (short tiles, e.g. two-token decode) has
  // nothing to store in this unit
  if (!rvalid[0] && !rvalid[1]) return;
  // select mode: the rows' thresholds; a wave whose rows keep nothing is done
  uint32_t tau_r[TW] = {kTauNone, kTauNone};
  if constexpr (SEL) {
#pragma unroll
    for (int t = 0; t < TW; ++t) tau_r[t] = rvalid[t] ? a.tau[rows[t]] : kTauNone;
    if (tau_r[0] == kTauNone && tau_r[1] == kTauNone) return;
  }

  // Q fragments of head 32*mb + c for both rows, and their MX scale words
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

  // half-wave g stores row g of the wave: its window relative to c0
  const int my_row = g ? rows[1] : rows[0];
  const int my_s = reinterpret_cast<const int32_t*>(a.plan + a.off_start)[my_row];
  const int my_e = reinterpret_cast<const int32_t*>(a.plan + a.off_end)[my_row];

  // K in fragment order and its scales in block order (internal.h), read with
  // buffer loads: the block offset is wave-uniform (SGPR), the lane offset a
  // constant and the chunk offset an immediate, so no vector instruction
  // computes an address.  Block kb0 + u holds columns c0 + 32u..; blocks past
  // the end of K are clamped to the last one: always in bounds, and the
  // columns they feed are never stored.
  const int nblk = (a.S_k + 31) >> 5;
  const int kb0 = c0 >> 5;  // c0 is a multiple of 32
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(a.kfrag) + int64_t(b) * nblk * (32 * T::ROWB), 0, nblk * (32 * T::ROWB), kBufWord3);
  const __amdgpu_buffer_rsrc_t srs =
      HAS_KS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.kscale) + int64_t(b) * nblk * 64, 0,
                                                 nblk * 256, kBufWord3)
             : krs;
  // From a paged cache the block's 32 keys are 32 consecutive rows of one
  // page: lane (c, g) reads row c at its chunk offsets, the page's first row
  // of the block is the scalar offset (block table entry clamped into the
  // cache, as the gather clamps it), and MX scale words are shifted here.
  const __amdgpu_buffer_rsrc_t pkrs =
      PD ? __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(a.kcache), 0,
                                             int(uint32_t(a.num_pages) * uint32_t(a.page_size) * T::ROWB), kBufWord3)
         : krs;
  const __amdgpu_buffer_rsrc_t psrs =
      PD && HAS_KS ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.kscache), 0,
                                                       int(uint32_t(a.num_pages) * uint32_t(a.page_size) * 4u),
                                                       kBufWord3)
                   : srs;
  const int32_t* btrow = PD ? a.btable + int64_t(b) * a.max_pages : nullptr;
  // paged: blocks are loaded in order, and the page of the next one is read
  // from the block table one load ahead, off the path of the key loads
  int pg_next = 0;
  if constexpr (PD) pg_next = __builtin_amdgcn_readfirstlane(btrow[uint32_t(min(kb0, nblk - 1)) >> a.bpp_shift]);
  auto kload = [&](int u, uint32_t (&bf)[QD], uint32_t& kword) {
    const int blk = min(kb0 + u, nblk - 1);
    if constexpr (PD) {
      const uint32_t rem = uint32_t(blk) & ((1u << a.bpp_shift) - 1u);
      int pg = pg_next;
      pg_next = __builtin_amdgcn_readfirstlane(btrow[uint32_t(min(blk + 1, nblk - 1)) >> a.bpp_shift]);
      pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      const uint32_t row0 = uint32_t(pg) * uint32_t(a.page_size) + rem * 32u;
#pragma unroll
      for (int v = 0; v < QD / 4; ++v) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(pkrs, c * T::ROWB + g * T::CBASE + v * T::CSTRIDE,
                                                              int(row0 * T::ROWB), 0);
        bf[4 * v + 0] = x[0];
        bf[4 * v + 1] = x[1];
        bf[4 * v + 2] = x[2];
        bf[4 * v + 3] = x[3];
      }
      if constexpr (HAS_KS) {
        kword = __builtin_amdgcn_raw_buffer_load_b32(psrs, c * 4, int(row0 * 4u), 0);
        if constexpr (T::MX) kword = g ? kword >> T::SCALE_SHIFT : kword;
      }
    } else {
#pragma unroll
      for (int v = 0; v < QD / 4; ++v) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(krs, lane * 16 + v * 1024, blk * (32 * T::ROWB), 0);
        bf[4 * v + 0] = x[0];
        bf[4 * v + 1] = x[1];
        bf[4 * v + 2] = x[2];
        bf[4 * v + 3] = x[3];
      }
      if constexpr (HAS_KS) kword = __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, blk * 256, 0);
    }
  };
  // MX: the lane half's E8M0 bytes of the column's scale word (stored shifted)
  auto kscale_mx = [&](uint32_t kword) { return kword; };

  // all k-steps of one 32x32 block: acc = Q(row t, heads 32*mb..) x K(32 columns)^T
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

  // Stores go through one buffer resource per row of the wave, based at the
  // unit's first column and num_records = the unit's width (0 for a padding
  // row): the hardware drops every write at an offset past it, so columns
  // past the unit, the lanes of the other half-wave (offset with the top bit
  // set) and, when not cleaning, out-of-window cells need no branch and no
  // address arithmetic beyond one running offset.  No branch means nothing
  // can be sunk into one.
  // The -inf of a cleaned cell is picked byte-wise by v_perm_b32 rather than
  // by a select: a select on a divergent condition may be turned into a
  // branch with the value's computation (MFMA blocks included) sunk into it,
  // and a matrix instruction under a partial exec mask still writes every
  // lane of its result, clobbering what the masked-off lanes held.
  constexpr int ES = OBF ? 2 : 4;
  constexpr uint32_t kDrop = 0x80000000u;
  __amdgpu_buffer_rsrc_t ors[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t)
    ors[t] = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char*>(a.out) + (int64_t(rows[t]) * a.ld + c0) * ES, 0, rvalid[t] ? (c1 - c0) * ES : 0,
        kBufWord3);
  const uint32_t half0 = g ? kDrop : 0u, half1 = g ? 0u : kDrop;
  const uint32_t s_rel = uint32_t(my_s - c0) * ES;                       // window start, bytes past c0
  const uint32_t w_len = uint32_t(max(my_e - my_s, 0)) * ES;             // window width in bytes
  // select mode: the rows' candidate areas, the lane's row's threshold and count
  __amdgpu_buffer_rsrc_t crs[TW];
  if constexpr (SEL) {
#pragma unroll
    for (int t = 0; t < TW; ++t) crs[t] = sel_rsrc(a, rows[t], rvalid[t], c0, c1 - c0);
  }
  uint32_t sel_cnt[TW] = {0u, 0u};
  const SelTau stau = sel_tau(tau_r[0], tau_r[1]);
  uint32_t sel_lo = 0, sel_len = 0;
  if constexpr (SEL) sel_window(my_s, my_e, c0, c1, sel_lo, sel_len);
  auto store = [&](float v, int u) {
    if constexpr (SEL) {
      sel_emit<OBF>(v, u, c, g, uint32_t(c0), sel_lo, sel_len, stau, sel_cnt[0], sel_cnt[1], crs[0], crs[1]);
      return;
    }
    const uint32_t off = uint32_t(32 * u + c) * ES;  // u = -1 wraps to a huge offset: dropped
    const bool inwin = off - s_rel < w_len;
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
      // bf16: a half-wave covers half of a 128-byte line and the next block
      // the other half, so these stores stay in L2 to meet there (non-temporal
      // ones left as two half-line writes)
      __builtin_amdgcn_raw_buffer_store_b16(h, ors[0], int(o0), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(h, ors[1], int(o1), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors[0], int(o0), 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors[1], int(o1), 0, kNonTemporal);
    }
  };

  // One pipeline stage: MFMA, 8 VALU, MFMA, 8 VALU, then a full scheduling
  // barrier so the next stage's instructions stay after this one's.
  auto interleave_stage = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Work is pipelined over 32x32 MFMA blocks: the MFMAs of one block run
  // while the epilogue of the previous block executes, with two accumulators
  // alternating; the fragments of later 32-column blocks are loaded while the
  // current one is computed.
  f32x16 accA = {}, accB = {};
  float p0 = 0.f, p1 = 0.f;

  if constexpr (!bf16_operands(F)) {
    // MXFP4 (FP8 and MXFP8 run score_kernel_x16).  Blocks per 32-column
    // block u: L (linear term of both rows from the weighted-query pieces),
    // then (row 0 | row 1) x (heads 0-31 | 32-63).  The pieces are e2m1 rows
    // packed like Q, so L is an ordinary fp4 block with the pieces as A rows:
    // piece p of row t on A row (p % 4) + 4t + 8 (p / 4), which the 32x32
    // output puts in lane half t, registers 0-7.  After the head-sum swap,
    // lane half t holds row t's columns, so the linear term adds in place.
    static_assert(F == IDX_IN_MXFP4_E2M1, "the FP8 formats use score_kernel_x16");
    using PF = PieceFmt<F>;
    uint32_t lf[QD];
    uint32_t sl;
    {
      const int tt = (c >> 2) & 1, pc = (c & 3) + 4 * (c >> 3);
      const bool has = c < 16 && pc < PF::N;
      const unsigned char* src = a.pieces + int64_t(rows[tt]) * kPieceRowBytes + (has ? pc : 0) * PF::BYTES;
#pragma unroll
      for (int v = 0; v < QD / 4; ++v) {
        const uint4 x = has ? *reinterpret_cast<const uint4*>(src + g * T::CBASE + v * T::CSTRIDE)
                            : make_uint4(0, 0, 0, 0);
        lf[4 * v + 0] = x.x;
        lf[4 * v + 1] = x.y;
        lf[4 * v + 2] = x.z;
        lf[4 * v + 3] = x.w;
      }
      const uint32_t word = has ? a.pscales[int64_t(rows[tt]) * kPieceSlots + pc] : 0x7F7F7F7Fu;
      sl = g ? (word >> T::SCALE_SHIFT) : word;  // as for MXFP4 Q
    }
    const float half_scale = 0.5f * a.sm_scale;

    auto mfma_lin = [&](f32x16& acc, const uint32_t (&bf)[QD], uint32_t sb) { mfma_block(acc, lf, sl, bf, sb); };
    auto epi_lin = [&](const f32x16& acc) {
      float v = acc[0];
#pragma unroll
      for (int r = 1; r < PF::N; ++r) v += acc[r];
      return v;
    };
    // weight and sum |S| of the lane's 16 heads of one block (fixed order)
    auto epi_abs = [&](const f32x16& acc, const float (&w)[16], float p) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p = __builtin_fmaf(w[r], __builtin_fabsf(acc[r]), p);
      return p;
    };
    auto combine_abs = [&](float q0, float q1, float lin) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(q0), __float_as_uint(q1), false, false);
      const float tot = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) + lin;
      return tot * half_scale;
    };

    float linv = 0.f;
    // X receives this block's first and last MFMA blocks; Y the other ones.
    // Each stage issues one MFMA block and the epilogue of the previous one;
    // the scheduling barriers keep that order and interleave each stage as
    // MFMA, 8 VALU, MFMA, 8 VALU so the vector work runs under the matrix
    // work.
    auto block_abs = [&](const uint32_t (&bf)[QD], uint32_t kword, int u, f32x16& X, f32x16& Y) {
      const uint32_t sb = kscale_mx(kword);
      mfma_lin(X, bf, sb);                        // L of u                       ||
      p1 = epi_abs(Y, wv[1][1], p1);              //   (row 1, heads 32-63) of u-1, completing u-1
      const float v = combine_abs(p0, p1, linv);
      interleave_stage();
      mfma_block(Y, qf[0][0], sa[0][0], bf, sb);  // (row 0, heads 0-31) of u    ||
      linv = epi_lin(X);                          //   L of u
      interleave_stage();
      mfma_block(X, qf[0][1], sa[0][1], bf, sb);  // (row 0, heads 32-63)        ||
      p0 = epi_abs(Y, wv[0][0], 0.f);             //   (row 0, heads 0-31)
      interleave_stage();
      mfma_block(Y, qf[1][0], sa[1][0], bf, sb);  // (row 1, heads 0-31)         ||
      p0 = epi_abs(X, wv[0][1], p0);              //   (row 0, heads 32-63)
      interleave_stage();
      mfma_block(X, qf[1][1], sa[1][1], bf, sb);  // (row 1, heads 32-63)        ||
      p1 = epi_abs(Y, wv[1][0], 0.f);             //   (row 1, heads 0-31)
      interleave_stage();
      store(v, u - 1);
    };

    // A ring of NB fragment buffers: block u reads buffer u % NB, and the
    // load of block u + NB - 1 goes into the buffer block u - 1 used, right
    // after that block's MFMAs were issued.  The scheduling barriers keep
    // each load there: hoisting it would force a register copy (and a wait
    // for the load) inside the loop.
    constexpr int NB = kfrag_ring<F>();
    uint32_t bfs[NB][QD];
    uint32_t kws[NB];
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) kload(i, bfs[i], kws[i]);
    // Everything loaded so far is needed before the first block anyway;
    // waiting for it here leaves only the loop's own loads pending at the
    // loop head, so the waits inside the loop need not cover the prologue.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const int n_iter = (2 * n_pairs + NB - 1) / NB;
    for (int s = 0; s < n_iter; ++s) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int u = NB * s + i;
        kload(u + NB - 1, bfs[(i + NB - 1) % NB], kws[(i + NB - 1) % NB]);
        if (i % 2 == 0)
          block_abs(bfs[i], kws[i], u, accA, accB);
        else
          block_abs(bfs[i], kws[i], u, accB, accA);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    p1 = epi_abs(accB, wv[1][1], p1);
    store(combine_abs(p0, p1, linv), NB * n_iter - 1);
  } else {
    // ReLU as a signed-integer max of the float's bits: for every non-NaN x,
    // x > 0 exactly when its bits are a positive int32, so max(bits, 0) is
    // max(x, 0) (with -0 giving +0) in one instruction and without the NaN
    // quieting a float max needs.  Weighted and summed over the lane's 16
    // heads of one block in a fixed order.
    auto epi_relu = [&](const f32x16& acc, const float (&w)[16], float p) {
#pragma unroll
      for (int r = 0; r < 16; ++r) p = __builtin_fmaf(w[r], __int_as_float(max(__float_as_int(acc[r]), 0)), p);
      return p;
    };
    // ks: the FP8 row scale of the lane's column (converted FP8 inputs)
    auto combine = [&](float q0, float q1, float ks) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(q0), __float_as_uint(q1), false, false);
      const float v = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * a.sm_scale;
      return T::ROWSCALE ? v * ks : v;
    };
    // (row, heads) blocks (0,0) (0,1) (1,0) (1,1), alternating accA / accB;
    // kprev: the row scale word of block u-1, kept past its ring buffer's
    // reuse
    float kprev = 1.f;
    auto block_relu = [&](const uint32_t (&bf)[QD], uint32_t kword, int u) {
      mfma_block(accA, qf[0][0], 0, bf, 0);  // (row 0, heads 0-31) of u  ||
      p1 = epi_relu(accB, wv[1][1], p1);     //   (row 1, heads 32-63) of u-1, completing u-1
      const float v = combine(p0, p1, kprev);
      kprev = __uint_as_float(kword);
      __builtin_amdgcn_sched_barrier(0);
      mfma_block(accB, qf[0][1], 0, bf, 0);  // (row 0, heads 32-63)      ||
      p0 = epi_relu(accA, wv[0][0], 0.f);    //   (row 0, heads 0-31)
      __builtin_amdgcn_sched_barrier(0);
      mfma_block(accA, qf[1][0], 0, bf, 0);  // (row 1, heads 0-31)       ||
      p0 = epi_relu(accB, wv[0][1], p0);     //   (row 0, heads 32-63)
      __builtin_amdgcn_sched_barrier(0);
      mfma_block(accB, qf[1][1], 0, bf, 0);  // (row 1, heads 32-63)      ||
      p1 = epi_relu(accA, wv[1][0], 0.f);    //   (row 1, heads 0-31)
      __builtin_amdgcn_sched_barrier(0);
      store(v, u - 1);
    };
    constexpr int NB = kfrag_ring<F>();
    uint32_t bfs[NB][QD];
    uint32_t kws[NB];
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) kload(i, bfs[i], kws[i]);
    // Everything loaded so far is needed before the first block anyway;
    // waiting for it here leaves only the loop's own loads pending at the
    // loop head, so the waits inside the loop need not cover the prologue.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const int n_iter = (2 * n_pairs + NB - 1) / NB;
    for (int s = 0; s < n_iter; ++s) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int u = NB * s + i;
        kload(u + NB - 1, bfs[(i + NB - 1) % NB], kws[(i + NB - 1) % NB]);
        block_relu(bfs[i], kws[i], u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    p1 = epi_relu(accB, wv[1][1], p1);
    store(combine(p0, p1, kprev), NB * n_iter - 1);
  }
  if constexpr (SEL) {
    if (c == 0 && (g ? rvalid[1] : rvalid[0])) sel_finish(a, my_row, u.chunk, c0, g ? sel_cnt[1] : sel_cnt[0]);
  }
}

// ---------------------------------------------------------------------------
// BF16 operands with one query row per wave (plain calls on contiguous keys,
// tiles of more than two rows).
//
// Two rows of BF16 Q take 128 registers, so score_kernel runs one wave per
// SIMD for BF16, and nothing covers a wave's own waits (the loads of its Q,
// of its next key block).  Here a workgroup's four waves take one row each,
// half a tile: a unit is (tile, chunk, half), two work positions per unit,
// and the 64 Q registers of one row leave room for two waves per SIMD, so
// two workgroups share a CU and one's loads run under the other's MFMAs.
// Per 32-column block a wave issues the two 32x32 blocks of its row (heads
// 0-31, 32-63) over all of d, each interleaved with the epilogue of the
// previous one, in the order score_kernel uses for one row, so every score
// is bitwise the one score_kernel gives.  After the head-sum swap both lane
// halves hold the row's 32 columns; the first half stores them.  When
// cleaning, each wave then writes -inf to its row outside the tile's coverage
// (the first chunk left of it, the last chunk right of it): on short rows
// (packed variable-length rows see about 420 keys) a tail of cleanup units
// had cost a tenth of the launch.
template <int F, bool WBF, bool OBF, bool CLEAN>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
    score_kernel_bf16w(const ScoreArgs a) {
  static_assert(bf16_operands(F), "BF16 operands only");
  using T = Fmt<F>;
  constexpr bool HAS_KS = T::ROWSCALE;
  constexpr int QD = T::LB / 4;  // dwords per lane per row
  constexpr int KD = T::KB / 4;  // dwords per lane per k-step

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5, c = lane & 31;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == a.B && hdr->S_q == a.S_q && hdr->S_k == a.S_k &&
                       hdr->H == 64 && hdr->D == 128 && hdr->tile_rows == kTileRows && hdr->n_tiles == a.n_tiles;
  const int pos = int(blockIdx.x);
  if (pos >= a.n_pos_compute) {
    cleanup_unit<OBF, CLEAN, kTileRows>(a, pos - a.n_pos_compute, plan_ok);
    return;
  }
  const bool own_clean = CLEAN && units_clean_own_rows(a);
  if (!plan_ok) {
    // no cleanup units to fill the rows with NaN: the first half of each
    // tile's first chunk does it
    if (own_clean && (pos & 1) == 0 && (pos >> 1) % a.n_chunk == 0)
      cleanup_unit<OBF, CLEAN, kTileRows>(a, (pos >> 1) / a.n_chunk, false);
    return;
  }
  // positions 2j and 2j + 1: the two halves of unit j, next to each other
  const Unit u = decode_unit(a, pos >> 1);
  // a tile whose rows all see nothing runs with no key block when it cleans
  // its rows: its one store falls outside the (empty) column range
  if (u.kind != kUnitCompute && !(own_clean && u.tile >= 0 && u.cl1 < a.S_k)) return;
  const int tile = u.tile, c0 = u.c0, c1 = u.c1;
  const int n_pairs = (c1 - c0 + 63) / 64;  // pairs of 32-column blocks
  const int b = tile / a.tiles_per_batch;

  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
  const int row = __builtin_amdgcn_readfirstlane(slot_row[int64_t(tile) * kTileRows + (pos & 1) * 4 + wave]);
  if (row < 0) return;  // a padding slot: nothing to score

  // Q fragments of heads 32*mb + c, weights of the lane's 16 heads per block
  uint32_t qf[2][QD];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t qrow = int64_t(row) * 64 + 32 * mb + c;
    const unsigned char* src = static_cast<const unsigned char*>(a.q) + qrow * T::ROWB + g * T::CBASE;
#pragma unroll
    for (int v = 0; v < QD / 4; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + v * T::CSTRIDE);
      qf[mb][4 * v + 0] = x.x;
      qf[mb][4 * v + 1] = x.y;
      qf[mb][4 * v + 2] = x.z;
      qf[mb][4 * v + 3] = x.w;
    }
  }
  float wv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int64_t off = int64_t(row) * 64 + 32 * mb + 8 * q4 + 4 * g;
      if constexpr (WBF) {
        const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.w) + off);
        wv[mb][4 * q4 + 0] = __uint_as_float(x.x << 16);
        wv[mb][4 * q4 + 1] = __uint_as_float(x.x & 0xFFFF0000u);
        wv[mb][4 * q4 + 2] = __uint_as_float(x.y << 16);
        wv[mb][4 * q4 + 3] = __uint_as_float(x.y & 0xFFFF0000u);
      } else {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.w) + off);
        wv[mb][4 * q4 + 0] = x.x;
        wv[mb][4 * q4 + 1] = x.y;
        wv[mb][4 * q4 + 2] = x.z;
        wv[mb][4 * q4 + 3] = x.w;
      }
    }
  }
  const int my_s = reinterpret_cast<const int32_t*>(a.plan + a.off_start)[row];
  const int my_e = reinterpret_cast<const int32_t*>(a.plan + a.off_end)[row];

  // K in fragment order (as score_kernel reads it)
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
  auto mfma_block = [&](f32x16& acc, const uint32_t (&q)[QD], const uint32_t (&bf)[QD]) {
    f32x16 d = {};
#pragma unroll
    for (int st = 0; st < T::KSTEPS; ++st) {
      bf16x8 av, bv;
      __builtin_memcpy(&av, &q[st * KD], 16);
      __builtin_memcpy(&bv, &bf[st * KD], 16);
      d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, d, 0, 0, 0);
    }
    acc = d;
  };

  // stores: one resource for the row, based at the unit's first column; the
  // second lane half and, without cleaning, cells outside the window drop
  constexpr int ES = OBF ? 2 : 4;
  constexpr uint32_t kDrop = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<unsigned char*>(a.out) + (int64_t(row) * a.ld + c0) * ES, 0, (c1 - c0) * ES, kBufWord3);
  const uint32_t half = g ? kDrop : 0u;
  const uint32_t s_rel = uint32_t(my_s - c0) * ES;
  const uint32_t w_len = uint32_t(max(my_e - my_s, 0)) * ES;
  auto store = [&](float v, int u) {
    const uint32_t off = uint32_t(32 * u + c) * ES;  // u = -1 wraps to a huge offset: dropped
    const bool inwin = off - s_rel < w_len;
    uint32_t o = off | half;
    if constexpr (!CLEAN) o = inwin ? o : kDrop;
    float val = v;
    if constexpr (CLEAN)
      val = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(v), 0xFF800000u,
                                                  inwin ? 0x07060504u : 0x03020100u));
    if constexpr (OBF) {
      const uint16_t h = __builtin_bit_cast(uint16_t, static_cast<__bf16>(val));  // round to nearest even
      __builtin_amdgcn_raw_buffer_store_b16(h, ors, int(o), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors, int(o), 0, kNonTemporal);
    }
  };

  // ReLU as a signed-integer max of the float's bits (as in score_kernel),
  // weighted and summed over the lane's 16 heads of one block
  auto epi_relu = [&](const f32x16& acc, const float (&w)[16], float p) {
#pragma unroll
    for (int r = 0; r < 16; ++r) p = __builtin_fmaf(w[r], __int_as_float(max(__float_as_int(acc[r]), 0)), p);
    return p;
  };
  // both lane halves' sums of the column, in each half
  auto combine = [&](float p, float ks) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    const float v = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * a.sm_scale;
    return T::ROWSCALE ? v * ks : v;
  };
  f32x16 accA = {}, accB = {};
  float p = 0.f;
  float kprev = 1.f;
  auto block = [&](const uint32_t (&bf)[QD], uint32_t kword, int u) {
    mfma_block(accA, qf[0], bf);        // heads 0-31 of u   ||
    p = epi_relu(accB, wv[1], p);       //   heads 32-63 of u-1, completing u-1
    const float v = combine(p, kprev);
    kprev = __uint_as_float(kword);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(accB, qf[1], bf);        // heads 32-63 of u  ||
    p = epi_relu(accA, wv[0], 0.f);     //   heads 0-31 of u
    __builtin_amdgcn_sched_barrier(0);
    store(v, u - 1);
  };
  constexpr int NB = 2;
  uint32_t bfs[NB][QD];
  uint32_t kws[NB] = {};
  kload(0, bfs[0], kws[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  for (int st = 0; st < n_pairs; ++st) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = NB * st + i;
      kload(u + 1, bfs[1 - i], kws[1 - i]);
      block(bfs[i], kws[i], u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  p = epi_relu(accB, wv[1], p);
  store(combine(p, kprev), 2 * n_pairs - 1);
  if (own_clean) clean_row_outside<OBF>(a, row, u.cl0, u.cl1, lane);
}

// ---------------------------------------------------------------------------
// 64-head kernel for FP8 and MXFP8 keys in fragment order, on 16x16x128 MFMAs
//
// Same units, rows per wave, windows and stores as score_kernel, but each wave
// cleans its own rows outside the coverage (no cleanup units); the
// contraction and the linear term are cut differently.  A 16x16x128 block
// takes all 128 d at once: A = 16 heads of one query row, B = 16 key columns.
// Per 32 columns a wave issues 2 rows x 4 head blocks x 2 column halves = 16
// of them (32 cycles each at the e4m3 rate, as many cycles as the eight
// 32x32x64 blocks of score_kernel), but the linear term qt . k now takes two
// blocks of 32 cycles instead of two of 64: A rows 0-3 / 8-11 (first column
// half) and 4-7 / 12-15 (second half) hold the four weighted-query
// pieces of rows 0 / 1, chained into one accumulator, so lane l ends up with
// row l/32, column l%32 of the linear term -- where the head-sum below puts
// the same cell.
//
// gfx950 operand placement of the scaled 16x16x128 e4m3 MFMA (probed on the
// GPU with random codes and scales): lane (n, q), n = l%16, q = l/16, holds
// row / column n, bytes 0-15 at k = 16q + [0,16) and bytes 16-31 at
// k = 64 + 16q + [0,16); k-block b = [32b, 32b+32) takes lane group b's scale
// byte.  With k = d, lane (n, q) therefore holds d-chunks q and q + 4 of 16
// bytes, and its scale byte is byte q of the E8M0 word (d-block q).  K in
// fragment order keeps chunk p of column c at (p/2)*1024 + (32*(p%2) + c)*16
// of its block, so each column half is two 16-byte loads per lane at a
// constant lane offset.
//
// Output: lane (n, q) register r = A row 4q + r, column n.  Each lane weights
// and sums its 4 heads per block into p[row][half]; two permlane32 swaps then
// one permlane16 swap fold the four lane groups so that lane l holds row l/32,
// column l%32 (16 (l/16 % 2) + l%16).
//
// Four weighted-query pieces leave a residual below 2^-16 of each d-block
// maximum of qt; by Cauchy-Schwarz its share of a score is at most
// 2^-16 sqrt(32) / 2 < 4.4e-5 of sm_scale * sum_h |w_h| |q_h| |k|.
template <int F, bool WBF, bool OBF, bool CLEAN, bool PD, bool SEL = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
    score_kernel_x16(const ScoreArgs a) {
  static_assert(F == IDX_IN_FP8_E4M3 || F == IDX_IN_MXFP8_E4M3, "e4m3 formats only");
  static_assert(!SEL || (!CLEAN && !PD), "select mode stores no scores and reads contiguous keys");
  if constexpr (SEL) {
    if (a.gate != nullptr && *a.gate == 0) return;  // a second pass with no row to redo
  }
  using T = Fmt<F>;
  static_assert(T::ROWB == 128 && T::CBASE == 16 && T::CSTRIDE == 32, "K fragment placement of the e4m3 formats");
  constexpr bool MX = T::MX;
  constexpr int TW = 2;  // query rows per wave
  constexpr int kLinPieces = 4;
  static_assert(kLinPieces <= PieceFmt<F>::N, "pieces written by the preparation");
  typedef float f32x4 __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4, g = lane >> 5, c = lane & 31;

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(a.plan);
  const bool plan_ok = hdr->magic == kPlanMagic && hdr->B == a.B && hdr->S_q == a.S_q && hdr->S_k == a.S_k &&
                       hdr->H == 64 && hdr->D == 128 && hdr->tile_rows == kTileRows && hdr->n_tiles == a.n_tiles;
  // one work position per workgroup, dealt in order by the hardware
  const int pos = int(blockIdx.x);
  if (pos >= a.n_pos_compute) {
    cleanup_unit<OBF, CLEAN, kTileRows>(a, pos - a.n_pos_compute, plan_ok);
    return;
  }
  // with no cleanup units in the launch, each wave cleans its own rows
  const bool own_clean = CLEAN && !PD && !SEL && units_clean_own_rows(a);
  if (!plan_ok) {
    if (own_clean && pos % a.n_chunk == 0) cleanup_unit<OBF, CLEAN, kTileRows>(a, pos / a.n_chunk, false);
    return;
  }
  const Unit u = decode_unit(a, pos);
  if (u.kind != kUnitCompute) {
    if (own_clean && u.tile >= 0 && u.cl1 < a.S_k) {  // a tile whose rows all see nothing
      const int32_t* srow = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
      for (int t = 0; t < 2; ++t) {
        const int r = __builtin_amdgcn_readfirstlane(srow[int64_t(u.tile) * kTileRows + wave * 2 + t]);
        if (r >= 0) clean_row_outside<OBF>(a, r, 0, 0, lane);
      }
    }
    return;
  }
  const int tile = u.tile;
  int c0 = u.c0, c1 = u.c1;  // columns [c0, c1) of the tile are this unit's
  // the wave whose tile slots hold this wave's rows: its own, or with
  // decode-sized tiles (wave_split: at most two rows per batch) slots 0 and 1
  // for every wave, each wave taking a quarter of the unit's columns
  int slot_wave = wave;
  if (!SEL && a.wave_split) {
    const int per = (((c1 - c0 + 63) / 64) + 3) / 4;  // 64-column pairs per wave
    const int w0 = c0 + 64 * per * wave;
    c1 = min(c1, w0 + 64 * per);
    c0 = w0;
    if (c0 >= c1) return;
    slot_wave = 0;
  }
  const int n_pairs = (c1 - c0 + 63) / 64;
  const int b = tile / a.tiles_per_batch;

  const int32_t* slot_row = reinterpret_cast<const int32_t*>(a.plan + a.off_slot);
  const int32_t first_row = slot_row[int64_t(tile) * kTileRows];
  int rows[TW];
  bool rvalid[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int r = slot_row[int64_t(tile) * kTileRows + slot_wave * TW + t];
    rvalid[t] = r >= 0;
    rows[t] = r >= 0 ? r : first_row;
  }
  if (!rvalid[0] && !rvalid[1]) return;
  // select mode: the rows' thresholds; a wave whose rows keep nothing is done
  uint32_t tau_r[TW] = {kTauNone, kTauNone};
  if constexpr (SEL) {
#pragma unroll
    for (int t = 0; t < TW; ++t) tau_r[t] = rvalid[t] ? a.tau[rows[t]] : kTauNone;
    if (tau_r[0] == kTauNone && tau_r[1] == kTauNone) return;
  }

  // Q: head 16 mb + n of row t, d-chunks q and q + 4, scale byte q
  i32x8 qf[TW][4];
  uint32_t sq[TW][4];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int64_t qrow = int64_t(rows[t]) * 64 + 16 * mb + n;
      const unsigned char* src = static_cast<const unsigned char*>(a.q) + qrow * 128 + 16 * q;
      const uint4 x0 = *reinterpret_cast<const uint4*>(src);
      const uint4 x1 = *reinterpret_cast<const uint4*>(src + 64);
      qf[t][mb] = i32x8{int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
      sq[t][mb] = MX ? uint32_t(static_cast<const uint8_t*>(a.q_scale)[qrow * 4 + q]) : 127u;
    }
  }
  // weights of the lane's output heads: register r of head block mb is head
  // 16 mb + 4 q + r
  float wv[TW][4][4];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int64_t off = int64_t(rows[t]) * 64 + 16 * mb + 4 * q;
      if constexpr (WBF) {
        const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.w) + off);
        wv[t][mb][0] = __uint_as_float(x.x << 16);
        wv[t][mb][1] = __uint_as_float(x.x & 0xFFFF0000u);
        wv[t][mb][2] = __uint_as_float(x.y << 16);
        wv[t][mb][3] = __uint_as_float(x.y & 0xFFFF0000u);
      } else {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(a.w) + off);
        wv[t][mb][0] = x.x;
        wv[t][mb][1] = x.y;
        wv[t][mb][2] = x.z;
        wv[t][mb][3] = x.w;
      }
    }
  }
  // sm_scale / 2 rides on the weights, so a block's fold needs no multiply
  // for it: the |S| sums come out scaled, the linear term is scaled as it
  // is added
  const float half_scale = 0.5f * a.sm_scale;
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[t][mb][e] *= half_scale;
  // pieces: A row n is piece n%4 of row n/8, in the first column half's
  // operand (le) when n%8 < 4, else in the second's (lo); zero elsewhere
  i32x8 le, lo;
  uint32_t sle, slo;
  {
    const int t = n >> 3, p = n & 3;
    const bool odd = (n & 4) != 0;
    const int64_t prow = t ? rows[1] : rows[0];
    const unsigned char* src = a.pieces + prow * kPieceRowBytes + p * PieceFmt<F>::BYTES + 16 * q;
    const uint4 x0 = *reinterpret_cast<const uint4*>(src);
    const uint4 x1 = *reinterpret_cast<const uint4*>(src + 64);
    const i32x8 v = {int(x0.x), int(x0.y), int(x0.z), int(x0.w), int(x1.x), int(x1.y), int(x1.z), int(x1.w)};
    const i32x8 z = {};
    const uint32_t sb = static_cast<const uint8_t*>(static_cast<const void*>(a.pscales))[(prow * kPieceSlots + p) * 4 + q];
    le = odd ? z : v;
    lo = odd ? v : z;
    sle = odd ? 127u : sb;
    slo = odd ? sb : 127u;
  }

  // half-wave g stores row g of the wave: its window relative to c0
  const int my_row = g ? rows[1] : rows[0];
  const int my_s = reinterpret_cast<const int32_t*>(a.plan + a.off_start)[my_row];
  const int my_e = reinterpret_cast<const int32_t*>(a.plan + a.off_end)[my_row];

  // K column halves: lane (n, q) reads column 16 h + n, d-chunks q and q + 4;
  // MX: the E8M0 byte of d-block q of that column; FP8: the fp32 row scale of
  // column l%32, which the lane stores.  Blocks past the end of K are clamped
  // to the last one: in bounds, and never stored.  From a paged cache (PD) a
  // block's 32 keys are 32 consecutive rows of one page, as in score_kernel.
  const int nblk = (a.S_k + 31) >> 5;
  const int kb0 = c0 >> 5;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(a.kfrag) + int64_t(b) * nblk * (32 * 128), 0, nblk * (32 * 128), kBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.kscale) + int64_t(b) * nblk * 64, 0, nblk * 256, kBufWord3);
  const __amdgpu_buffer_rsrc_t pkrs =
      PD ? __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(a.kcache), 0,
                                             int(uint32_t(a.num_pages) * uint32_t(a.page_size) * 128u), kBufWord3)
         : krs;
  const __amdgpu_buffer_rsrc_t psrs =
      PD ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(a.kscache), 0,
                                             int(uint32_t(a.num_pages) * uint32_t(a.page_size) * 4u), kBufWord3)
         : srs;
  const int32_t* btrow = PD ? a.btable + int64_t(b) * a.max_pages : nullptr;
  // paged: blocks are loaded in order, and the page of the next one is read
  // from the block table one load ahead, off the path of the key loads
  int pg_next = 0;
  if constexpr (PD) pg_next = __builtin_amdgcn_readfirstlane(btrow[uint32_t(min(kb0, nblk - 1)) >> a.bpp_shift]);
  const int koff = (q >> 1) * 1024 + (32 * (q & 1) + n) * 16;
  auto kload = [&](int u, i32x8 (&bf)[2], uint32_t (&sb)[2], uint32_t& ks) {
    const int blk = min(kb0 + u, nblk - 1);
    if constexpr (PD) {
      const uint32_t rem = uint32_t(blk) & ((1u << a.bpp_shift) - 1u);
      int pg = pg_next;
      pg_next = __builtin_amdgcn_readfirstlane(btrow[uint32_t(min(blk + 1, nblk - 1)) >> a.bpp_shift]);
      pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
      const uint32_t row0 = uint32_t(pg) * uint32_t(a.page_size) + rem * 32u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(pkrs, (16 * h + n) * 128 + 16 * q, int(row0 * 128u), 0);
        const u32x4 x1 =
            __builtin_amdgcn_raw_buffer_load_b128(pkrs, (16 * h + n) * 128 + 16 * q + 64, int(row0 * 128u), 0);
        bf[h] = i32x8{int(x0[0]), int(x0[1]), int(x0[2]), int(x0[3]), int(x1[0]), int(x1[1]), int(x1[2]), int(x1[3])};
        if constexpr (MX)
          sb[h] = uint32_t(__builtin_amdgcn_raw_buffer_load_b8(psrs, (16 * h + n) * 4 + q, int(row0 * 4u), 0));
        else
          sb[h] = 127u;
      }
      if constexpr (!MX) ks = __builtin_amdgcn_raw_buffer_load_b32(psrs, c * 4, int(row0 * 4u), 0);
      return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 256 * h, blk * (32 * 128), 0);
      const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 256 * h + 2048, blk * (32 * 128), 0);
      bf[h] = i32x8{int(x0[0]), int(x0[1]), int(x0[2]), int(x0[3]), int(x1[0]), int(x1[1]), int(x1[2]), int(x1[3])};
      if constexpr (MX)
        sb[h] = uint32_t(__builtin_amdgcn_raw_buffer_load_b8(srs, (16 * h + n) * 4 + q, blk * 256, 0));
      else
        sb[h] = 127u;
    }
    if constexpr (!MX) ks = __builtin_amdgcn_raw_buffer_load_b32(srs, lane * 4, blk * 256, 0);
  };

  auto mfma16 = [&](const i32x8& av, uint32_t sA, const i32x8& bv, uint32_t sB, const f32x4& acc) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, int(sA), 0, int(sB));
  };

  // stores: as in score_kernel (one buffer resource per row, drops instead of
  // branches), -inf by one select
  constexpr int ES = OBF ? 2 : 4;
  constexpr uint32_t kDrop = 0x80000000u;
  __amdgpu_buffer_rsrc_t ors[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t)
    ors[t] = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char*>(a.out) + (int64_t(rows[t]) * a.ld + c0) * ES, 0, rvalid[t] ? (c1 - c0) * ES : 0,
        kBufWord3);
  const uint32_t half0 = g ? kDrop : 0u, half1 = g ? 0u : kDrop;
  const uint32_t s_rel = uint32_t(my_s - c0) * ES;
  const uint32_t w_len = uint32_t(max(my_e - my_s, 0)) * ES;
  // select mode: the rows' candidate areas, the lane's row's threshold and count
  __amdgpu_buffer_rsrc_t crs[TW];
  if constexpr (SEL) {
#pragma unroll
    for (int t = 0; t < TW; ++t) crs[t] = sel_rsrc(a, rows[t], rvalid[t], c0, c1 - c0);
  }
  uint32_t sel_cnt[TW] = {0u, 0u};
  const SelTau stau = sel_tau(tau_r[0], tau_r[1]);
  uint32_t sel_lo = 0, sel_len = 0;
  if constexpr (SEL) sel_window(my_s, my_e, c0, c1, sel_lo, sel_len);
  auto store = [&](float v, int u) {
    if constexpr (SEL) {
      sel_emit<OBF>(v, u, c, g, uint32_t(c0), sel_lo, sel_len, stau, sel_cnt[0], sel_cnt[1], crs[0], crs[1]);
      return;
    }
    const uint32_t off = uint32_t(32 * u + c) * ES;  // u = -1 wraps to a huge offset: dropped
    const bool inwin = off - s_rel < w_len;
    uint32_t o0 = off | half0, o1 = off | half1;
    if constexpr (!CLEAN) {
      o0 = inwin ? o0 : kDrop;
      o1 = inwin ? o1 : kDrop;
    }
    float val = v;
    if constexpr (CLEAN) val = inwin ? v : -__builtin_inff();  // one select
    if constexpr (OBF) {
      const uint16_t hv = __builtin_bit_cast(uint16_t, static_cast<__bf16>(val));
      // cached, as in score_kernel: the line's other half comes with the next block
      __builtin_amdgcn_raw_buffer_store_b16(hv, ors[0], int(o0), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(hv, ors[1], int(o1), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors[0], int(o0), 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors[1], int(o1), 0, kNonTemporal);
    }
  };

  // p[row][half]: weighted |S| of the lane's heads (weights carry
  // sm_scale / 2); fold the lane groups
  auto combine = [&](const float (&p)[TW][2], float lin, float ks) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0][0]), __float_as_uint(p[1][0]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0][1]), __float_as_uint(p[1][1]), false, false);
    const float x = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
    const float y = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
    const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const float tot = __builtin_fmaf(lin, half_scale, __uint_as_float(s2[0]) + __uint_as_float(s2[1]));
    return MX ? tot : tot * ks;
  };

  // Software pipeline over steps: per 32-column block 18 MFMAs, column half
  // by column half: the half's linear MFMA, then its 8 (row, head block)
  // MFMAs, so the B operand changes twice per block (measured about 1 %
  // faster than alternating it every MFMA, under the same power limit).  The
  // epilogue of a step runs three steps later, behind three other MFMAs, so
  // it never waits for the matrix pipe.  Accumulators rotate over four slots
  // (36 steps per loop iteration of two blocks is a multiple of four).  A
  // block's head-sum is folded and stored one step after its last epilogue.
  constexpr int kSteps = 18, kLag = 3;
  constexpr int kLin2 = 9;  // step of the second half's linear MFMA
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accL[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  float p[2][TW][2] = {};
  float lin[2] = {0.f, 0.f};
  float kblk[2] = {1.f, 1.f};
  i32x8 bfs[2][2];
  uint32_t sbs[2][2];
  uint32_t kss[2] = {0u, 0u};

  // epilogue of step j (0 <= j < 2 kSteps) of a loop iteration
  auto epilogue = [&](int j) {
    const int i = j / kSteps, k = j % kSteps;
    if (k == kLin2) {
      const f32x4& r = accL[i];
      lin[i] = (r[0] + r[1]) + (r[2] + r[3]);
    } else if (k != 0) {
      const int hb = k < kLin2 ? k - 1 : k - 2, h = hb >> 3, t = (hb >> 2) & 1, mb = hb & 3;
      float s = mb == 0 ? 0.f : p[i][t][h];
      const f32x4& r = acc[j & 3];
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_fmaf(wv[t][mb][e], __builtin_fabsf(r[e]), s);
      p[i][t][h] = s;
    }
  };

  kload(0, bfs[0], sbs[0], kss[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // The loop carries block 0's scale bytes from one iteration to the next.
  // Hiding the prologue's values from the optimiser keeps their zero
  // extension ahead of the loop-carried merge, where the loads already did
  // it; otherwise a mask per byte lands at the top of every iteration.
  if constexpr (MX) asm volatile("" : "+v"(sbs[0][0]), "+v"(sbs[0][1]));
  const int n_iter = n_pairs;  // two blocks per iteration
  for (int s = 0; s < n_iter; ++s) {
#pragma unroll
    for (int j = 0; j < 2 * kSteps; ++j) {
      const int i = j / kSteps, k = j % kSteps;
      const int u = 2 * s + i;
      if (k == 0) {
        kblk[i] = __uint_as_float(kss[i]);
        kload(u + 1, bfs[1 - i], sbs[1 - i], kss[1 - i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (k == 0) {
        accL[i] = mfma16(le, sle, bfs[i][0], sbs[i][0], f32x4{0.f, 0.f, 0.f, 0.f});
      } else if (k == kLin2) {
        accL[i] = mfma16(lo, slo, bfs[i][1], sbs[i][1], accL[i]);
      } else {
        const int hb = k < kLin2 ? k - 1 : k - 2, h = hb >> 3, t = (hb >> 2) & 1, mb = hb & 3;
        acc[j & 3] = mfma16(qf[t][mb], sq[t][mb], bfs[i][h], sbs[i][h], f32x4{0.f, 0.f, 0.f, 0.f});
      }
      // the epilogue of step j - kLag (of the previous iteration for j < kLag)
      epilogue((j - kLag + 2 * kSteps) % (2 * kSteps));
      // the previous block's last epilogue ran one step ago: fold and store it
      if (k == kLag) {
        const int pi = 1 - i;
        store(combine(p[pi], lin[pi], kblk[pi]), u - 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // drain: the last block's final epilogues, then its fold and store
#pragma unroll
  for (int j = 2 * kSteps - kLag; j < 2 * kSteps; ++j) epilogue(j);
  store(combine(p[1], lin[1], kblk[1]), 2 * n_iter - 1);
  if constexpr (SEL) {
    if (c == 0 && (g ? rvalid[1] : rvalid[0])) sel_finish(a, my_row, u.chunk, c0, g ? sel_cnt[1] : sel_cnt[0]);
  }
  if (own_clean) {
#pragma unroll
    for (int t = 0; t < TW; ++t)
      if (rvalid[t]) clean_row_outside<OBF>(a, rows[t], u.cl0, u.cl1, lane);
  }
}

// One launch of `kernel`: a workgroup per work position.
template <typename K>
hipError_t launch_units(K kernel, const ScoreArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kernel, dim3(unsigned(a.n_positions)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int F, bool WBF, bool OBF, bool CLEAN>
hipError_t launch_score_t(const ScoreArgs& a, hipStream_t stream) {
  const bool pd = a.kcache != nullptr;
  if (a.cand != nullptr) {  // select mode: launched without cleaning, on contiguous keys
    if constexpr (CLEAN) {
      return hipErrorInvalidValue;
    } else {
      if (pd) return hipErrorInvalidValue;
      if constexpr (F == IDX_IN_FP8_E4M3 || F == IDX_IN_MXFP8_E4M3)
        return launch_units(score_kernel_x16<F, WBF, OBF, false, false, true>, a, stream);
      else
        return launch_units(score_kernel<F, WBF, OBF, false, false, true>, a, stream);
    }
  }
  // the plain FP8-family kernel cleans its own rows: no cleanup units (the
  // MXFP4 / generic kernel keeps them: there the cleaning lengthened the last
  // chunks of long rows, which end the launch)
  ScoreArgs own = a;
  if (CLEAN && !pd && !a.wave_split && !a.dyn_units) own.n_positions = a.n_pos_compute;
  if constexpr (F == IDX_IN_FP8_E4M3 || F == IDX_IN_MXFP8_E4M3) {
    if (pd) return launch_units(score_kernel_x16<F, WBF, OBF, CLEAN, true>, a, stream);
    return launch_units(score_kernel_x16<F, WBF, OBF, CLEAN, false>, own, stream);
  } else if (pd) {
    if constexpr (F == kInBF16RowScale) return hipErrorInvalidValue;  // converted keys are never read from a cache
    else
      return launch_units(score_kernel<F, WBF, OBF, CLEAN, true>, a, stream);
  } else {
    if constexpr (bf16_operands(F)) {
      // one row per wave: two positions per compute unit; with cleaning, each
      // wave cleans its own row (no cleanup units)
      const int64_t n_clean = CLEAN ? 0 : int64_t(a.n_positions) - a.n_pos_compute;
      if (!a.wave_split && !a.dyn_units && 2 * int64_t(a.n_pos_compute) + n_clean < (int64_t(1) << 31)) {
        ScoreArgs h = a;
        h.n_pos_compute = 2 * a.n_pos_compute;
        h.n_positions = int32_t(h.n_pos_compute + n_clean);
        return launch_units(score_kernel_bf16w<F, WBF, OBF, CLEAN>, h, stream);
      }
    }
    return launch_units(score_kernel<F, WBF, OBF, CLEAN, false>, a, stream);
  }
}

}  // namespace idx
