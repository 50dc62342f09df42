/*
 * Plain fp64 CPU oracle for lightning-indexer scoring ("MQA logits").
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the GPU library.
 *
 * What it computes is the plain definition of the scoring, written out:
 *
 *   score[b,i,j] = sm_scale * sum_{h ascending} w[b,i,h] * max(0, dot_h)
 *   dot_h        = sum_{d ascending} Qd[b,i,h,d] * Kd[b,j,d]
 *
 * for start[b,i] <= j < end[b,i], and -inf for every other column.  The pages
 * name the operation and its pieces without printing the formula: the
 * DeepGEMM pull request 435 ("Improve SM100 MX MQA logits clean-output
 * performance", Performance section and reproducer) fixes the shapes q[m,64,D],
 * k[n,D], w[m,64], output [m,n] with per-row windows [start, end); the
 * cudnn-frontend pull request 416 ("DSA indexer forward: add a lean SM100 fast
 * path", What and Precision / determinism sections) fixes the one shared KV
 * head for 64 query heads, the per-call sm_scale, the head-sum and fp32
 * scores with -inf outside the window.  ReLU on each head's dot and the
 * weighting before the head-sum follow the plainest reading of those pieces.
 *
 * Dequantisation is exact in fp64 and follows the public OCP 8-bit float and
 * OCP Microscaling v1.0 definitions:
 *   bf16  : the 16 bits are the top half of an IEEE binary32
 *   e4m3fn: (-1)^s 2^(e-7) (1 + m/8) for e >= 1, (-1)^s 2^-6 (m/8) for e = 0,
 *           S.1111.111 is NaN, no infinities
 *   e2m1  : (-1)^s 2^(e-1) (1 + m/2) for e >= 1, (-1)^s (m/2) for e = 0
 *   E8M0  : 2^(e-127), 0xFF is NaN
 * FP8 inputs carry one fp32 scale per K row, folded into Kd.  MX inputs carry
 * one E8M0 byte per 32 elements of D: byte b (bits 8b..8b+7) of the int32 word
 * scales elements [32b, 32b+32); MXFP4 stores two codes per byte, the low
 * nibble holding the even element.
 *
 * Windows: explicit [start,end) are clamped as s = clamp(start,0,S_k),
 * e = clamp(end,s,S_k).  From a per-batch causal offset the window is
 * [0, clamp(S_k - S_q + off + i + 1, 0, S_k)), in 64-bit arithmetic (the
 * offset convention that cudnn-frontend pull request 416 states for its
 * legacy kernel, "What" section, aligned so that offset 0 lets the last
 * query row see every key).
 *
 * Alongside each score the oracle returns the per-cell error scale
 *   bound = |sm_scale| * |Kd[j]|_2 * sum_h |w[h]| * |Qd[h]|_2
 * against which a result's deviation is measured.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_FP8 = 1, OR_MXFP8 = 2, OR_MXFP4 = 3 };
enum { OR_W_F32 = 0, OR_W_BF16 = 1 };

double oracle_dec_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_dec_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

double oracle_dec_e2m1(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 0x3, m = c & 1;
  double v;
  if (e == 0)
    v = 0.5 * (double)m;
  else
    v = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -v : v;
}

double oracle_dec_e8m0(uint8_t e) {
  if (e == 0xFF) return NAN;
  return ldexp(1.0, (int)e - 127);
}

/* Element d of one row of codes, before any block scale. */
static double dec_elem(int fmt, const void* row, int d) {
  switch (fmt) {
    case OR_BF16: return oracle_dec_bf16(((const uint16_t*)row)[d]);
    case OR_FP8:
    case OR_MXFP8: return oracle_dec_e4m3(((const uint8_t*)row)[d]);
    default: {
      uint8_t byte = ((const uint8_t*)row)[d >> 1];
      return oracle_dec_e2m1((d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF));
    }
  }
}

static size_t row_bytes(int fmt, int D) {
  switch (fmt) {
    case OR_BF16: return (size_t)D * 2;
    case OR_FP8:
    case OR_MXFP8: return (size_t)D;
    default: return (size_t)D / 2;
  }
}

/* Window of every row, [B*S_q] each.  Explicit starts/ends (both non-NULL) win
 * over offsets; offsets NULL means offset 0 for every batch. */
void oracle_windows(int B, int S_q, int S_k, const int32_t* offsets, const int32_t* starts,
                    const int32_t* ends, int32_t* win_start, int32_t* win_end) {
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < S_q; ++i) {
      int64_t r = (int64_t)b * S_q + i, s, e;
      if (starts && ends) {
        s = starts[r];
        e = ends[r];
        if (s < 0) s = 0;
        if (s > S_k) s = S_k;
        if (e < s) e = s;
        if (e > S_k) e = S_k;
      } else {
        int64_t off = offsets ? (int64_t)offsets[b] : 0;
        s = 0;
        e = (int64_t)S_k - (int64_t)S_q + off + (int64_t)i + 1;
        if (e < 0) e = 0;
        if (e > S_k) e = S_k;
      }
      win_start[r] = (int32_t)s;
      win_end[r] = (int32_t)e;
    }
  }
}

/*
 * Packed variable-length (THD) windows with ratio-compressed keys, as the
 * cudnn-frontend pull request 416 describes them ("DSA indexer forward",
 * THD/varlen commit): query tokens of n_seg segments are packed into one row
 * range (segment s holds rows [cu_q[s], cu_q[s+1])), their compressed keys
 * into one column range (segment s holds [cu_k[s], cu_k[s+1])), and every row
 * sees an absolute window that starts at its segment's first key.  The pages
 * give the start (cu_seqlens_k of the segment) and say the window length is
 * the ratio-causal visible count without printing it; the reading taken here
 * is that compressed key c of a segment stands for its query tokens
 * [c*ratio, (c+1)*ratio) and becomes visible once all of them are, so the
 * local row t sees floor((t + 1) / ratio) keys.  The window never leaves its
 * segment; rows outside every segment see nothing.  Everything is clamped to
 * [0, m_total] in 64-bit integers.
 */
void oracle_windows_thd(int n_seg, const int32_t* cu_q, const int32_t* cu_k, int ratio, int T_q, int m_total,
                        int32_t* win_start, int32_t* win_end) {
  for (int i = 0; i < T_q; ++i) {
    win_start[i] = 0;
    win_end[i] = 0;
  }
  for (int seg = 0; seg < n_seg; ++seg) {
    for (int64_t i = cu_q[seg]; i < cu_q[seg + 1]; ++i) {
      if (i < 0 || i >= T_q) continue;
      const int64_t t = i - cu_q[seg];
      int64_t s = cu_k[seg], e = s + (t + 1) / ratio, lim = cu_k[seg + 1];
      if (e > lim) e = lim;
      if (s < 0) s = 0;
      if (s > m_total) s = m_total;
      if (e < s) e = s;
      if (e > m_total) e = m_total;
      win_start[i] = (int32_t)s;
      win_end[i] = (int32_t)e;
    }
  }
}

/*
 * Paged keys (decode): request b holds ctx[b] keys in pages of page_size
 * rows; its logical key j is row j % page_size of physical page
 * block_table[b * max_pages + j / page_size].  The pages name paged MQA
 * logits (DeepGEMM pull request 435, Validation section: the paged test
 * shares the scoring core) without printing the layout; this is the plainest
 * one, and the windows follow: query token i of the request's S_q newest
 * tokens sees [0, ctx - S_q + i + 1), clamped to [0, S_k] (ctx itself clamped
 * to [0, S_k]).
 *
 * oracle_gather_paged writes the dense K of every request ([B, S_k] rows of
 * row_bytes, and its per-row scale words when scale_bytes > 0), zero past the
 * request's keys.
 */
void oracle_gather_paged(int B, int S_k, int row_bytes, int scale_bytes, const uint8_t* k_cache,
                         const uint8_t* k_scale_cache, const int32_t* block_table, const int32_t* ctx,
                         int page_size, int max_pages, uint8_t* k_out, uint8_t* k_scale_out) {
  for (int b = 0; b < B; ++b) {
    int64_t n = ctx[b];
    if (n < 0) n = 0;
    if (n > S_k) n = S_k;
    for (int64_t j = 0; j < S_k; ++j) {
      uint8_t* dst = k_out + ((int64_t)b * S_k + j) * row_bytes;
      uint8_t* sdst = scale_bytes ? k_scale_out + ((int64_t)b * S_k + j) * scale_bytes : 0;
      if (j < n) {
        const int64_t page = block_table[(int64_t)b * max_pages + j / page_size];
        const int64_t row = page * page_size + j % page_size;
        memcpy(dst, k_cache + row * row_bytes, (size_t)row_bytes);
        if (scale_bytes) memcpy(sdst, k_scale_cache + row * scale_bytes, (size_t)scale_bytes);
      } else {
        memset(dst, 0, (size_t)row_bytes);
        if (scale_bytes) memset(sdst, 0, (size_t)scale_bytes);
      }
    }
  }
}

void oracle_windows_paged(int B, int S_q, int S_k, const int32_t* ctx, int32_t* win_start, int32_t* win_end) {
  for (int b = 0; b < B; ++b) {
    int64_t n = ctx[b];
    if (n < 0) n = 0;
    if (n > S_k) n = S_k;
    for (int i = 0; i < S_q; ++i) {
      int64_t e = n - S_q + i + 1;
      if (e < 0) e = 0;
      if (e > S_k) e = S_k;
      win_start[(int64_t)b * S_q + i] = 0;
      win_end[(int64_t)b * S_q + i] = (int32_t)e;
    }
  }
}

/* Dequantised K of one batch: Kd[j*D + d] and |Kd[j]|_2 in kn[j]. */
static void dequant_k(int fmt, int S_k, int D, const uint8_t* kb, const void* k_scale_b, double* Kd,
                      double* kn) {
  size_t rb = row_bytes(fmt, D);
  for (int j = 0; j < S_k; ++j) {
    const void* row = kb + (size_t)j * rb;
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
      double v = dec_elem(fmt, row, d);
      if (fmt == OR_FP8) v *= (double)((const float*)k_scale_b)[j];
      if (fmt == OR_MXFP8 || fmt == OR_MXFP4) {
        uint32_t word = ((const uint32_t*)k_scale_b)[j];
        v *= oracle_dec_e8m0((uint8_t)(word >> (8 * (d / 32))));
      }
      Kd[(size_t)j * D + d] = v;
      ss += v * v;
    }
    kn[j] = sqrt(ss);
  }
}

/*
 * Scores of the listed rows (global row ids b*S_q+i; rows == NULL means all
 * B*S_q rows in order).  ref and bound are [n_rows, S_k] fp64.  Returns the
 * number of OpenMP threads used, or -1 on bad arguments / allocation failure.
 * threads <= 0 uses the OpenMP default.
 */
int oracle_mqa_logits(int B, int S_q, int S_k, int H, int D, int fmt, const void* q,
                      const uint32_t* q_scale, const void* k, const void* k_scale, const void* w,
                      int w_fmt, double sm_scale, const int32_t* win_start, const int32_t* win_end,
                      const int64_t* rows, int64_t n_rows, double* ref, double* bound, int threads) {
  if (B <= 0 || S_q <= 0 || S_k <= 0 || H <= 0 || D <= 0) return -1;
  if ((fmt == OR_MXFP8 || fmt == OR_MXFP4) && (D % 32 != 0 || D > 128)) return -1;
  if (fmt == OR_MXFP4 && D % 2 != 0) return -1;
  if (!rows) n_rows = (int64_t)B * S_q;
  size_t qrb = row_bytes(fmt, D);
  double* Kd = (double*)malloc(sizeof(double) * (size_t)B * S_k * D);
  double* kn = (double*)malloc(sizeof(double) * (size_t)B * S_k);
  if (!Kd || !kn) {
    free(Kd);
    free(kn);
    return -1;
  }
  for (int b = 0; b < B; ++b) {
    const void* ksb = NULL;
    if (fmt == OR_FP8) ksb = (const float*)k_scale + (size_t)b * S_k;
    if (fmt == OR_MXFP8 || fmt == OR_MXFP4) ksb = (const uint32_t*)k_scale + (size_t)b * S_k;
    dequant_k(fmt, S_k, D, (const uint8_t*)k + (size_t)b * S_k * qrb, ksb, Kd + (size_t)b * S_k * D,
              kn + (size_t)b * S_k);
  }
  int used = 1;
  int fail = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : omp_get_max_threads())
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    /* Qt[d*H + h] = Qd[h][d]: laid out so the inner loop runs over heads and
     * every per-head dot still sums d in ascending order */
    double* Qt = (double*)malloc(sizeof(double) * (size_t)H * D);
    double* qn = (double*)malloc(sizeof(double) * (size_t)H);
    double* wd = (double*)malloc(sizeof(double) * (size_t)H);
    double* dot = (double*)malloc(sizeof(double) * (size_t)H);
    if (!Qt || !qn || !wd || !dot) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t n = 0; n < n_rows; ++n) {
        int64_t r = rows ? rows[n] : n;
        int b = (int)(r / S_q);
        double* out = ref + (size_t)n * S_k;
        double* bnd = bound + (size_t)n * S_k;
        for (int h = 0; h < H; ++h) {
          const uint8_t* qrow = (const uint8_t*)q + ((size_t)r * H + h) * qrb;
          double ss = 0.0;
          for (int d = 0; d < D; ++d) {
            double v = dec_elem(fmt, qrow, d);
            if (fmt == OR_MXFP8 || fmt == OR_MXFP4) {
              uint32_t word = q_scale[(size_t)r * H + h];
              v *= oracle_dec_e8m0((uint8_t)(word >> (8 * (d / 32))));
            }
            Qt[(size_t)d * H + h] = v;
            ss += v * v;
          }
          qn[h] = sqrt(ss);
          wd[h] = (w_fmt == OR_W_F32) ? (double)((const float*)w)[(size_t)r * H + h]
                                      : oracle_dec_bf16(((const uint16_t*)w)[(size_t)r * H + h]);
        }
        int32_t s = win_start[r], e = win_end[r];
        for (int j = 0; j < S_k; ++j) {
          if (j < s || j >= e) {
            out[j] = -INFINITY;
            bnd[j] = 0.0;
            continue;
          }
          const double* kj = Kd + ((size_t)b * S_k + j) * D;
          for (int h = 0; h < H; ++h) dot[h] = 0.0;
          for (int d = 0; d < D; ++d) {
            const double kv = kj[d];
            const double* qd = Qt + (size_t)d * H;
            for (int h = 0; h < H; ++h) dot[h] += qd[h] * kv;
          }
          double acc = 0.0, bs = 0.0;
          for (int h = 0; h < H; ++h) {
            double relu = dot[h] > 0.0 ? dot[h] : 0.0;
            acc += wd[h] * relu;
            bs += fabs(wd[h]) * qn[h];
          }
          out[j] = sm_scale * acc;
          bnd[j] = fabs(sm_scale) * kn[(size_t)b * S_k + j] * bs;
        }
      }
    }
    free(Qt);
    free(qn);
    free(wd);
    free(dot);
  }
  free(Kd);
  free(kn);
  return fail ? -1 : used;
}

/*
 * Top-k selection over scores (the selection the pages place after the
 * indexer: the sparse-attention page consumes a fixed number of key indices
 * per query, 2048 for its DSv3.2 configurations, without saying how they are
 * chosen).  The plainest reading, written out: among the columns of row r's
 * window [win_start[r], win_end[r]), rank by score, larger first, equal
 * scores (+0 and -0 are equal) by smaller column first, NaN after every
 * number; the first k ranked columns are the selection.  It is listed in
 * rank order (by_column = 0) or by ascending column (by_column = 1).  Rows
 * with fewer than k window columns fill the rest with column -1 and score
 * -inf.  The sorts are the C library's qsort.
 *
 * vals: [n_rows, ld] fp32 scores (bf16 scores widened exactly by the caller).
 * Out: idx [n_rows, k] int32, val [n_rows, k] fp32.  Returns 0, -1 on
 * allocation failure.
 */
typedef struct {
  float v;
  int32_t j;
} or_cand;

static int or_rank(const void* pa, const void* pb) {
  const or_cand* a = (const or_cand*)pa;
  const or_cand* b = (const or_cand*)pb;
  const int an = isnan(a->v) != 0, bn = isnan(b->v) != 0;
  if (an != bn) return an ? 1 : -1;  /* NaN after every number */
  if (!an) {
    if (a->v > b->v) return -1;      /* larger score first */
    if (a->v < b->v) return 1;
  }
  return (a->j > b->j) - (a->j < b->j);  /* equal scores: smaller column first */
}

static int or_by_column(const void* pa, const void* pb) {
  const or_cand* a = (const or_cand*)pa;
  const or_cand* b = (const or_cand*)pb;
  return (a->j > b->j) - (a->j < b->j);
}

int oracle_topk(int64_t n_rows, int S_k, const float* vals, int64_t ld, const int32_t* win_start,
                const int32_t* win_end, int k, int by_column, int32_t* idx, float* val) {
  or_cand* c = (or_cand*)malloc(sizeof(or_cand) * (size_t)(S_k > 0 ? S_k : 1));
  if (!c) return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    int32_t s = win_start[r], e = win_end[r];
    int n = 0;
    for (int32_t j = s; j < e; ++j) {
      c[n].v = vals[r * ld + j];
      c[n].j = j;
      ++n;
    }
    qsort(c, (size_t)n, sizeof(or_cand), or_rank);
    if (by_column) qsort(c, (size_t)(n < k ? n : k), sizeof(or_cand), or_by_column);
    for (int t = 0; t < k; ++t) {
      if (t < n) {
        idx[r * k + t] = c[t].j;
        val[r * k + t] = c[t].v;
      } else {
        idx[r * k + t] = -1;
        val[r * k + t] = -INFINITY;
      }
    }
  }
  free(c);
  return 0;
}
