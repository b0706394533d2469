/*
 * dsa_oracle.c -- plain, slow CPU oracle for the DeepSeek-Sparse-Attention
 * (DSA) hot path.  TEST INFRASTRUCTURE ONLY: it is built and called by the
 * test suite, the smoke check and the bench's CPU-baseline leg, never by the
 * product path.  It shares no code, header or table with the HIP library.
 *
 * Everything is computed in double precision with explicit loops, in the
 * order the definitions are written:
 *
 *  1. Lightning-indexer scores (the DSA indexer named in lmdeploy PR 4737
 *     "feat: support GLM-5.2", section "Changes", and in mlx-lm PR 1419's
 *     description as the MLA + DSA "lightning indexer"; the pages name it
 *     without a formula, so the formula is the plain one
 *         score[t,s] = sum_h w[t,h] * max(0, sum_d qI[t,h,d] * kI[s,d])
 *     for every cached token s <= pos(t)).
 *  2. Per-row top-k: a full sort of (score, s) pairs, higher score first and
 *     lower s on ties; when pos(t)+1 <= K every valid token is kept (mstar
 *     PR 387, section "Body", and the mlx-lm PR 1419 description both state
 *     that a context no longer than index_topk makes the sparse path the
 *     same as dense attention over every token).  Selected positions are emitted in ascending
 *     order and the row is padded with -1 (negative entries are invalid,
 *     lmdeploy PR 4968 "add glm5.3-flash support", commit notes on padding
 *     sparse FlashMLA indices with invalid entries).
 *  3. Sparse weight-absorbed MLA: for each query row and head, a dense
 *     softmax over the selected latent rows only; K is the whole
 *     [latent || rope] row and V its latent part, and the value
 *     up-projection happens after attention (mlx-lm PR 1419, the commit that
 *     extends the single-token gather path to small L; mstar PR 387 section
 *     "Tests" checks absorbed against dense MLA).  Rows are
 *     read through the per-request page table (zero-copy paged view,
 *     lmdeploy PR 4737 section "Five-layer ablations").
 *  4. OCP OFP8 E4M3 decoding of block-scaled fp8 latent rows (the BF16/FP8
 *     sparse cache paths of lmdeploy PR 4737, section "Changes"); the
 *     decoder follows the OCP 8-bit floating point specification.
 *  6. Affine 8-bit latent rows (the int8 MLA latent cache of mlx-lm PR 1419's
 *     description: only the latent is quantised, and dequantised on read):
 *     dim d of the latent is scale[d/128] * code + bias[d/128] with code an
 *     unsigned byte; the rope part stays bf16.
 *  5. Indexer query/key preparation before the scores (the fused indexer
 *     preparation of lmdeploy PR 4737, section "Changes"; mlx-lm PR 1419's
 *     description: GLM-5.2's indexer uses non-interleaved RoPE and a key
 *     LayerNorm with eps 1e-6, DeepSeek-V3.2 the interleaved form and 1e-5).
 *     Each new row's query heads are rotated at the row's position, its key
 *     is layer-normalised and rotated, and the key is written into the paged
 *     pool at that position.
 *
 * Batch convention: request b owns query rows cu_q[b] .. cu_q[b+1]-1; the
 * j-th of them sits at position pos = seq_len[b] - q_len[b] + j and sees the
 * cached tokens 0..pos (draft tokens are causal inside the draft).
 * Logical token s of request b lives at page page_table[b*pt_stride + s/P],
 * slot s%P.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_NOT_FINITE 2
#define ORC_BAD_PAGE 3

/* ---- batch helpers ---------------------------------------------------- */

/* Find the request that owns query row t, and that row's position. */
static int row_info(int B, const int32_t *cu_q, const int32_t *seq_lens, int t,
                    int *b_out, int64_t *pos_out) {
  for (int b = 0; b < B; ++b) {
    if (t >= cu_q[b] && t < cu_q[b + 1]) {
      int q_len = cu_q[b + 1] - cu_q[b];
      *b_out = b;
      *pos_out = (int64_t)seq_lens[b] - q_len + (t - cu_q[b]);
      return ORC_OK;
    }
  }
  return ORC_BAD_ARG;
}

/* Physical slot of logical token s of request b, or -1 when unmapped. */
static int64_t token_slot(const int32_t *page_table, int pt_stride, int page_size,
                          int num_pages, int b, int64_t s) {
  if (s < 0) return -1;
  int64_t lp = s / page_size;
  if (lp >= pt_stride) return -1;
  int32_t page = page_table[(int64_t)b * pt_stride + lp];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + s % page_size;
}

/* ---- number formats ---------------------------------------------------- */

/* OCP OFP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN and
 * there are no infinities.  Largest finite value 448. */
double oracle_e4m3_to_double(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int expo = (byte >> 3) & 0xF;
  int mant = byte & 0x7;
  double mag;
  if (expo == 0xF && mant == 0x7) return NAN;
  if (expo == 0)
    mag = ldexp((double)mant / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);
  return sign ? -mag : mag;
}

/* The e4m3fn code nearest to x, ties to the even code (the one whose
 * mantissa field is even).  Magnitudes past 448, the largest finite value,
 * give 448; NaN gives the NaN code.  The e4m3fn values of one binade
 * [2^E, 2^(E+1)), E >= -6, are spaced 2^(E-3); below 2^-6 (subnormals) the
 * spacing is 2^-9. */
uint8_t oracle_e4m3_encode(double x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= 448.0) return sign | 0x7E;
  int k;
  frexp(a, &k);            /* a = m * 2^k, m in [0.5, 1): binade E = k - 1 */
  int E = k - 1;
  if (E < -6) E = -6;      /* subnormals share the spacing of the lowest binade */
  const double quantum = ldexp(1.0, E - 3);
  const double units = a / quantum; /* exact: quantum is a power of two */
  double n = floor(units);
  const double frac = units - n;
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
  /* n quanta of 2^(E-3): 8 <= n <= 16 in a normal binade, 0 <= n <= 8 below */
  int expo, mant;
  if (k - 1 < -6) {        /* subnormal range: n in [0, 8]; n == 8 is 2^-6 */
    if (n >= 8.0) { expo = 1; mant = 0; }
    else { expo = 0; mant = (int)n; }
  } else if (n >= 16.0) {  /* rounded up into the next binade */
    expo = E + 7 + 1; mant = 0;
  } else {
    expo = E + 7; mant = (int)n - 8;
  }
  if (expo > 15 || (expo == 15 && mant == 7)) { expo = 15; mant = 6; }
  if (n == 0.0) return sign;
  return (uint8_t)(sign | (expo << 3) | mant);
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Decode one 656-byte fp8 latent row into `dst` (dc + dr doubles):
 * bytes 0..511 e4m3 latent, bytes 512..527 four little-endian f32 block
 * scales (block i covers latent dims 128*i .. 128*i+127), bytes 528..655
 * the 64-wide rope part in bf16. */
static void decode_fp8_row(const uint8_t *row, int dc, int dr, double *dst) {
  float scales[4];
  memcpy(scales, row + 512, sizeof scales);
  for (int d = 0; d < dc; ++d) dst[d] = oracle_e4m3_to_double(row[d]) * (double)scales[d / 128];
  for (int d = 0; d < dr; ++d) {
    uint16_t bits;
    memcpy(&bits, row + 528 + 2 * d, 2);
    dst[dc + d] = bf16_bits_to_double(bits);
  }
}

/* Affine int8 latent row (672 bytes for Dc = 512, Dr = 64): Dc unsigned codes,
 * Dc/128 f32 scales, Dc/128 f32 biases, then Dr bf16 rope values;
 * latent dim d = scale[d/128] * code[d] + bias[d/128]. */
static void decode_int8_row(const uint8_t *row, int dc, int dr, double *dst) {
  const int nb = dc / 128;
  for (int d = 0; d < dc; ++d) {
    float scale, bias;
    memcpy(&scale, row + dc + 4 * (d / 128), sizeof scale);
    memcpy(&bias, row + dc + 4 * nb + 4 * (d / 128), sizeof bias);
    dst[d] = (double)scale * (double)row[d] + (double)bias;
  }
  for (int d = 0; d < dr; ++d) {
    uint16_t bits;
    memcpy(&bits, row + dc + 8 * nb + 2 * d, sizeof bits);
    dst[dc + d] = bf16_bits_to_double(bits);
  }
}

/* ---- 1. indexer scores --------------------------------------------------- */

/*
 * Row i of the call is query row rows[i] of the batch (row i itself when
 * rows == NULL).  Per-row inputs are compact over the call's rows:
 * q_idx [n_rows, Hi, Di], w [n_rows, Hi]; k_pool [num_pages * P, Di] (doubles).
 * Writes scores[i*ld + s] for s = 0..pos; entries beyond pos are left untouched.
 */
int oracle_index_scores(int B, const int32_t *cu_q, const int32_t *seq_lens,
                        const int32_t *page_table, int pt_stride, int page_size, int num_pages,
                        const double *q_idx, const double *w, const double *k_pool,
                        int Hi, int Di, const int32_t *rows, int n_rows,
                        double *scores, int64_t ld) {
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : status)
  for (int i = 0; i < n_rows; ++i) {
    int t = rows ? rows[i] : i;
    int b;
    int64_t pos;
    if (row_info(B, cu_q, seq_lens, t, &b, &pos) != ORC_OK || pos + 1 > ld) {
      status = ORC_BAD_ARG;
      continue;
    }
    const double *qt = q_idx + (int64_t)i * Hi * Di;
    const double *wt = w + (int64_t)i * Hi;
    for (int64_t s = 0; s <= pos; ++s) {
      int64_t slot = token_slot(page_table, pt_stride, page_size, num_pages, b, s);
      if (slot < 0) {
        status = ORC_BAD_PAGE;
        break;
      }
      const double *k = k_pool + slot * Di;
      double acc = 0.0;
      for (int h = 0; h < Hi; ++h) {
        double dot = 0.0;
        for (int d = 0; d < Di; ++d) dot += qt[(int64_t)h * Di + d] * k[d];
        double relu = dot > 0.0 ? dot : 0.0;
        acc += wt[h] * relu;
      }
      scores[(int64_t)i * ld + s] = acc;
    }
  }
  return status;
}

/* ---- 2. top-k --------------------------------------------------------------- */

typedef struct {
  double score;
  int64_t s;
} scored_token;

/* Higher score first; equal scores (including -0.0 == +0.0) by lower s. */
static int by_score_desc_then_pos(const void *a, const void *b) {
  const scored_token *x = (const scored_token *)a, *y = (const scored_token *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int by_int_asc(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/*
 * scores [n_rows, ld] holds each listed row's scores (row i is query row
 * rows[i], or i when rows == NULL).  Writes idx [n_rows, K].
 */
int oracle_topk(int B, const int32_t *cu_q, const int32_t *seq_lens,
                const double *scores, int64_t ld, int K, const int32_t *rows, int n_rows,
                int32_t *idx) {
  if (K <= 0) return ORC_BAD_ARG;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : status)
  for (int i = 0; i < n_rows; ++i) {
    int t = rows ? rows[i] : i;
    int b;
    int64_t pos;
    int32_t *out = idx + (int64_t)i * K;
    if (row_info(B, cu_q, seq_lens, t, &b, &pos) != ORC_OK || pos + 1 > ld) {
      status = ORC_BAD_ARG;
      continue;
    }
    int64_t n = pos + 1;
    int64_t keep = n < K ? n : K;
    if (n <= K) {
      for (int64_t j = 0; j < n; ++j) out[j] = (int32_t)j;
    } else {
      scored_token *all = (scored_token *)malloc((size_t)n * sizeof *all);
      int finite = 1;
      for (int64_t s = 0; s < n; ++s) {
        all[s].score = scores[(int64_t)i * ld + s];
        all[s].s = s;
        if (!isfinite(all[s].score)) finite = 0;
      }
      if (!finite) status = ORC_NOT_FINITE;
      qsort(all, (size_t)n, sizeof *all, by_score_desc_then_pos);
      for (int64_t j = 0; j < K; ++j) out[j] = (int32_t)all[j].s;
      free(all);
      qsort(out, (size_t)K, sizeof *out, by_int_asc);
    }
    for (int64_t j = keep; j < K; ++j) out[j] = -1;
  }
  return status;
}

/* ---- 3. sparse absorbed MLA ------------------------------------------------- */

/*
 * Per-row inputs are compact over the call's rows (row i is query row
 * rows[i]): q [n_rows, H, Dc+Dr] doubles, idx [n_rows, K] logical positions.
 * kv: when kv_fmt == 0, doubles [num_pages*P, Dc+Dr]; kv_fmt == 1, raw fp8
 * 656-byte rows [num_pages*P, 656]; kv_fmt == 2, raw affine int8 672-byte rows.  An entry is used when 0 <= s <= pos(t) and its
 * page is mapped; others are skipped (re-masked).  Rows are accumulated in
 * ascending j.  out [n_rows, H, Dc], lse [n_rows, H] (natural log).  A row with
 * no usable entry gives out = 0 and lse = -inf.
 */
int oracle_sparse_mla(int B, const int32_t *cu_q, const int32_t *seq_lens,
                      const int32_t *page_table, int pt_stride, int page_size, int num_pages,
                      const double *q, int kv_fmt, const void *kv, const int32_t *idx, int K,
                      int H, int Dc, int Dr, double scale, const int32_t *rows, int n_rows,
                      double *out, double *lse) {
  const int D = Dc + Dr;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : status)
  for (int i = 0; i < n_rows; ++i) {
    int t = rows ? rows[i] : i;
    int b;
    int64_t pos;
    if (row_info(B, cu_q, seq_lens, t, &b, &pos) != ORC_OK) {
      status = ORC_BAD_ARG;
      continue;
    }
    /* gather the usable rows once (decoded to double) */
    double *rowbuf = (double *)malloc((size_t)K * D * sizeof(double));
    double *logit = (double *)malloc((size_t)K * sizeof(double));
    int n_used = 0;
    for (int j = 0; j < K; ++j) {
      int64_t s = idx[(int64_t)i * K + j];
      if (s < 0 || s > pos) continue;
      int64_t slot = token_slot(page_table, pt_stride, page_size, num_pages, b, s);
      if (slot < 0) continue;
      double *dst = rowbuf + (int64_t)n_used * D;
      if (kv_fmt == 1)
        decode_fp8_row((const uint8_t *)kv + slot * 656, Dc, Dr, dst);
      else if (kv_fmt == 2)
        decode_int8_row((const uint8_t *)kv + slot * (Dc + 8 * (Dc / 128) + 2 * Dr), Dc, Dr, dst);
      else
        memcpy(dst, (const double *)kv + slot * D, (size_t)D * sizeof(double));
      ++n_used;
    }
    for (int h = 0; h < H; ++h) {
      const double *qh = q + ((int64_t)i * H + h) * D;
      double *oh = out + ((int64_t)i * H + h) * Dc;
      for (int d = 0; d < Dc; ++d) oh[d] = 0.0;
      if (n_used == 0) {
        lse[(int64_t)i * H + h] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int j = 0; j < n_used; ++j) {
        const double *r = rowbuf + (int64_t)j * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qh[d] * r[d];
        logit[j] = scale * dot;
        if (logit[j] > m) m = logit[j];
      }
      double denom = 0.0;
      for (int j = 0; j < n_used; ++j) denom += exp(logit[j] - m);
      for (int j = 0; j < n_used; ++j) {
        double p = exp(logit[j] - m) / denom;
        const double *r = rowbuf + (int64_t)j * D;
        for (int d = 0; d < Dc; ++d) oh[d] += p * r[d];
      }
      lse[(int64_t)i * H + h] = m + log(denom);
    }
    free(rowbuf);
    free(logit);
  }
  return status;
}

/* Decode a whole int8 pool [n_rows, 672] into doubles [n_rows, Dc+Dr]. */
void oracle_decode_int8_rows(const uint8_t *rows, int64_t n_rows, int Dc, int Dr, double *dst) {
  const int64_t rb = Dc + 8 * (Dc / 128) + 2 * Dr;
  for (int64_t r = 0; r < n_rows; ++r) decode_int8_row(rows + r * rb, Dc, Dr, dst + r * (Dc + Dr));
}

/* Decode a whole fp8 pool [n_rows, 656] into doubles [n_rows, Dc+Dr]. */
void oracle_decode_fp8_rows(const uint8_t *rows, int64_t n_rows, int Dc, int Dr, double *dst) {
  for (int64_t r = 0; r < n_rows; ++r) decode_fp8_row(rows + r * 656, Dc, Dr, dst + r * (Dc + Dr));
}

/* Decode a page-blocked fp8 index-key pool into `dst` ([num_pages * P, Di]
 * doubles): page p holds P rows of Di e4m3 codes (row_stride bytes apart),
 * then, at byte P * row_stride of the page, P little-endian f32 scales, one
 * per token; key value = e4m3(code) * scale. */
void oracle_decode_fp8_keys(const uint8_t *pool, int64_t num_pages, int P, int Di, int64_t row_stride,
                            int64_t page_stride, double *dst) {
  for (int64_t p = 0; p < num_pages; ++p) {
    const uint8_t *page = pool + p * page_stride;
    for (int i = 0; i < P; ++i) {
      float scale;
      memcpy(&scale, page + (int64_t)P * row_stride + 4 * i, sizeof scale);
      for (int d = 0; d < Di; ++d)
        dst[(p * P + i) * Di + d] = oracle_e4m3_to_double(page[i * row_stride + d]) * (double)scale;
    }
  }
}

/* ---- 5. indexer preparation ------------------------------------------- */

/* Rotary embedding of the first R dims of x (length D) at table row `row`:
 * pair i (0 <= i < R/2) is dims (i, i + R/2) when not interleaved and
 * (2i, 2i+1) when interleaved; it turns by the angle whose cosine and sine
 * are cos_tab[row*R/2 + i] and sin_tab[row*R/2 + i]:
 *     (a, b) -> (a cos - b sin, a sin + b cos).
 * Dims R .. D-1 pass through unchanged. */
static void rope(const double *x, double *y, int D, int R, int interleaved,
                 const double *cos_row, const double *sin_row) {
  for (int d = R; d < D; ++d) y[d] = x[d];
  for (int i = 0; i < R / 2; ++i) {
    int ia = interleaved ? 2 * i : i;
    int ib = interleaved ? 2 * i + 1 : i + R / 2;
    double a = x[ia], b = x[ib], c = cos_row[i], s = sin_row[i];
    y[ia] = a * c - b * s;
    y[ib] = a * s + b * c;
  }
}

/* LayerNorm over D values: (x - mean) / sqrt(var + eps) * gamma + beta, with
 * var the mean squared deviation (population variance). */
static void layer_norm(const double *x, double *y, int D, const double *gamma,
                       const double *beta, double eps) {
  double mean = 0.0, var = 0.0;
  for (int d = 0; d < D; ++d) mean += x[d];
  mean /= D;
  for (int d = 0; d < D; ++d) var += (x[d] - mean) * (x[d] - mean);
  var /= D;
  double inv = 1.0 / sqrt(var + eps);
  for (int d = 0; d < D; ++d) y[d] = (x[d] - mean) * inv * gamma[d] + beta[d];
}

/* For every query row t (position p = pos(t)):
 *   q_out[t,h,:] = rope(q_in[t,h,:], p)          for each of the H heads
 *   k_out[t,:]   = rope(layer_norm(k_in[t,:]), p)
 * and, when pool != NULL, k_out[t,:] is stored at the row's token slot of
 * the pool image ([num_pages*P, D], page table applied; rows whose page is
 * not mapped are not stored).  pos_out[t] receives p.  Returns ORC_BAD_ARG
 * when a position falls outside the rope table. */
int oracle_indexer_prepare(int B, const int32_t *cu_q, const int32_t *seq_lens,
                           const int32_t *page_table, int pt_stride, int page_size, int num_pages,
                           int T, const double *q_in, const double *k_in, const double *gamma,
                           const double *beta, double eps, const double *cos_tab,
                           const double *sin_tab, int64_t tab_rows, int R, int interleaved,
                           int H, int D, double *q_out, double *k_out, double *pool,
                           int64_t *pos_out) {
  if (R < 0 || R > D || R % 2 != 0) return ORC_BAD_ARG;
  double *kn = (double *)malloc(sizeof(double) * (size_t)D);
  if (!kn) return ORC_BAD_ARG;
  int st = ORC_OK;
  for (int t = 0; t < T && st == ORC_OK; ++t) {
    int b;
    int64_t p;
    if (row_info(B, cu_q, seq_lens, t, &b, &p) != ORC_OK || p < 0 || p >= tab_rows) {
      st = ORC_BAD_ARG;
      break;
    }
    pos_out[t] = p;
    const double *c = cos_tab + p * (R / 2), *s = sin_tab + p * (R / 2);
    for (int h = 0; h < H; ++h)
      rope(q_in + ((int64_t)t * H + h) * D, q_out + ((int64_t)t * H + h) * D, D, R, interleaved, c, s);
    layer_norm(k_in + (int64_t)t * D, kn, D, gamma, beta, eps);
    rope(kn, k_out + (int64_t)t * D, D, R, interleaved, c, s);
    if (pool) {
      int64_t slot = token_slot(page_table, pt_stride, page_size, num_pages, b, p);
      if (slot >= 0) memcpy(pool + slot * D, k_out + (int64_t)t * D, sizeof(double) * (size_t)D);
    }
  }
  free(kn);
  return st;
}

/* Threads the OpenMP loops above use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the thread count of the loops above (no effect without OpenMP). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
