/*
 * Plain CPU oracle for top-k sparse decode attention (C11, double precision).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product library. It shares no
 * code with the HIP path.
 *
 * Sources, by the title of each page and its section:
 *  - "QSA HiSparse -- SGLang plugin", Supported versions / Run: the KV cache
 *    is FP8 E4M3 in 64-token pages.
 *  - "QSA cache sharding" (sglang PR #43527), Implementation: pages of a
 *    request are reached through the request-to-token mapping; token
 *    selection is an exact Top-K with deterministic token-ID tie-breaking;
 *    sparse attention runs over the selected tokens and partial outputs are
 *    combined by an FP32 log-sum-exp merge.
 *  - "Context parallelism for QSA attention and the sparse indexer" (sglang
 *    PR #39721), Motivation: the indexer scores index keys and selects top-k
 *    per query row; sparse GQA attention runs over the selected tokens.
 *  - "Support double sparsity" (sglang PR #1459), Speedup Evaluation and the
 *    forward_extend traceback in the discussion: the label cache holds K at
 *    a per-head set of heavy channels; heavy-token count = top-k.
 *
 * Readings where the pages are silent (each is listed with the design
 * notes): the QSA score is sum_h w_h * max(0, q_h . k_t) with unit index-K
 * scale; the double-sparsity row is one per (request, KV head) and its query
 * is the sum of the group's query heads at the heavy channels; FP8 is the
 * OCP E4M3 "FN" encoding with one f32 scale per physical page; ties go to
 * the lower logical token index; results are listed in ascending index
 * order padded with -1; chunk c of m selected tokens is the contiguous range
 * [floor(c*m/C), floor((c+1)*m/C)).
 */
#include "tsd_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decoders */

/* OCP 8-bit floating point, E4M3 variant: sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 is subnormal (2^-6 * m/8); the
 * all-ones exponent with all-ones mantissa is the only NaN; no infinities.
 * Largest finite magnitude 448 = 2^8 * 1.75. */
double tsd_oracle_decode_fp8e4m3(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32 value. */
double tsd_oracle_decode_bf16(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* IEEE binary16: sign, 5 exponent bits with bias 15, 10 mantissa bits. */
double tsd_oracle_decode_fp16(uint16_t bits) {
  int s = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1F;
  int m = bits & 0x3FF;
  double mag;
  if (e == 0x1F) mag = m ? NAN : INFINITY;
  else if (e == 0) mag = ldexp((double)m / 1024.0, -14);
  else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -mag : mag;
}

/* The 256 FP8 values, tabulated once from the decoder above so that large
 * scans do not call ldexp per element. */
static double fp8_table[256];

/* Filled when the library is loaded, before any call, so that calls from
 * several threads only read it. */
__attribute__((constructor)) static void fp8_table_fill(void) {
  for (int c = 0; c < 256; ++c)
    fp8_table[c] = tsd_oracle_decode_fp8e4m3((uint8_t)c);
}

static double fp8(uint8_t code) { return fp8_table[code]; }

static double decode_elem(const void *base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_BF16: return tsd_oracle_decode_bf16(((const uint16_t *)base)[i]);
    case ORC_FP16: return tsd_oracle_decode_fp16(((const uint16_t *)base)[i]);
    case ORC_FP8E4M3: return fp8(((const uint8_t *)base)[i]);
    case ORC_F32: return (double)((const float *)base)[i];
    default: return NAN;
  }
}

static int dtype_ok(int dtype) {
  return dtype == ORC_BF16 || dtype == ORC_FP16 || dtype == ORC_FP8E4M3 ||
         dtype == ORC_F32;
}

/* ------------------------------------------------------------ slot mapping */

/* Logical token t of request b lives in page page_table[b][t / page_size],
 * at offset t % page_size. */
int64_t tsd_oracle_slot(const int32_t *page_table, int64_t pt_stride, int b,
                        int64_t t, int page_size, int64_t num_pages) {
  int64_t page = page_table[(int64_t)b * pt_stride + t / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return page * page_size + t % page_size;
}

/* ------------------------------------------------------------------ scores */

/* Double-sparsity query of row (b, g): the group's query heads summed at the
 * heavy channels chan[g, 0 .. r). */
static void ds_row_query(int b, int g, int H_q, int G, int D, int r,
                         const void *q, int q_dtype, const int32_t *chan,
                         double *qs) {
  for (int j = 0; j < r; ++j) {
    int c = chan[g * r + j];
    double acc = 0.0;
    for (int h = g * G; h < (g + 1) * G; ++h)
      acc += decode_elem(q, q_dtype, ((int64_t)b * H_q + h) * D + c);
    qs[j] = acc;
  }
}

/* Label score of one token slot for KV head g. */
static double ds_point(const double *qs, int r, int H_kv, int g,
                       const void *label, int label_dtype, int64_t slot) {
  double acc = 0.0;
  for (int j = 0; j < r; ++j)
    acc += qs[j] * decode_elem(label, label_dtype, (slot * H_kv + g) * r + j);
  return acc;
}

static int ds_args_ok(int B, int H_q, int H_kv, int D, int r, int q_dtype,
                      int label_dtype, int page_size) {
  return B >= 0 && H_q > 0 && H_kv > 0 && H_q % H_kv == 0 && D > 0 && r > 0 &&
         page_size > 0 && dtype_ok(q_dtype) && dtype_ok(label_dtype);
}

int tsd_oracle_ds_scores(int B, int H_q, int H_kv, int D, int r,
                         const void *q, int q_dtype, const int32_t *chan,
                         const void *label, int label_dtype,
                         const int32_t *page_table, int64_t pt_stride,
                         const int32_t *seq_lens, int64_t num_pages,
                         int page_size, double *scores, int64_t score_stride) {
  if (!ds_args_ok(B, H_q, H_kv, D, r, q_dtype, label_dtype, page_size))
    return ORC_E_ARG;
  int G = H_q / H_kv;
  double *qs = (double *)malloc(sizeof(double) * (size_t)r);
  if (!qs) return ORC_E_ARG;
  for (int b = 0; b < B; ++b) {
    for (int g = 0; g < H_kv; ++g) {
      ds_row_query(b, g, H_q, G, D, r, q, q_dtype, chan, qs);
      double *row = scores + ((int64_t)b * H_kv + g) * score_stride;
      for (int64_t t = 0; t < seq_lens[b]; ++t) {
        int64_t slot =
            tsd_oracle_slot(page_table, pt_stride, b, t, page_size, num_pages);
        if (slot < 0) { free(qs); return ORC_E_PAGE; }
        row[t] = ds_point(qs, r, H_kv, g, label, label_dtype, slot);
      }
    }
  }
  free(qs);
  return ORC_OK;
}

int tsd_oracle_ds_score_points(int B, int H_q, int H_kv, int D, int r,
                               const void *q, int q_dtype, const int32_t *chan,
                               const void *label, int label_dtype,
                               const int32_t *page_table, int64_t pt_stride,
                               const int32_t *seq_lens, int64_t num_pages,
                               int page_size, int64_t npts,
                               const int32_t *pt_row, const int64_t *pt_t,
                               double *out) {
  if (!ds_args_ok(B, H_q, H_kv, D, r, q_dtype, label_dtype, page_size))
    return ORC_E_ARG;
  int G = H_q / H_kv;
  double *qs = (double *)malloc(sizeof(double) * (size_t)r);
  if (!qs) return ORC_E_ARG;
  for (int64_t p = 0; p < npts; ++p) {
    int row = pt_row[p];
    int b = row / H_kv, g = row % H_kv;
    if (row < 0 || b >= B || pt_t[p] < 0 || pt_t[p] >= seq_lens[b]) {
      free(qs);
      return ORC_E_INDEX;
    }
    int64_t slot = tsd_oracle_slot(page_table, pt_stride, b, pt_t[p],
                                   page_size, num_pages);
    if (slot < 0) { free(qs); return ORC_E_PAGE; }
    ds_row_query(b, g, H_q, G, D, r, q, q_dtype, chan, qs);
    out[p] = ds_point(qs, r, H_kv, g, label, label_dtype, slot);
  }
  free(qs);
  return ORC_OK;
}

/* Number of keys query row i sees: the request's length, or for a causal
 * prefill row at position p, the p + 1 keys 0 .. p (never beyond the
 * request's length). */
static int64_t qsa_row_len(int i, int R, const int32_t *seq_lens,
                           const int32_t *q_pos) {
  int64_t n = seq_lens[i / R];
  if (q_pos) {
    int64_t p1 = (int64_t)q_pos[i] + 1;
    if (p1 < 0) p1 = 0;
    if (p1 < n) n = p1;
  }
  return n < 0 ? 0 : n;
}

/* Index score of row i against the index key stored at slot:
 * sum_h w[i,h] * max(0, sum_d qi[i,h,d] * ki[slot,d]). */
static double qsa_point(int i, int H_i, int D_i, const uint8_t *index_q,
                        const float *index_w, const uint8_t *index_k,
                        int64_t slot) {
  double s = 0.0;
  for (int h = 0; h < H_i; ++h) {
    double dot = 0.0;
    for (int d = 0; d < D_i; ++d)
      dot += fp8(index_q[((int64_t)i * H_i + h) * D_i + d]) *
             fp8(index_k[slot * D_i + d]);
    if (dot > 0.0) s += (double)index_w[(int64_t)i * H_i + h] * dot;
  }
  return s;
}

int tsd_oracle_qsa_scores(int rows, int R, int H_i, int D_i,
                          const uint8_t *index_q, const float *index_w,
                          const uint8_t *index_k, const int32_t *page_table,
                          int64_t pt_stride, const int32_t *seq_lens,
                          const int32_t *q_pos, int64_t num_pages,
                          int page_size, double *scores, int64_t score_stride) {
  if (rows < 0 || R <= 0 || H_i <= 0 || D_i <= 0 || page_size <= 0)
    return ORC_E_ARG;
  for (int i = 0; i < rows; ++i) {
    int b = i / R;
    int64_t n = qsa_row_len(i, R, seq_lens, q_pos);
    double *row = scores + (int64_t)i * score_stride;
    for (int64_t t = 0; t < n; ++t) {
      int64_t slot =
          tsd_oracle_slot(page_table, pt_stride, b, t, page_size, num_pages);
      if (slot < 0) return ORC_E_PAGE;
      row[t] = qsa_point(i, H_i, D_i, index_q, index_w, index_k, slot);
    }
  }
  return ORC_OK;
}

int tsd_oracle_qsa_score_points(int rows, int R, int H_i, int D_i,
                                const uint8_t *index_q, const float *index_w,
                                const uint8_t *index_k,
                                const int32_t *page_table, int64_t pt_stride,
                                const int32_t *seq_lens, const int32_t *q_pos,
                                int64_t num_pages, int page_size, int64_t npts,
                                const int32_t *pt_row, const int64_t *pt_t,
                                double *out) {
  if (rows < 0 || R <= 0 || H_i <= 0 || D_i <= 0 || page_size <= 0)
    return ORC_E_ARG;
  for (int64_t p = 0; p < npts; ++p) {
    int i = pt_row[p];
    if (i < 0 || i >= rows || pt_t[p] < 0 ||
        pt_t[p] >= qsa_row_len(i, R, seq_lens, q_pos))
      return ORC_E_INDEX;
    int64_t slot = tsd_oracle_slot(page_table, pt_stride, i / R, pt_t[p],
                                   page_size, num_pages);
    if (slot < 0) return ORC_E_PAGE;
    out[p] = qsa_point(i, H_i, D_i, index_q, index_w, index_k, slot);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------- top-k */

typedef struct {
  float s;
  int32_t t;
} scored_t;

/* Order: larger score first; equal scores (as floats: -0 == +0) by lower
 * token index. */
static int by_score_then_index(const void *pa, const void *pb) {
  const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->t > b->t) - (a->t < b->t);
}

static int by_index(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

int tsd_oracle_topk(const float *scores, int64_t stride, int rows,
                    const int32_t *row_lens, int k, int32_t *idx,
                    int32_t *count) {
  if (rows < 0 || k <= 0) return ORC_E_ARG;
  for (int row = 0; row < rows; ++row) {
    int64_t n = row_lens[row] > 0 ? row_lens[row] : 0;
    int32_t *out = idx + (int64_t)row * k;
    scored_t *all = (scored_t *)malloc(sizeof(scored_t) * (size_t)(n ? n : 1));
    if (!all) return ORC_E_ARG;
    for (int64_t t = 0; t < n; ++t) {
      all[t].s = scores[(int64_t)row * stride + t];
      all[t].t = (int32_t)t;
      if (isnan(all[t].s)) { free(all); return ORC_E_NAN; }
    }
    qsort(all, (size_t)n, sizeof(scored_t), by_score_then_index);
    int64_t m = n < k ? n : k;
    for (int64_t j = 0; j < m; ++j) out[j] = all[j].t;
    qsort(out, (size_t)m, sizeof(int32_t), by_index);
    for (int64_t j = m; j < k; ++j) out[j] = -1;
    if (count) count[row] = (int32_t)m;
    free(all);
  }
  return ORC_OK;
}

int tsd_oracle_topk_merge_sharded(const float *scores, int64_t stride,
                                  const int32_t *idx, const int32_t *count,
                                  int W, int rows, int kl, int page_size,
                                  int k, int32_t *out_idx,
                                  int32_t *out_count) {
  if (W < 1 || rows < 0 || kl < 0 || k <= 0 || page_size < 1) return ORC_E_ARG;
  scored_t *all = (scored_t *)malloc(sizeof(scored_t) * (size_t)(W * kl + 1));
  if (!all) return ORC_E_ARG;
  for (int row = 0; row < rows; ++row) {
    int64_t n = 0;
    for (int w = 0; w < W; ++w) {
      const int64_t sr = (int64_t)w * rows + row;
      int32_t c = count[sr];
      if (c > kl) c = kl;
      for (int32_t j = 0; j < c; ++j) {
        const int32_t u = idx[sr * kl + j];
        if (u < 0) continue;
        const float sc = scores[sr * stride + u];
        if (isnan(sc)) { free(all); return ORC_E_NAN; }
        all[n].s = sc;
        all[n].t = (int32_t)(((int64_t)(u / page_size) * W + w) * page_size +
                             u % page_size);
        ++n;
      }
    }
    qsort(all, (size_t)n, sizeof(scored_t), by_score_then_index);
    const int64_t m = n < k ? n : k;
    int32_t *out = out_idx + (int64_t)row * k;
    for (int64_t j = 0; j < m; ++j) out[j] = all[j].t;
    qsort(out, (size_t)m, sizeof(int32_t), by_index);
    for (int64_t j = m; j < k; ++j) out[j] = -1;
    if (out_count) out_count[row] = (int32_t)m;
  }
  free(all);
  return ORC_OK;
}

/* ------------------------------------------------------------ cache append */

uint8_t tsd_oracle_encode_fp8e4m3(double x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {  /* every finite non-negative code */
    const double err = fabs(a - tsd_oracle_decode_fp8e4m3((uint8_t)c));
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  if (a >= 448.0) best = 0x7E;
  return (uint8_t)(sign | best);
}

/* f32 value of element i of a 16-bit array, or of an f32 array (dtype 4). */
static float half_or_f32(const void *base, int dtype, int64_t i) {
  if (dtype == 4) return ((const float *)base)[i];
  return (float)decode_elem(base, dtype, i);
}

int tsd_oracle_kv_append(int B, int64_t pt_stride, const int32_t *page_table,
                         int64_t num_pages, int page_size,
                         const int32_t *positions, const int32_t *n_new,
                         int max_new, int H_kv, int D, const void *k_new,
                         const void *v_new, int new_dtype, void *k_pool,
                         void *v_pool, int kv_dtype, float *k_scale,
                         float *v_scale, const int32_t *channel_idx, int r,
                         void *label_pool, const void *index_k_new,
                         int index_dtype, void *index_k_pool, int D_i) {
  if (B < 0 || max_new < 0 || page_size < 1) return ORC_E_ARG;
  const int fp8 = kv_dtype == ORC_FP8E4M3;
  if (k_pool && (new_dtype != ORC_BF16 && new_dtype != ORC_FP16)) return ORC_E_ARG;
  if (k_pool && !fp8 && kv_dtype != new_dtype) return ORC_E_ARG;
  if (k_pool && fp8 && (!k_scale || !v_scale)) return ORC_E_ARG;
  const int64_t row = (int64_t)H_kv * D;
  for (int b = 0; b < B; ++b) {
    int32_t n = n_new[b] < 0 ? 0 : n_new[b];
    if (n > max_new) n = max_new;
    const int64_t pos = positions[b];
    /* page scales of the pages this call starts, from the values it writes */
    if (k_pool && fp8) {
      for (int32_t i = 0; i < n; ++i) {
        const int64_t t = pos + i;
        if (t < 0 || t >= pt_stride * page_size) continue;
        const int64_t lp = t / page_size;
        const int32_t page = page_table[(int64_t)b * pt_stride + lp];
        if (page < 0 || page >= num_pages) continue;
        if (lp * page_size < pos) continue;  /* page began before this call */
        if (t != lp * page_size && i != 0) continue;  /* once per page */
        float ka = 0.f, va = 0.f;
        int32_t written = 0;
        for (int32_t i2 = i; i2 < n && (pos + i2) / page_size == lp; ++i2) {
          ++written;
          for (int64_t e = 0; e < row; ++e) {
            const int64_t at = ((int64_t)b * max_new + i2) * row + e;
            const float kv = fabsf(half_or_f32(k_new, new_dtype, at));
            const float vv = fabsf(half_or_f32(v_new, new_dtype, at));
            if (kv > ka) ka = kv;
            if (vv > va) va = vv;
          }
        }
        /* a page the call does not fill gets 4x the range of its values:
         * two binades for the tokens later calls append to it */
        const float room = written == page_size ? 1.0f : 4.0f;
        k_scale[page] = ka > 0.f ? ka / 448.0f * room : 1.0f;
        v_scale[page] = va > 0.f ? va / 448.0f * room : 1.0f;
      }
    }
    for (int32_t i = 0; i < n; ++i) {
      const int64_t t = pos + i;
      if (t < 0 || t >= pt_stride * page_size) continue;
      const int32_t page = page_table[(int64_t)b * pt_stride + t / page_size];
      if (page < 0 || page >= num_pages) continue;
      const int64_t slot = (int64_t)page * page_size + t % page_size;
      const int64_t src = ((int64_t)b * max_new + i) * row;
      if (k_pool) {
        for (int64_t e = 0; e < row; ++e) {
          if (fp8) {
            const float kq = half_or_f32(k_new, new_dtype, src + e) / k_scale[page];
            const float vq = half_or_f32(v_new, new_dtype, src + e) / v_scale[page];
            ((uint8_t *)k_pool)[slot * row + e] = tsd_oracle_encode_fp8e4m3(kq);
            ((uint8_t *)v_pool)[slot * row + e] = tsd_oracle_encode_fp8e4m3(vq);
          } else {
            ((uint16_t *)k_pool)[slot * row + e] = ((const uint16_t *)k_new)[src + e];
            ((uint16_t *)v_pool)[slot * row + e] = ((const uint16_t *)v_new)[src + e];
          }
        }
      }
      if (label_pool) {
        for (int g = 0; g < H_kv; ++g)
          for (int j = 0; j < r; ++j) {
            const int32_t ch = channel_idx[g * r + j];
            ((uint16_t *)label_pool)[(slot * H_kv + g) * r + j] =
                ch >= 0 && ch < D
                    ? ((const uint16_t *)k_new)[src + (int64_t)g * D + ch]
                    : 0; /* a channel outside [0, D) stores 0 */
          }
      }
      if (index_k_pool) {
        const int64_t isrc = ((int64_t)b * max_new + i) * D_i;
        for (int d = 0; d < D_i; ++d)
          ((uint8_t *)index_k_pool)[slot * D_i + d] = tsd_oracle_encode_fp8e4m3(
              half_or_f32(index_k_new, index_dtype, isrc + d));
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------ block compression */

int tsd_oracle_index_k_compress(int B, int Bs, const uint8_t *index_k_pool,
                                const int32_t *page_table, int64_t pt_stride,
                                int64_t num_pages, const int32_t *seq_lens,
                                const int32_t *from_block,
                                const int32_t *cpage_table, int64_t cpt_stride,
                                int64_t num_cpages, int page_size, int D_i,
                                uint8_t *ck_pool) {
  if (B < 0 || Bs < 1 || page_size < 1 || D_i < 1) return ORC_E_ARG;
  double *acc = (double *)malloc(sizeof(double) * (size_t)D_i);
  if (!acc) return ORC_E_ARG;
  for (int b = 0; b < B; ++b) {
    int64_t n = seq_lens[b] < 0 ? 0 : seq_lens[b];
    if (n > pt_stride * page_size) n = pt_stride * page_size;
    const int64_t nblk = (n + Bs - 1) / Bs;
    for (int64_t j = from_block[b] < 0 ? 0 : from_block[b]; j < nblk; ++j) {
      if (j >= cpt_stride * page_size) break;
      const int32_t cpage = cpage_table[(int64_t)b * cpt_stride + j / page_size];
      if (cpage < 0 || cpage >= num_cpages) continue;
      const int64_t t0 = j * Bs, t1 = (j + 1) * Bs < n ? (j + 1) * Bs : n;
      int ok = 1;
      for (int d = 0; d < D_i; ++d) acc[d] = 0.0;
      for (int64_t t = t0; t < t1 && ok; ++t) {
        const int32_t page = page_table[(int64_t)b * pt_stride + t / page_size];
        if (page < 0 || page >= num_pages) { ok = 0; break; }
        const int64_t slot = (int64_t)page * page_size + t % page_size;
        for (int d = 0; d < D_i; ++d)
          acc[d] += tsd_oracle_decode_fp8e4m3(index_k_pool[slot * D_i + d]);
      }
      if (!ok) continue;
      const int64_t cslot = (int64_t)cpage * page_size + j % page_size;
      for (int d = 0; d < D_i; ++d) {
        const float mean = (float)(acc[d] / (double)(t1 - t0));
        ck_pool[cslot * D_i + d] = tsd_oracle_encode_fp8e4m3(mean);
      }
    }
  }
  free(acc);
  return ORC_OK;
}

int tsd_oracle_expand_blocks(int rows, const int32_t *sel, const int32_t *count,
                             int kb, int Bs, const int32_t *row_lens, int kt,
                             int32_t *tok, int32_t *tok_count) {
  if (rows < 0 || kb < 1 || Bs < 1 || kt < 1) return ORC_E_ARG;
  for (int row = 0; row < rows; ++row) {
    const int64_t n = row_lens[row] < 0 ? 0 : row_lens[row];
    int32_t c = count[row] < 0 ? 0 : count[row];
    if (c > kb) c = kb;
    int64_t m = 0;
    for (int32_t i = 0; i < c; ++i) {
      const int64_t j = sel[(int64_t)row * kb + i];
      if (j < 0) continue;
      for (int64_t t = j * Bs; t < (j + 1) * Bs && t < n && m < kt; ++t)
        tok[(int64_t)row * kt + m++] = (int32_t)t;
    }
    for (int64_t i = m; i < kt; ++i) tok[(int64_t)row * kt + i] = -1;
    if (tok_count) tok_count[row] = (int32_t)m;
  }
  return ORC_OK;
}

/* --------------------------------------------------------------- attention */

/* Dequantised element d of token slot, KV head g. */
static double kv_elem(const void *pool, int dtype, const float *scale,
                      int64_t slot, int page_size, int H_kv, int D, int g,
                      int d) {
  double v = decode_elem(pool, dtype, (slot * H_kv + g) * D + d);
  if (dtype == ORC_FP8E4M3) v *= (double)scale[slot / page_size];
  return v;
}

int tsd_oracle_sparse_attention(int B, int H_q, int H_kv, int D, int H_sel,
                                int k, int C, const void *q, int q_dtype,
                                const void *k_pool, const void *v_pool,
                                int kv_dtype, const float *k_scale,
                                const float *v_scale,
                                const int32_t *page_table, int64_t pt_stride,
                                const int32_t *seq_lens, int64_t num_pages,
                                int page_size, const int32_t *idx,
                                const int32_t *count, double softmax_scale,
                                double *o_part, double *lse_part) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 || D <= 0 ||
      k <= 0 || C <= 0 || !(H_sel == 1 || H_sel == H_kv) ||
      !dtype_ok(q_dtype) || !dtype_ok(kv_dtype) || page_size <= 0)
    return ORC_E_ARG;
  if (kv_dtype == ORC_FP8E4M3 && (!k_scale || !v_scale)) return ORC_E_ARG;
  int G = H_q / H_kv;
  double *z = (double *)malloc(sizeof(double) * (size_t)k);
  int64_t *slots = (int64_t *)malloc(sizeof(int64_t) * (size_t)k);
  if (!z || !slots) { free(z); free(slots); return ORC_E_ARG; }
  int rc = ORC_OK;
  for (int b = 0; b < B && rc == ORC_OK; ++b) {
    for (int h = 0; h < H_q && rc == ORC_OK; ++h) {
      int g = h / G;
      int sel_row = (H_sel == 1) ? 0 : g;
      const int32_t *sel = idx + ((int64_t)b * H_sel + sel_row) * k;
      int64_t m = count[(int64_t)b * H_sel + sel_row];
      if (m < 0) m = 0;
      if (m > k) m = k;
      for (int c = 0; c < C; ++c) {
        int64_t lo = (int64_t)c * m / C, hi = (int64_t)(c + 1) * m / C;
        double *o = o_part + (((int64_t)b * H_q + h) * C + c) * D;
        double *lse = lse_part + ((int64_t)b * H_q + h) * C + c;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (hi <= lo) { *lse = -INFINITY; continue; }
        double zmax = -INFINITY;
        for (int64_t j = lo; j < hi; ++j) {
          int64_t t = sel[j];
          if (t < 0 || t >= seq_lens[b]) { rc = ORC_E_INDEX; break; }
          int64_t slot = tsd_oracle_slot(page_table, pt_stride, b, t,
                                         page_size, num_pages);
          if (slot < 0) { rc = ORC_E_PAGE; break; }
          slots[j - lo] = slot;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += decode_elem(q, q_dtype, ((int64_t)b * H_q + h) * D + d) *
                   kv_elem(k_pool, kv_dtype, k_scale, slot, page_size, H_kv,
                           D, g, d);
          z[j - lo] = softmax_scale * dot;
          if (z[j - lo] > zmax) zmax = z[j - lo];
        }
        if (rc != ORC_OK) break;
        double sum = 0.0;
        for (int64_t j = lo; j < hi; ++j) sum += exp(z[j - lo] - zmax);
        double l = zmax + log(sum);
        *lse = l;
        for (int64_t j = lo; j < hi; ++j) {
          double p = exp(z[j - lo] - l);
          for (int d = 0; d < D; ++d)
            o[d] += p * kv_elem(v_pool, kv_dtype, v_scale, slots[j - lo],
                                page_size, H_kv, D, g, d);
        }
      }
    }
  }
  free(z);
  free(slots);
  return rc;
}

int tsd_oracle_lse_merge(const double *o_part, const double *lse_part,
                         int rows, int C, int D, double *out,
                         double *out_lse) {
  if (rows < 0 || C <= 0 || D <= 0) return ORC_E_ARG;
  for (int i = 0; i < rows; ++i) {
    const double *lse = lse_part + (int64_t)i * C;
    double M = -INFINITY;
    for (int c = 0; c < C; ++c)
      if (lse[c] > M) M = lse[c];
    double *o = out + (int64_t)i * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      if (out_lse) out_lse[i] = -INFINITY;
      continue;
    }
    double W = 0.0;
    for (int c = 0; c < C; ++c) W += exp(lse[c] - M);
    for (int c = 0; c < C; ++c) {
      double a = exp(lse[c] - M) / W;
      if (a == 0.0) continue;
      const double *oc = o_part + ((int64_t)i * C + c) * D;
      for (int d = 0; d < D; ++d) o[d] += a * oc[d];
    }
    if (out_lse) out_lse[i] = M + log(W);
  }
  return ORC_OK;
}

int tsd_oracle_dense_attention(int B, int H_q, int H_kv, int D, const void *q,
                               int q_dtype, const void *k_pool,
                               const void *v_pool, int kv_dtype,
                               const float *k_scale, const float *v_scale,
                               const int32_t *page_table, int64_t pt_stride,
                               const int32_t *seq_lens, int64_t num_pages,
                               int page_size, double softmax_scale,
                               double *out, double *out_lse) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0 || D <= 0 ||
      !dtype_ok(q_dtype) || !dtype_ok(kv_dtype) || page_size <= 0)
    return ORC_E_ARG;
  if (kv_dtype == ORC_FP8E4M3 && (!k_scale || !v_scale)) return ORC_E_ARG;
  int G = H_q / H_kv;
  for (int b = 0; b < B; ++b) {
    int64_t n = seq_lens[b] > 0 ? seq_lens[b] : 0;
    double *z = (double *)malloc(sizeof(double) * (size_t)(n ? n : 1));
    if (!z) return ORC_E_ARG;
    for (int h = 0; h < H_q; ++h) {
      int g = h / G;
      double *o = out + ((int64_t)b * H_q + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (n == 0) {
        if (out_lse) out_lse[(int64_t)b * H_q + h] = -INFINITY;
        continue;
      }
      /* logits, softmax with the usual max shift, weighted sum of values */
      double zmax = -INFINITY;
      for (int64_t t = 0; t < n; ++t) {
        int64_t slot =
            tsd_oracle_slot(page_table, pt_stride, b, t, page_size, num_pages);
        if (slot < 0) { free(z); return ORC_E_PAGE; }
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += decode_elem(q, q_dtype, ((int64_t)b * H_q + h) * D + d) *
                 kv_elem(k_pool, kv_dtype, k_scale, slot, page_size, H_kv, D,
                         g, d);
        z[t] = softmax_scale * dot;
        if (z[t] > zmax) zmax = z[t];
      }
      double sum = 0.0;
      for (int64_t t = 0; t < n; ++t) sum += exp(z[t] - zmax);
      for (int64_t t = 0; t < n; ++t) {
        int64_t slot =
            tsd_oracle_slot(page_table, pt_stride, b, t, page_size, num_pages);
        double p = exp(z[t] - zmax) / sum;
        for (int d = 0; d < D; ++d)
          o[d] += p * kv_elem(v_pool, kv_dtype, v_scale, slot, page_size,
                              H_kv, D, g, d);
      }
      if (out_lse) out_lse[(int64_t)b * H_q + h] = zmax + log(sum);
    }
    free(z);
  }
  return ORC_OK;
}
