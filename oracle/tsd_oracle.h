/*
 * Plain CPU oracle for top-k sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no source with the HIP path.
 *
 * Every function is a direct, slow transcription of the definition it cites:
 * nested loops, double-precision accumulation, no blocking, fusion or
 * reordering. Layouts match the ones the library takes (token-major paged
 * pools addressed by slot = page_table[b][t / page_size] * page_size +
 * t % page_size) so the same input bytes feed both sides.
 */
#ifndef TSD_ORACLE_H
#define TSD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings of the stored tensors. */
enum {
  ORC_BF16 = 1,     /* bfloat16: 1 sign, 8 exponent, 7 mantissa bits      */
  ORC_FP16 = 2,     /* IEEE-754 binary16                                    */
  ORC_FP8E4M3 = 3,  /* OCP 8-bit float E4M3 ("FN": no inf, one NaN code)  */
  ORC_F32 = 4       /* IEEE-754 binary32                                    */
};

/* Error codes returned by the oracle (0 = success). */
enum {
  ORC_OK = 0,
  ORC_E_ARG = -1,       /* bad argument (shape, dtype, null)              */
  ORC_E_PAGE = -2,      /* a page id outside [0, num_pages)               */
  ORC_E_INDEX = -3,     /* a selected token index outside [0, len)        */
  ORC_E_NAN = -4        /* a NaN score handed to top-k                    */
};

/* Decoders, written from the format definitions. */
double tsd_oracle_decode_fp8e4m3(uint8_t code);
double tsd_oracle_decode_bf16(uint16_t bits);
double tsd_oracle_decode_fp16(uint16_t bits);

/* Physical slot of logical token t of request b, or -1 when the page id
 * read from the page table lies outside [0, num_pages). */
int64_t tsd_oracle_slot(const int32_t *page_table, int64_t pt_stride, int b,
                        int64_t t, int page_size, int64_t num_pages);

/* Double-sparsity label score, one row per (request, KV head):
 *   s[b*H_kv+g][t] = sum_j ( sum_{h in group g} q[b,h,chan[g,j]] )
 *                          * label[slot(b,t), g, j]        for t < seq_lens[b]
 * q: [B, H_q, D] (q_dtype), chan: [H_kv, r], label: [slots, H_kv, r]
 * (label_dtype). Writes scores[row*score_stride + t] for t < len only. */
int tsd_oracle_ds_scores(int B, int H_q, int H_kv, int D, int r,
                         const void *q, int q_dtype, const int32_t *chan,
                         const void *label, int label_dtype,
                         const int32_t *page_table, int64_t pt_stride,
                         const int32_t *seq_lens, int64_t num_pages,
                         int page_size, double *scores, int64_t score_stride);

/* QSA-style index score, one row per query row i (request b = i / R):
 *   s[i][t] = sum_h w[i,h] * max(0, sum_d qi[i,h,d] * ki[slot(b,t), d])
 * for t < n_i, n_i = seq_lens[b] (q_pos == NULL) or
 * min(q_pos[i] + 1, seq_lens[b]) (causal prefill rows; q_pos < 0 -> 0).
 * index_q: [rows, H_i, D_i] FP8 codes, index_w: [rows, H_i] f32,
 * index_k: [slots, D_i] FP8 codes (unit scale). */
int tsd_oracle_qsa_scores(int rows, int R, int H_i, int D_i,
                          const uint8_t *index_q, const float *index_w,
                          const uint8_t *index_k, const int32_t *page_table,
                          int64_t pt_stride, const int32_t *seq_lens,
                          const int32_t *q_pos, int64_t num_pages,
                          int page_size, double *scores, int64_t score_stride);

/* The two score definitions above evaluated only at listed points
 * (pt_row[p], pt_t[p]), p < npts, for sampled checks of large inputs. A point
 * outside a row's length is rejected with ORC_E_INDEX. */
int tsd_oracle_ds_score_points(int B, int H_q, int H_kv, int D, int r,
                               const void *q, int q_dtype, const int32_t *chan,
                               const void *label, int label_dtype,
                               const int32_t *page_table, int64_t pt_stride,
                               const int32_t *seq_lens, int64_t num_pages,
                               int page_size, int64_t npts,
                               const int32_t *pt_row, const int64_t *pt_t,
                               double *out);
int tsd_oracle_qsa_score_points(int rows, int R, int H_i, int D_i,
                                const uint8_t *index_q, const float *index_w,
                                const uint8_t *index_k,
                                const int32_t *page_table, int64_t pt_stride,
                                const int32_t *seq_lens, const int32_t *q_pos,
                                int64_t num_pages, int page_size, int64_t npts,
                                const int32_t *pt_row, const int64_t *pt_t,
                                double *out);

/* Exact top-k per row over scores[row*stride + 0 .. row_lens[row]):
 * the m = min(k, n) indices of the largest scores, equal scores ranked by
 * lower index, returned in ascending index order and padded with -1 up to k.
 * count[row] = m (count may be NULL). Scores compare as floats, so -0 == +0;
 * a NaN is rejected with ORC_E_NAN. */
int tsd_oracle_topk(const float *scores, int64_t stride, int rows,
                    const int32_t *row_lens, int k, int32_t *idx,
                    int32_t *count);

/* The OCP E4M3 code nearest to x: round to nearest, ties to the code with
 * an even mantissa, magnitudes beyond 448 saturating to +-448 (the encoding
 * has no infinity); the sign of x is kept, so -0 and small negatives give
 * 0x80. x must not be NaN. */
uint8_t tsd_oracle_encode_fp8e4m3(double x);

/* Cache append ("Support double sparsity", forward_extend: the label cache
 * is K gathered at the heavy channels and is stored with every new token;
 * "Context parallelism for QSA attention and the sparse indexer",
 * Motivation: the indexer stores raw index-K for every token).
 * For request b the new tokens are positions positions[b] + i for
 * i < clamp(n_new[b], 0, max_new); a position outside the page table's
 * reach, or on a page id outside [0, num_pages), is skipped.
 * Each new token's rows go to slot = page_table[b][t/page_size]*page_size +
 * t%page_size:
 *  - K and V (k_new/v_new [B, max_new, H_kv, D] in new_dtype, a 16-bit
 *    encoding): copied when kv_dtype == new_dtype; for FP8 pools encoded as
 *    e(v / scale) with the page's f32 scale. A page none of whose tokens
 *    precede positions[b] starts in this call: its scale becomes
 *    amax / 448 (1 if amax is 0) over the values this call writes to it
 *    (all heads and dims, K and V separately) and is stored in
 *    k_scale/v_scale; any other page keeps its stored scale. The scale and
 *    the quotient are computed in f32, the code from the f32 quotient.
 *  - label (if label_pool): label[slot][g][j] = K_new[g][channel_idx[g][j]]
 *    in new_dtype (bit copy); a channel outside [0, D) stores 0.
 *  - index-K (if index_k_pool): index_k[slot][d] = e(index_k_new[b][i][d])
 *    with index_k_new in index_dtype (bf16, fp16, or 4 for f32) rounded to
 *    f32 first.
 * Pools not passed (NULL) are left alone. */
int tsd_oracle_kv_append(int B, int64_t pt_stride, const int32_t *page_table,
                         int64_t num_pages, int page_size,
                         const int32_t *positions, const int32_t *n_new,
                         int max_new, int H_kv, int D, const void *k_new,
                         const void *v_new, int new_dtype, void *k_pool,
                         void *v_pool, int kv_dtype, float *k_scale,
                         float *v_scale, const int32_t *channel_idx, int r,
                         void *label_pool, const void *index_k_new,
                         int index_dtype, void *index_k_pool, int D_i);

/* Block-compressed index keys ("QSA cache sharding": QSA compressed cache
 * and compressed blocks chosen by top-k; "Context parallelism for QSA
 * attention and the sparse indexer": block compression of the raw index-K
 * before scoring). Block j of request b holds its tokens
 * [j*Bs, min((j+1)*Bs, len_b)); its key is the mean of their decoded FP8
 * index keys, computed exactly in double, rounded to f32, then encoded to
 * FP8 (nearest, ties to even, saturating). Blocks
 * [from_block[b], ceil(len_b / Bs)) are written, into a paged pool of
 * compressed keys: block j of request b lives at slot
 * cpage_table[b][j / page_size] * page_size + j % page_size of ck_pool
 * [cslots][D_i]. Token pages and compressed pages outside their pools are
 * skipped (a block with a token on a bad page is not written). */
int tsd_oracle_index_k_compress(int B, int Bs, const uint8_t *index_k_pool,
                                const int32_t *page_table, int64_t pt_stride,
                                int64_t num_pages, const int32_t *seq_lens,
                                const int32_t *from_block,
                                const int32_t *cpage_table, int64_t cpt_stride,
                                int64_t num_cpages, int page_size, int D_i,
                                uint8_t *ck_pool);

/* Expansion of selected blocks to their tokens: for each row, the blocks
 * sel[row][0 .. count[row]) (ascending) become the tokens
 * [j*Bs, min((j+1)*Bs, len_row)) in ascending order, written to
 * tok[row][0 .. m) and padded with -1 up to kt; tok_count[row] = m (at most
 * kt: blocks past the capacity are dropped). */
int tsd_oracle_expand_blocks(int rows, const int32_t *sel, const int32_t *count,
                             int kb, int Bs, const int32_t *row_lens, int kt,
                             int32_t *tok, int32_t *tok_count);

/* Exact global top-k from W page-owner shards ("QSA cache sharding",
 * Distributed QSA execution: every rank selects over its own pages, the
 * candidates are exchanged, and one exact top-k with token-id tie-breaking
 * is formed). Shard w owns the logical pages p with p % W == w of every row;
 * its local token u is the global token
 *   t = ((u / page_size) * W + w) * page_size + u % page_size.
 * Inputs per shard: scores [W][rows][stride] in local order, the local top-k
 * lists idx [W][rows][kl] (local tokens, -1 padded) and count [W][rows].
 * Output per row: the m = min(k, sum of counts) candidates ranked highest by
 * (score descending, global token ascending), as global tokens in ascending
 * order, -1 padded to k; out_count[row] = m. A NaN score is ORC_E_NAN. */
int tsd_oracle_topk_merge_sharded(const float *scores, int64_t stride,
                                  const int32_t *idx, const int32_t *count,
                                  int W, int rows, int kl, int page_size,
                                  int k, int32_t *out_idx,
                                  int32_t *out_count);

/* Chunked sparse GQA attention over selected tokens.
 * For request b, query head h (KV head g = h / (H_q / H_kv)) and chunk c of
 * the row's ascending selection list sel[0 .. m): tokens
 * sel[floor(c*m/C) .. floor((c+1)*m/C)), z_t = scale * q[b,h] . Khat_t,
 * lse_c = log sum_t exp(z_t), o_c = sum_t exp(z_t - lse_c) * Vhat_t.
 * Khat = decode(K) * k_scale[page] for FP8 pools, decode(K) otherwise.
 * idx: [B, H_sel, k] with H_sel == 1 (one list per request) or H_kv (one
 * list per KV head); count: [B, H_sel]. Empty chunk -> o = 0, lse = -inf.
 * Outputs are double: o_part [B, H_q, C, D], lse_part [B, H_q, C]. */
int tsd_oracle_sparse_attention(int B, int H_q, int H_kv, int D, int H_sel,
                                int k, int C, const void *q, int q_dtype,
                                const void *k_pool, const void *v_pool,
                                int kv_dtype, const float *k_scale,
                                const float *v_scale,
                                const int32_t *page_table, int64_t pt_stride,
                                const int32_t *seq_lens, int64_t num_pages,
                                int page_size, const int32_t *idx,
                                const int32_t *count, double softmax_scale,
                                double *o_part, double *lse_part);

/* Log-sum-exp merge of C partial results per row:
 *   M = max_c lse_c, W = sum_c exp(lse_c - M),
 *   out = sum_c exp(lse_c - M) * o_c / W, out_lse = M + log W;
 * all lse_c = -inf -> out = 0, out_lse = -inf. */
int tsd_oracle_lse_merge(const double *o_part, const double *lse_part,
                         int rows, int C, int D, double *out, double *out_lse);

/* Textbook dense attention over every token t < seq_lens[b], used only to
 * check invariants (top-k >= context must reproduce it). */
int tsd_oracle_dense_attention(int B, int H_q, int H_kv, int D, const void *q,
                               int q_dtype, const void *k_pool,
                               const void *v_pool, int kv_dtype,
                               const float *k_scale, const float *v_scale,
                               const int32_t *page_table, int64_t pt_stride,
                               const int32_t *seq_lens, int64_t num_pages,
                               int page_size, double softmax_scale,
                               double *out, double *out_lse);

#ifdef __cplusplus
}
#endif
#endif /* TSD_ORACLE_H */
