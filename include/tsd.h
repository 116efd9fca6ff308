/*
 * tsd.h -- C ABI of libtsd.so, top-k sparse decode attention for AMD MI355X
 * (gfx950).
 *
 * The decode path is four calls, each an asynchronous launch on the caller's
 * HIP stream:
 *
 *   sparse_index_score  score every cached token of every query row with a
 *                       cheap key (double-sparsity label K, or a QSA-style
 *                       FP8 index K);
 *   topk_select         exact top-k per row, lowest token index first among
 *                       equal scores, listed in ascending index order;
 *   sparse_gqa_decode   gather the selected tokens' K/V from the 64-token
 *                       paged cache and run GQA attention over them, split
 *                       into chunks, with FP32 partial outputs and LSEs;
 *   lse_merge           combine the chunks with an FP32 log-sum-exp merge.
 *
 * Where the operations come from (page title, section):
 *   - "QSA HiSparse -- SGLang plugin", Supported versions / Run: FP8 E4M3
 *     KV cache in 64-token pages, up to 8 running requests.
 *   - "QSA cache sharding" (sglang PR #43527), Implementation: the request
 *     token mapping into cache pages; exact Top-K with deterministic token-ID
 *     tie-breaking; sparse attention over the selected tokens; FP32
 *     log-sum-exp merge of partial outputs; fixed-address buffers and
 *     consumers bounded by lengths for CUDA-graph replay.
 *   - "Context parallelism for QSA attention and the sparse indexer" (sglang
 *     PR #39721), Motivation: the indexer scores index keys and selects
 *     top-k per query row, for decode and for chunked-prefill rows; sparse
 *     GQA attention over the selection.
 *   - "Support double sparsity" (sglang PR #1459), Speedup Evaluation and
 *     the forward_extend traceback: label K = K at per-head heavy channels
 *     ([tokens, heads, heavy channels]); heavy-token count = top-k.
 *
 * Conventions shared by every call
 *   - Every pointer argument is caller-owned DEVICE memory unless stated.
 *     The library allocates nothing, never synchronises the stream, never
 *     reads device memory on the host and keeps no state, so a sequence of
 *     calls can be captured into a HIP graph and calls are thread-safe.
 *   - Return 0 on success. A negative value (TSD_E_*) means the host-side
 *     arguments were rejected and NOTHING was launched. A positive value is
 *     the hipError_t of a failed launch.
 *   - Paged pools are token-major and slot-addressed: token t of request b
 *     lives at slot = page_table[b * pt_stride + t / 64] * 64 + t % 64.
 *     page_size must be 64.
 *   - Lengths and indices live in device memory, so kernels bound every
 *     access themselves: a length is clamped to what the host arguments can
 *     hold (pt_stride * 64 tokens, score_stride / max_len entries); page-table
 *     entries at or past ceil(len / 64) are never used (a scan may load any
 *     of the row's pt_stride entries before the length arrives, but never
 *     the pages they name), so stale tails are fine; a page id outside
 *     [0, num_pages) or a selected index outside [0, len) is skipped rather
 *     than dereferenced (that data is a caller error and its contribution
 *     is dropped).
 */
#ifndef TSD_H
#define TSD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSD_ABI_VERSION 1

/* Element encodings. FP8 is OCP E4M3 "FN" (bias 7, max 448, no inf). */
enum {
  TSD_BF16 = 1,
  TSD_FP16 = 2,
  TSD_FP8_E4M3 = 3,
  TSD_F32 = 4       /* IEEE binary32 (kv_append's index_k_new only)      */
};

/* Status codes (negative: rejected on the host, nothing launched). */
enum {
  TSD_OK = 0,
  TSD_E_NULL = -1,        /* a required pointer is NULL                      */
  TSD_E_DTYPE = -2,       /* unsupported or inconsistent element encoding    */
  TSD_E_SHAPE = -3,       /* a size is negative, zero where it must not be,
                             or exceeds a supported bound                    */
  TSD_E_PAGE_SIZE = -4,   /* page_size != 64                                 */
  TSD_E_GQA = -5,         /* H_q % H_kv != 0, or H_sel not in {1, H_kv}      */
  TSD_E_K = -6,           /* top_k outside [1, 4096]                         */
  TSD_E_CHUNKS = -7,      /* chunks outside [1, 64]                          */
  TSD_E_WORKSPACE = -8,   /* workspace NULL or smaller than required         */
  TSD_E_UNSUPPORTED = -9, /* a valid but unsupported configuration (D, r...) */
  TSD_E_MODE = -10,       /* unknown score mode                              */
  TSD_E_ABI = -11,        /* args struct built for another ABI version       */
  TSD_E_SCRATCH = -12     /* needs more than the built-in scratch of
                             topk_select_noalloc                             */
};

/* Supported bounds of this version. */
#define TSD_HEAD_DIM 128    /* D of K/V and of the index keys                */
#define TSD_MAX_INDEX_HEADS 16
#define TSD_MAX_TOPK 4096
#define TSD_MAX_CHUNKS 64
#define TSD_MAX_GQA_GROUP 16
#define TSD_PAGE_SIZE 64

/* ------------------------------------------------------------------------
 * sparse_index_score
 *
 * Mode TSD_SCORE_DS_LABEL (double sparsity). One row per (request b, KV
 * head g), row = b * H_kv + g, n = seq_lens[b] keys:
 *   scores[row][t] = sum_{j<r} qs[b,g,j] * label_pool[slot(b,t)][g][j],
 *   qs[b,g,j]      = sum_{h = g*G .. g*G+G-1} q[b][h][channel_idx[g][j]],
 * G = H_q / H_kv (the query of a GQA group is the sum of its heads).
 *   q            [B, H_q, D]        bf16 or fp16 (q_dtype), D == 128
 *   channel_idx  [H_kv, r]          int32, each in [0, D), 1 <= r <= 128
 *   label_pool   [num_pages*64, H_kv, r]  same encoding as q
 *
 * Mode TSD_SCORE_QSA_INDEX (index keys). One row per query row i, request
 * b = i / rows_per_req, rows = B * rows_per_req:
 *   scores[i][t] = sum_{h<H_i} index_w[i][h] *
 *                  max(0, sum_{d<D_i} index_q[i][h][d] * index_k[slot(b,t)][d])
 * for t < n_i, n_i = seq_lens[b] (q_pos == NULL: decode rows) or
 * min(q_pos[i] + 1, seq_lens[b]) (causal chunked-prefill rows; q_pos < 0
 * gives 0 keys).
 *   index_q      [rows, H_i, D_i]   FP8 E4M3 codes, H_i <= 16, D_i == 128
 *   index_w      [rows, H_i]        f32
 *   index_k_pool [num_pages*64, D_i] FP8 E4M3 codes (unit scale)
 *   q_pos        [rows] int32 or NULL
 *
 * Output: scores f32 [rows, score_stride]. Exactly the entries t < n of
 * every row are written -- also when n <= top_k -- and the tail of each row
 * is left untouched. A key on an out-of-range page scores -inf.
 * row_lens_out (optional, int32 [rows]) receives each row's n, the count
 * topk_select takes as its row length.
 * ------------------------------------------------------------------------ */
enum { TSD_SCORE_DS_LABEL = 1, TSD_SCORE_QSA_INDEX = 2 };

typedef struct tsd_score_args {
  int32_t abi_version;           /* TSD_ABI_VERSION                          */
  int32_t mode;                  /* TSD_SCORE_*                              */
  /* batch view of the paged cache */
  int32_t B;                     /* requests, >= 0                           */
  int32_t page_size;             /* 64                                       */
  const int32_t *page_table;     /* [B, pt_stride] physical page ids        */
  int64_t pt_stride;             /* >= 1                                     */
  const int32_t *seq_lens;       /* [B] cached tokens per request           */
  int64_t num_pages;             /* pages in every pool                      */
  /* double sparsity (mode DS_LABEL) */
  const void *q;
  int32_t q_dtype;               /* TSD_BF16 | TSD_FP16                      */
  int32_t H_q;
  int32_t H_kv;
  int32_t D;
  const int32_t *channel_idx;
  int32_t r;
  int32_t label_dtype;           /* == q_dtype                               */
  const void *label_pool;
  /* index keys (mode QSA_INDEX) */
  const uint8_t *index_q;
  const float *index_w;
  const uint8_t *index_k_pool;
  const int32_t *q_pos;          /* NULL for decode                          */
  int32_t rows_per_req;          /* >= 1                                     */
  int32_t H_i;
  int32_t D_i;
  int32_t reserved0;
  /* output */
  float *scores;
  int64_t score_stride;          /* >= 1                                     */
  int32_t *row_lens_out;         /* [rows] or NULL                           */
} tsd_score_args;

int sparse_index_score(const tsd_score_args *a, hipStream_t stream);

/* ------------------------------------------------------------------------
 * topk_select
 *
 * For each row, n = clamp(row_lens[row], 0, min(max_len, stride)) and
 * m = min(k, n): idx[row][0 .. m) are the indices of the m largest of
 * scores[row][0 .. n), in strictly ascending order; among equal scores the
 * lower index is taken. idx[row][m .. k) = -1; count[row] = m (count may be
 * NULL). Scores compare as floats: -0 and +0 are equal; +-inf are allowed;
 * NaN is outside the contract. Any entry of scores[row][0 .. min(max_len,
 * stride)) may be read, whatever the row's length (entries at or past it
 * are ignored), so the whole [rows, stride] buffer must be allocated.
 *   scores   [rows, stride] f32          row_lens [rows] int32
 *   idx      [rows, k] int32             count    [rows] int32 or NULL
 *   max_len  host-side bound on every row length (sizes the launch)
 *   ws       device workspace of at least topk_select_workspace_bytes()
 *            bytes, 16-byte aligned, caller-owned (one workspace per
 *            concurrent call); TSD_E_WORKSPACE if NULL, too small or
 *            misaligned. Its contents on entry do not matter: the call
 *            zeroes the histograms it needs (one small launch) and returns
 *            with its first rows * 5120 32-bit words zero again.
 * 1 <= k <= 4096; 0 <= rows <= 65535; stride >= max_len >= 0;
 * max_len <= 16,777,216.
 * ------------------------------------------------------------------------ */
size_t topk_select_workspace_bytes(int rows, int max_len, int k);

int topk_select(const float *scores, int64_t stride, int rows,
                const int32_t *row_lens, int max_len, int k, int32_t *idx,
                int32_t *count, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * topk_select_ex
 *
 * topk_select with flags. TSD_TOPK_WS_ZEROED tells the call that the first
 * rows * 5120 32-bit words of ws (the histograms) are zero already, which
 * skips the zeroing launch: true when the workspace was zero-filled, or was
 * last used by a completed selection call (topk_select, topk_select_ex or
 * sparse_index_topk, on the same stream or ordered before this one) with at
 * least as many rows, since every such call leaves them zero. Other flag
 * bits: TSD_E_UNSUPPORTED. Everything else as for topk_select.
 * ------------------------------------------------------------------------ */
#define TSD_TOPK_WS_ZEROED 1

int topk_select_ex(const float *scores, int64_t stride, int rows,
                   const int32_t *row_lens, int max_len, int k, int32_t *idx,
                   int32_t *count, void *ws, size_t ws_bytes, int flags,
                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * topk_select_noalloc
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * selection of topk_select, identical results, with its workspace in a
 * fixed device array inside the library instead of a caller buffer. The
 * call allocates nothing; the array (topk_select_noalloc_max_bytes() =
 * 8 MiB) exists once per GPU the library runs on and lives until the
 * process ends. A selection that needs more than that,
 * topk_select_workspace_bytes(rows, max_len, k) > the maximum, returns
 * TSD_E_SCRATCH with nothing launched (8 rows of 262,144 need 2.3 MB, one
 * row of 1,048,576 1.1 MB). Every call on a GPU shares that GPU's array and
 * clears what must start at zero itself, so calls that overlap on one GPU
 * (other streams, other threads) race: order them. The first call on a
 * device looks up the array's address there. Arguments and errors
 * otherwise as for topk_select.
 * ------------------------------------------------------------------------ */
size_t topk_select_noalloc_max_bytes(void);

int topk_select_noalloc(const float *scores, int64_t stride, int rows,
                        const int32_t *row_lens, int max_len, int k,
                        int32_t *idx, int32_t *count, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sparse_index_topk
 *
 * sparse_index_score followed by topk_select on the scores it writes, with
 * identical results, in fewer passes: for long rows the index scan also
 * builds the first radix-digit histogram of every row, so the selection
 * skips its own histogram pass and one read of the scores (QSA_INDEX mode;
 * DS_LABEL runs the two steps back to back); rows of up to 32,768 entries
 * are selected, as by topk_select, in one launch that reads each row once
 * and uses the workspace only for its zeroing contract (see topk_select).
 * The scores are still written to a->scores.
 *   a->row_lens_out  required: receives each row's key count
 *   rows             B * H_kv (DS) or B * rows_per_req (QSA)
 *   max_len          min(a->score_stride, a->pt_stride * 64)
 *   ws / ws_bytes    topk_select_workspace_bytes(rows, max_len, k) bytes
 *   idx, count, k, flags   as for topk_select_ex
 * ------------------------------------------------------------------------ */
int sparse_index_topk(const tsd_score_args *a, int k, int32_t *idx,
                      int32_t *count, void *ws, size_t ws_bytes, int flags,
                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * topk_merge_sharded
 *
 * Exact global top-k from W page-owner shards ("QSA cache sharding", sglang
 * PR #43527, Distributed QSA execution: each rank selects over its own
 * pages, the candidates are exchanged, and one exact top-k with token-id
 * tie-breaking is formed). Shard w owns the logical pages p with
 * p % W == w of every row; its local token u is the global token
 * ((u / 64) * W + w) * 64 + u % 64. The inputs are each shard's scores in
 * its local token order and its topk_select output; for each row the call
 * writes the m = min(k, valid candidates) candidates ranked highest by
 * (score descending, global token ascending) as global tokens in strictly
 * ascending order, then -1 padding; count[row] = m. When every shard
 * selected kl >= k (or all of its tokens), the result equals topk_select on
 * the unsharded row.
 *   scores       [W, rows, stride] f32   shard-local scores
 *   idx_local    [W, rows, kl] int32     shard topk_select outputs
 *   count_local  [W, rows] int32         their counts (entries j >= count,
 *                                        and tokens outside [0, stride),
 *                                        are ignored)
 *   idx          [rows, k] int32 out     count [rows] int32 out or NULL
 * 1 <= W <= 16; 1 <= kl, k <= 4096; W * kl <= 16,384; rows <= 65,535;
 * W * stride <= 2^31 - 1. No workspace; nothing is allocated.
 * ------------------------------------------------------------------------ */
int topk_merge_sharded(const float *scores, int64_t stride,
                       const int32_t *idx_local, const int32_t *count_local,
                       int W, int rows, int kl, int k, int32_t *idx,
                       int32_t *count, hipStream_t stream);

/* ------------------------------------------------------------------------
 * sparse_gqa_decode
 *
 * For request b, query head h, KV head g = h / G (G = H_q / H_kv) and chunk
 * c < chunks of the selection sel = idx[b][s][0 .. m), s = 0 if H_sel == 1
 * (one list shared by all KV heads) else g, m = clamp(count[b][s], 0, k):
 *   tokens  sel[floor(c*m/C) .. floor((c+1)*m/C))   (C = chunks)
 *   z_t     = softmax_scale * sum_d q[b][h][d] * Khat[slot(b,t)][g][d]
 *   lse_part[b][h][c]  = log sum_t exp(z_t)                  (natural log)
 *   o_part[b][h][c][:] = sum_t exp(z_t - lse) * Vhat[slot(b,t)][g][:]
 * Khat/Vhat = the stored value (bf16/fp16), or the FP8 code times
 * k_scale / v_scale of the token's physical page. An empty chunk (or a
 * request with no selection) writes o = 0 and lse = -inf. Only pages below
 * ceil(len / 64) are read.
 *   q        [B, H_q, D] bf16 or fp16, D == 128
 *   k_pool   [num_pages*64, H_kv, D]   bf16 | fp16 | fp8 (kv_dtype)
 *   v_pool   same as k_pool
 *   k_scale, v_scale [num_pages] f32 (FP8 only; NULL otherwise)
 *   idx      [B, H_sel, k] int32 ascending, -1 padded   count [B, H_sel]
 *   o_part   [B, H_q, chunks, D] f32     lse_part [B, H_q, chunks] f32
 * Sparse-decode threshold ("Support double sparsity", Speedup Evaluation:
 * short contexts decode densely): a request whose length len (clamped to
 * pt_stride * 64) is at most dense_len attends to every token 0 .. len-1 as
 * its selection (m = len; its idx entries and count are not used, though
 * its row of idx, allocated like every other, may be loaded). dense_len = 0
 * turns this off.
 * Block selections (idx_block = Bs in {2, 4, ..., 64}; 0 or 1 = token
 * indices): idx row holds the first count ascending indices of selected
 * blocks of Bs tokens (block j = tokens [j*Bs, min((j+1)*Bs, len)), as
 * index_k_compress builds them), k being the block capacity. The selection is
 * then the blocks' tokens in order, position p being token
 * idx[p / Bs] * Bs + p % Bs, and m = count * Bs less the tokens of the last
 * block at or past len: the token list expand_blocks writes for such a
 * selection, so the result equals attention over that list. An entry outside
 * [0, ceil(len / Bs)) keeps its positions and its tokens are skipped.
 * For a 16-bit cache q must have the cache's encoding; an FP8 cache takes
 * bf16 or fp16 queries. H_q % H_kv == 0, G <= 16, 1 <= chunks <= 64,
 * 1 <= k <= 4096, dense_len >= 0.
 * ------------------------------------------------------------------------ */
typedef struct tsd_attn_args {
  int32_t abi_version;           /* TSD_ABI_VERSION                          */
  int32_t B;
  int32_t H_q;
  int32_t H_kv;
  int32_t D;
  int32_t q_dtype;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  int32_t kv_dtype;
  int32_t page_size;             /* 64                                       */
  const float *k_scale;
  const float *v_scale;
  const int32_t *page_table;
  int64_t pt_stride;
  const int32_t *seq_lens;
  int64_t num_pages;
  const int32_t *idx;
  const int32_t *count;
  int32_t H_sel;                 /* 1 or H_kv                                */
  int32_t k;
  int32_t chunks;
  float softmax_scale;           /* usually 1/sqrt(D)                        */
  float *o_part;
  float *lse_part;
  int32_t dense_len;             /* requests with len <= dense_len: dense    */
  int32_t idx_block;             /* 0 or 1: token indices; else block size   */
} tsd_attn_args;

int sparse_gqa_decode(const tsd_attn_args *a, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lse_merge
 *
 * For each of rows partial sets (rows = B * H_q) with C chunks:
 *   M = max_c lse_part[row][c],  W = sum_c exp(lse_part[row][c] - M)
 *   out[row][:] = sum_c exp(lse_part[row][c] - M) * o_part[row][c][:] / W
 *   out_lse[row] = M + log W
 * All chunks empty (every lse = -inf): out = 0, out_lse = -inf.
 *   o_part [rows, C, D] f32   lse_part [rows, C] f32
 *   out    [rows, D] f32      out_lse  [rows] f32 or NULL
 * 1 <= C <= 64, 1 <= D <= 512, D % 4 == 0.
 * ------------------------------------------------------------------------ */
int lse_merge(const float *o_part, const float *lse_part, int rows, int C,
              int D, float *out, float *out_lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * kv_append
 *
 * Stores the rows of newly appended tokens into the paged pools ("Support
 * double sparsity", forward_extend in the discussion: the label cache is K
 * gathered at the heavy channels and is written with every new token;
 * "Context parallelism for QSA attention and the sparse indexer",
 * Motivation: the indexer stores raw index-K for every token). For request
 * b the new tokens are the positions positions[b] + i,
 * i < clamp(n_new[b], 0, max_new); token t goes to
 * slot = page_table[b][t / 64] * 64 + t % 64. A position at or past
 * pt_stride * 64, or on a page id outside [0, num_pages), is skipped.
 *  - K and V (when k_new is not NULL): k_new, v_new [B, max_new, H_kv, D]
 *    in new_dtype (BF16/FP16). A pool in new_dtype gets a copy. An FP8
 *    pool gets code(value / scale) with the page's f32 scale: a page none
 *    of whose tokens precede positions[b] is started by the call and its
 *    scale becomes amax / 448 (1 for amax 0) over the values the call
 *    writes to it (all heads and dims; K and V separately) when the call
 *    writes all 64 of its tokens, and 4 * amax / 448 when it writes fewer
 *    (headroom for the tokens later calls append), stored in k_scale /
 *    v_scale; any other page keeps its stored scale, and values beyond
 *    448 * scale saturate. Scale and quotient are computed in f32;
 *    code() rounds to nearest, ties to even.
 *  - label (when channel_idx is not NULL): label_pool [slots, H_kv, r]
 *    (new_dtype) gets K_new[g][channel_idx[g][j]] for j < r (a channel
 *    outside [0, D) stores 0).
 *  - index-K (when index_k_new is not NULL): index_k_pool [slots, D_i]
 *    FP8 gets code(index_k_new[b][i][d]) (unit scale), index_k_new
 *    [B, max_new, D_i] in index_dtype (BF16, FP16 or F32).
 * D = D_i = 128; 1 <= r <= D; H_kv * D <= 4096; every row and pool
 * pointer 16-byte aligned (else TSD_E_UNSUPPORTED). A call with no pool to
 * write launches nothing. Two calls that write the same page of an FP8 pool
 * must not run concurrently.
 * ------------------------------------------------------------------------ */
typedef struct tsd_append_args {
  int32_t abi_version;        /* TSD_ABI_VERSION                             */
  int32_t B;
  int32_t page_size;          /* must be 64                                  */
  int32_t max_new;            /* host bound on n_new[b] (sizes the launch)   */
  const int32_t *page_table;  /* [B, pt_stride]                              */
  int64_t pt_stride;
  int64_t num_pages;
  const int32_t *positions;   /* [B] first new position of each request      */
  const int32_t *n_new;       /* [B] new tokens of each request              */
  int32_t H_kv, D;
  int32_t new_dtype;          /* encoding of k_new / v_new / label           */
  int32_t kv_dtype;           /* pool encoding: new_dtype or TSD_FP8_E4M3    */
  const void *k_new, *v_new;
  void *k_pool, *v_pool;
  float *k_scale, *v_scale;   /* [num_pages], FP8 pools only                 */
  const int32_t *channel_idx; /* [H_kv, r]                                   */
  void *label_pool;
  int32_t r;
  int32_t index_dtype;
  const void *index_k_new;
  void *index_k_pool;
  int32_t D_i;
  int32_t reserved0;
} tsd_append_args;

int kv_append(const tsd_append_args *a, hipStream_t stream);

/* ------------------------------------------------------------------------
 * index_k_compress / expand_blocks
 *
 * Block-compressed QSA selection ("QSA cache sharding": the compressed
 * cache and the top-k over compressed blocks; "Context parallelism for QSA
 * attention and the sparse indexer": block compression of the raw index-K
 * before scoring). Block j of request b holds its tokens
 * [j*Bs, min((j+1)*Bs, len_b)), Bs = block_size in {1, 2, 4, ..., 64}.
 *
 * index_k_compress writes the compressed key of blocks
 * [from_block[b], from_block[b] + max_blocks) that lie below
 * ceil(len_b / Bs) (from_block NULL: 0): the mean of the block's decoded
 * FP8 index keys (exact in f64, rounded to f32, encoded to FP8 by round to
 * nearest even, saturating at 448), stored at slot
 * cpage_table[b][j / 64] * 64 + j % 64 of ck_pool [cslots, 128]. A block
 * with a token on a page outside [0, num_pages), or whose compressed page
 * is outside [0, num_cpages), is not written. The compressed pool is an
 * index-K pool of its own: sparse_index_score / sparse_index_topk score and
 * select blocks through cpage_table with seq_lens = ceil(len / Bs).
 *
 * expand_blocks turns each row's selected blocks sel [rows, kb] (ascending,
 * first count[row] entries, negatives ignored) into their tokens in
 * ascending order: tok [rows, kt] (-1 padded), tok_count [rows] (NULL ok)
 * = the number written, at most kt. row_lens [rows] are the token lengths.
 * 1 <= kb, kt <= 4096; rows <= 65,535. index_k_pool and ck_pool must be
 * 16-byte aligned (else TSD_E_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
typedef struct tsd_compress_args {
  int32_t abi_version;          /* TSD_ABI_VERSION                           */
  int32_t B;
  int32_t page_size;            /* must be 64                                */
  int32_t block_size;           /* Bs                                        */
  const uint8_t *index_k_pool;  /* [slots, 128] FP8                          */
  const int32_t *page_table;    /* [B, pt_stride]                            */
  int64_t pt_stride;
  int64_t num_pages;
  const int32_t *seq_lens;      /* [B] token lengths                         */
  const int32_t *from_block;    /* [B] or NULL                               */
  int32_t max_blocks;           /* host bound on blocks written per request  */
  int32_t D_i;                  /* 128                                       */
  uint8_t *ck_pool;             /* [cslots, 128] FP8                         */
  const int32_t *cpage_table;   /* [B, cpt_stride]                           */
  int64_t cpt_stride;
  int64_t num_cpages;
} tsd_compress_args;

int index_k_compress(const tsd_compress_args *a, hipStream_t stream);

int expand_blocks(const int32_t *sel, const int32_t *count, int rows, int kb,
                  int block_size, const int32_t *row_lens, int kt,
                  int32_t *tok, int32_t *tok_count, hipStream_t stream);

/* Human-readable name of a status code (static string, host only). */
const char *tsd_strerror(int status);

/* TSD_ABI_VERSION of the built library. */
int tsd_abi_version(void);

/* SHA-256 (64 hex digits, static string) of the sources the library was
 * built from, so that a binding can refuse a library built from other
 * sources than the ones beside it. */
const char *tsd_source_sha256(void);

/* sizeof the argument structs as compiled into the library, so a binding
 * can check its own layout. */
size_t tsd_sizeof_score_args(void);
size_t tsd_sizeof_attn_args(void);
size_t tsd_sizeof_append_args(void);
size_t tsd_sizeof_compress_args(void);

#ifdef __cplusplus
}
#endif
#endif /* TSD_H */
