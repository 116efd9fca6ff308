// C-ABI entry points of libtsd.so: host-side validation, then the launch.
// Validation never touches the HIP runtime or device memory, so every error
// path returns before anything is enqueued (and can be exercised on a host
// without a GPU).
#include <limits>

#include "launch.h"
#include "tsd.h"

// Set by the build to the SHA-256 of the library's sources.
#ifndef TSD_SOURCE_SHA256
#define TSD_SOURCE_SHA256 "unknown"
#endif

namespace {

constexpr int64_t kMaxGrid = std::numeric_limits<int32_t>::max();

bool half_enc(int e) { return e == TSD_BF16 || e == TSD_FP16; }
bool any_enc(int e) { return half_enc(e) || e == TSD_FP8_E4M3; }

int check_batch_view(int32_t B, int32_t page_size, const int32_t* pt,
                     int64_t pt_stride, const int32_t* lens,
                     int64_t num_pages) {
  if (B < 0 || pt_stride < 1 || num_pages < 0) return TSD_E_SHAPE;
  if (page_size != TSD_PAGE_SIZE) return TSD_E_PAGE_SIZE;
  if (B > 0 && (!pt || !lens)) return TSD_E_NULL;
  if (B > 65535) return TSD_E_UNSUPPORTED;
  return TSD_OK;
}

int validate_score(const tsd_score_args* a) {
  if (!a) return TSD_E_NULL;
  if (a->abi_version != TSD_ABI_VERSION) return TSD_E_ABI;
  if (a->mode != TSD_SCORE_DS_LABEL && a->mode != TSD_SCORE_QSA_INDEX)
    return TSD_E_MODE;
  int rc = check_batch_view(a->B, a->page_size, a->page_table, a->pt_stride,
                            a->seq_lens, a->num_pages);
  if (rc) return rc;
  if (a->score_stride < 1) return TSD_E_SHAPE;
  if (a->B > 0 && !a->scores) return TSD_E_NULL;
  if (a->mode == TSD_SCORE_DS_LABEL) {
    if (a->B > 0 && (!a->q || !a->channel_idx || !a->label_pool))
      return TSD_E_NULL;
    if (!half_enc(a->q_dtype) || a->label_dtype != a->q_dtype)
      return TSD_E_DTYPE;
    if (a->H_q < 1 || a->H_kv < 1 || a->r < 1 || a->D < 1) return TSD_E_SHAPE;
    if (a->H_q % a->H_kv) return TSD_E_GQA;
    if (a->D != TSD_HEAD_DIM || a->r > a->D) return TSD_E_UNSUPPORTED;
    if (a->H_kv > 128 || static_cast<int64_t>(a->H_kv) * a->r > 4096)
      return TSD_E_UNSUPPORTED;
    if (a->pt_stride > kMaxGrid) return TSD_E_UNSUPPORTED;
  } else {
    if (a->B > 0 && (!a->index_q || !a->index_w || !a->index_k_pool))
      return TSD_E_NULL;
    if (a->rows_per_req < 1 || a->H_i < 1 || a->D_i < 1) return TSD_E_SHAPE;
    if (a->H_i > TSD_MAX_INDEX_HEADS || a->D_i != TSD_HEAD_DIM)
      return TSD_E_UNSUPPORTED;
    const int64_t rows = static_cast<int64_t>(a->B) * a->rows_per_req;
    if (rows > kMaxGrid) return TSD_E_UNSUPPORTED;
    if (a->pt_stride * TSD_PAGE_SIZE > kMaxGrid) return TSD_E_UNSUPPORTED;
    const int64_t waves = rows * ((a->pt_stride + 3) / 4);
    if (waves / 4 + 1 > kMaxGrid) return TSD_E_UNSUPPORTED;
  }
  return TSD_OK;
}

int validate_topk(const float* scores, int64_t stride, int rows,
                  const int32_t* row_lens, int max_len, int k, int32_t* idx,
                  void* ws, size_t ws_bytes) {
  if (rows < 0 || max_len < 0 || stride < 1 || stride < max_len)
    return TSD_E_SHAPE;
  if (k < 1 || k > TSD_MAX_TOPK) return TSD_E_K;
  if (rows > 65535 || max_len > tsd::topk_max_len()) return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  if (!scores || !row_lens || !idx) return TSD_E_NULL;
  if (!ws || ws_bytes < tsd::topk_workspace(rows, max_len, k) ||
      (reinterpret_cast<uintptr_t>(ws) & 15u) != 0)
    return TSD_E_WORKSPACE;
  return TSD_OK;
}

int validate_attn(const tsd_attn_args* a) {
  if (!a) return TSD_E_NULL;
  if (a->abi_version != TSD_ABI_VERSION) return TSD_E_ABI;
  int rc = check_batch_view(a->B, a->page_size, a->page_table, a->pt_stride,
                            a->seq_lens, a->num_pages);
  if (rc) return rc;
  if (a->H_q < 1 || a->H_kv < 1 || a->D < 1) return TSD_E_SHAPE;
  if (a->H_q % a->H_kv) return TSD_E_GQA;
  if (a->H_sel != 1 && a->H_sel != a->H_kv) return TSD_E_GQA;
  if (a->H_q / a->H_kv > TSD_MAX_GQA_GROUP) return TSD_E_UNSUPPORTED;
  if (a->D != TSD_HEAD_DIM) return TSD_E_UNSUPPORTED;
  if (a->H_kv > 65535) return TSD_E_UNSUPPORTED;
  if (a->k < 1 || a->k > TSD_MAX_TOPK) return TSD_E_K;
  if (a->chunks < 1 || a->chunks > TSD_MAX_CHUNKS) return TSD_E_CHUNKS;
  if (a->dense_len < 0) return TSD_E_SHAPE;
  if (a->idx_block < 0 || a->idx_block > TSD_PAGE_SIZE ||
      (a->idx_block & (a->idx_block - 1)) != 0)
    return TSD_E_UNSUPPORTED;
  if (!any_enc(a->kv_dtype) || !half_enc(a->q_dtype)) return TSD_E_DTYPE;
  if (a->kv_dtype != TSD_FP8_E4M3 && a->q_dtype != a->kv_dtype)
    return TSD_E_DTYPE;
  if (a->B == 0) return TSD_OK;
  if (!a->q || !a->k_pool || !a->v_pool || !a->idx || !a->count ||
      !a->o_part || !a->lse_part)
    return TSD_E_NULL;
  if (a->kv_dtype == TSD_FP8_E4M3 && (!a->k_scale || !a->v_scale))
    return TSD_E_NULL;
  return TSD_OK;
}

int validate_merge(const float* o_part, const float* lse_part, int rows,
                   int C, int D, float* out) {
  if (rows < 0 || D < 1) return TSD_E_SHAPE;
  if (C < 1 || C > TSD_MAX_CHUNKS) return TSD_E_CHUNKS;
  if (D > 512) return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  if (!o_part || !lse_part || !out) return TSD_E_NULL;
  return TSD_OK;
}

int launch_status(hipError_t e) {
  return e == hipSuccess ? TSD_OK : static_cast<int>(e);
}

}  // namespace

extern "C" {

int sparse_index_score(const tsd_score_args* a, hipStream_t stream) {
  const int rc = validate_score(a);
  if (rc) return rc;
  if (a->B == 0) return TSD_OK;
  if (a->mode == TSD_SCORE_DS_LABEL)
    return launch_status(tsd::launch_ds_scan(*a, stream));
  return launch_status(tsd::launch_qsa_scan(*a, stream));
}

int sparse_index_topk(const tsd_score_args* a, int k, int32_t* idx,
                      int32_t* count, void* ws, size_t ws_bytes, int flags,
                      hipStream_t stream) {
  int rc = validate_score(a);
  if (rc) return rc;
  if (flags & ~TSD_TOPK_WS_ZEROED) return TSD_E_UNSUPPORTED;
  const int64_t rows64 = a->mode == TSD_SCORE_DS_LABEL
                             ? static_cast<int64_t>(a->B) * a->H_kv
                             : static_cast<int64_t>(a->B) * a->rows_per_req;
  int64_t max_len = a->score_stride;
  if (a->pt_stride * TSD_PAGE_SIZE < max_len) max_len = a->pt_stride * TSD_PAGE_SIZE;
  if (rows64 > 65535 || max_len > tsd::topk_max_len()) return TSD_E_UNSUPPORTED;
  const int rows = static_cast<int>(rows64);
  rc = validate_topk(a->scores, a->score_stride, rows, a->row_lens_out,
                     static_cast<int>(max_len), k, idx, ws, ws_bytes);
  if (rc) return rc;
  if (a->B == 0) return TSD_OK;
  hipError_t e = hipSuccess;
  if (!(flags & TSD_TOPK_WS_ZEROED)) e = tsd::launch_topk_clear(ws, rows, stream);
  if (e != hipSuccess) return launch_status(e);
  if (tsd::topk_small_fits(static_cast<int>(max_len), rows, k)) {
    e = a->mode == TSD_SCORE_QSA_INDEX ? tsd::launch_qsa_scan(*a, stream)
                                       : tsd::launch_ds_scan(*a, stream);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(tsd::launch_topk_small(
        a->scores, a->score_stride, rows, a->row_lens_out,
        static_cast<int>(max_len), k, idx, count, stream));
  }
  if (a->mode == TSD_SCORE_QSA_INDEX && a->rows_per_req < 64) {
    e = tsd::launch_qsa_scan(*a, stream, ws, k);
  } else if (a->mode == TSD_SCORE_QSA_INDEX) {  // prefill rows: tiled kernel
    e = tsd::launch_qsa_scan(*a, stream);
    if (e == hipSuccess)
      e = tsd::launch_topk_hist1(a->scores, a->score_stride, rows,
                                 a->row_lens_out, static_cast<int>(max_len), k,
                                 ws, stream);
  } else {
    e = tsd::launch_ds_scan(*a, stream);
    if (e == hipSuccess)
      e = tsd::launch_topk_hist1(a->scores, a->score_stride, rows,
                                 a->row_lens_out, static_cast<int>(max_len), k,
                                 ws, stream);
  }
  if (e != hipSuccess) return launch_status(e);
  return launch_status(tsd::launch_topk_finish(
      a->scores, a->score_stride, rows, a->row_lens_out,
      static_cast<int>(max_len), k, idx, count, ws, stream));
}

size_t topk_select_workspace_bytes(int rows, int max_len, int k) {
  if (rows <= 0 || max_len < 0) return 0;
  return tsd::topk_workspace(rows, max_len, k);
}

int topk_select(const float* scores, int64_t stride, int rows,
                const int32_t* row_lens, int max_len, int k, int32_t* idx,
                int32_t* count, void* ws, size_t ws_bytes, hipStream_t stream) {
  return topk_select_ex(scores, stride, rows, row_lens, max_len, k, idx, count,
                        ws, ws_bytes, 0, stream);
}

int topk_select_ex(const float* scores, int64_t stride, int rows,
                   const int32_t* row_lens, int max_len, int k, int32_t* idx,
                   int32_t* count, void* ws, size_t ws_bytes, int flags,
                   hipStream_t stream) {
  const int rc = validate_topk(scores, stride, rows, row_lens, max_len, k,
                               idx, ws, ws_bytes);
  if (rc) return rc;
  if (flags & ~TSD_TOPK_WS_ZEROED) return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  return launch_status(tsd::launch_topk(scores, stride, rows, row_lens,
                                        max_len, k, idx, count, ws,
                                        (flags & TSD_TOPK_WS_ZEROED) != 0,
                                        stream));
}

int topk_merge_sharded(const float* scores, int64_t stride,
                       const int32_t* idx_local, const int32_t* count_local,
                       int W, int rows, int kl, int k, int32_t* idx,
                       int32_t* count, hipStream_t stream) {
  if (W < 1 || rows < 0 || kl < 1 || stride < 1) return TSD_E_SHAPE;
  if (k < 1 || k > TSD_MAX_TOPK) return TSD_E_K;
  if (W > 16 || rows > 65535 || kl > TSD_MAX_TOPK ||
      static_cast<int64_t>(W) * kl > tsd::topk_merge_max_candidates() ||
      static_cast<int64_t>(W) * stride > std::numeric_limits<int32_t>::max())
    return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  if (!scores || !idx_local || !count_local || !idx) return TSD_E_NULL;
  return launch_status(tsd::launch_topk_merge_sharded(
      scores, stride, idx_local, count_local, W, rows, kl, k, idx, count,
      stream));
}

static bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int kv_append(const tsd_append_args* a, hipStream_t stream) {
  if (!a) return TSD_E_NULL;
  if (a->abi_version != TSD_ABI_VERSION) return TSD_E_ABI;
  if (a->page_size != TSD_PAGE_SIZE) return TSD_E_PAGE_SIZE;
  if (a->B < 0 || a->max_new < 0 || a->pt_stride < 1 || a->num_pages < 0)
    return TSD_E_SHAPE;
  if (a->B > 65535) return TSD_E_UNSUPPORTED;
  const bool kv = a->k_new != nullptr, label = a->channel_idx != nullptr,
             index = a->index_k_new != nullptr;
  if (kv || label) {
    if (a->new_dtype != TSD_BF16 && a->new_dtype != TSD_FP16) return TSD_E_DTYPE;
    if (a->H_kv < 1 || a->D < 1) return TSD_E_SHAPE;
    if (a->D != TSD_HEAD_DIM || a->H_kv * a->D > 4096) return TSD_E_UNSUPPORTED;
  }
  if (kv) {
    if (a->kv_dtype != a->new_dtype && a->kv_dtype != TSD_FP8_E4M3)
      return TSD_E_DTYPE;
    if (!a->v_new || !a->k_pool || !a->v_pool) return TSD_E_NULL;
    if (a->kv_dtype == TSD_FP8_E4M3 && (!a->k_scale || !a->v_scale))
      return TSD_E_NULL;
    if (!aligned16(a->k_new) || !aligned16(a->v_new) ||
        !aligned16(a->k_pool) || !aligned16(a->v_pool))
      return TSD_E_UNSUPPORTED;
  }
  if (label) {
    if (!a->k_new || !a->label_pool) return TSD_E_NULL;
    if (a->r < 1) return TSD_E_SHAPE;
    if (a->r > a->D) return TSD_E_UNSUPPORTED;
  }
  if (index) {
    if (a->index_dtype != TSD_BF16 && a->index_dtype != TSD_FP16 &&
        a->index_dtype != TSD_F32)
      return TSD_E_DTYPE;
    if (!a->index_k_pool) return TSD_E_NULL;
    if (a->D_i != TSD_HEAD_DIM) return TSD_E_UNSUPPORTED;
    if (!aligned16(a->index_k_new) || !aligned16(a->index_k_pool))
      return TSD_E_UNSUPPORTED;
  }
  if (a->B == 0 || a->max_new == 0 || !(kv || label || index)) return TSD_OK;
  if (!a->page_table || !a->positions || !a->n_new) return TSD_E_NULL;
  return launch_status(tsd::launch_kv_append(*a, stream));
}

static bool block_size_ok(int bs) {
  return bs >= 1 && bs <= TSD_PAGE_SIZE && (bs & (bs - 1)) == 0;
}

int index_k_compress(const tsd_compress_args* a, hipStream_t stream) {
  if (!a) return TSD_E_NULL;
  if (a->abi_version != TSD_ABI_VERSION) return TSD_E_ABI;
  if (a->page_size != TSD_PAGE_SIZE) return TSD_E_PAGE_SIZE;
  if (a->B < 0 || a->max_blocks < 0 || a->pt_stride < 1 ||
      a->cpt_stride < 1 || a->num_pages < 0 || a->num_cpages < 0)
    return TSD_E_SHAPE;
  if (!block_size_ok(a->block_size)) return TSD_E_UNSUPPORTED;
  if (a->D_i != TSD_HEAD_DIM || a->B > 65535) return TSD_E_UNSUPPORTED;
  if (a->B == 0 || a->max_blocks == 0) return TSD_OK;
  if (!a->index_k_pool || !a->page_table || !a->seq_lens || !a->ck_pool ||
      !a->cpage_table)
    return TSD_E_NULL;
  if (!aligned16(a->index_k_pool) || !aligned16(a->ck_pool)) return TSD_E_UNSUPPORTED;
  return launch_status(tsd::launch_index_k_compress(*a, stream));
}

int expand_blocks(const int32_t* sel, const int32_t* count, int rows, int kb,
                  int block_size, const int32_t* row_lens, int kt,
                  int32_t* tok, int32_t* tok_count, hipStream_t stream) {
  if (rows < 0) return TSD_E_SHAPE;
  if (kb < 1 || kb > TSD_MAX_TOPK || kt < 1 || kt > TSD_MAX_TOPK) return TSD_E_K;
  if (!block_size_ok(block_size) || rows > 65535) return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  if (!sel || !count || !row_lens || !tok) return TSD_E_NULL;
  return launch_status(tsd::launch_expand_blocks(
      sel, count, rows, kb, block_size, row_lens, kt, tok, tok_count, stream));
}

int sparse_gqa_decode(const tsd_attn_args* a, hipStream_t stream) {
  const int rc = validate_attn(a);
  if (rc) return rc;
  if (a->B == 0) return TSD_OK;
  return launch_status(tsd::launch_sparse_gqa(*a, stream));
}

int lse_merge(const float* o_part, const float* lse_part, int rows, int C,
              int D, float* out, float* out_lse, hipStream_t stream) {
  const int rc = validate_merge(o_part, lse_part, rows, C, D, out);
  if (rc) return rc;
  if (rows == 0) return TSD_OK;
  return launch_status(
      tsd::launch_lse_merge(o_part, lse_part, rows, C, D, out, out_lse, stream));
}

const char* tsd_strerror(int status) {
  switch (status) {
    case TSD_OK: return "success";
    case TSD_E_NULL: return "a required pointer is NULL";
    case TSD_E_DTYPE: return "unsupported or inconsistent element encoding";
    case TSD_E_SHAPE: return "invalid size or stride";
    case TSD_E_PAGE_SIZE: return "page_size must be 64";
    case TSD_E_GQA: return "H_q must be a multiple of H_kv and H_sel 1 or H_kv";
    case TSD_E_K: return "top_k must lie in [1, 4096]";
    case TSD_E_CHUNKS: return "chunks must lie in [1, 64]";
    case TSD_E_WORKSPACE: return "workspace missing or too small";
    case TSD_E_UNSUPPORTED: return "configuration not supported by this library";
    case TSD_E_MODE: return "unknown score mode";
    case TSD_E_ABI: return "argument struct from another ABI version";
    case TSD_E_SCRATCH:
      return "selection needs more than the built-in scratch of "
             "topk_select_noalloc";
    default:
      return status > 0 ? "HIP launch failed (status is the hipError_t)"
                        : "unknown status";
  }
}

int tsd_abi_version(void) { return TSD_ABI_VERSION; }
const char* tsd_source_sha256(void) { return TSD_SOURCE_SHA256; }
size_t tsd_sizeof_score_args(void) { return sizeof(tsd_score_args); }
size_t tsd_sizeof_attn_args(void) { return sizeof(tsd_attn_args); }
size_t tsd_sizeof_append_args(void) { return sizeof(tsd_append_args); }
size_t tsd_sizeof_compress_args(void) { return sizeof(tsd_compress_args); }

}  // extern "C"
