// Internal launchers of libtsd.so (host side). Arguments have already been
// validated by the C-ABI entry points when these run.
#pragma once

#include <hip/hip_runtime.h>

#include "tsd.h"

namespace tsd {

// topk_ws (optional): a cleared top-k workspace for rows = B * rows_per_req;
// the scan then also builds each row's digit-1 histograms (rows with
// n <= hist_k skip them).
hipError_t launch_qsa_scan(const tsd_score_args& a, hipStream_t s,
                           void* topk_ws = nullptr, int hist_k = 0);
hipError_t launch_ds_scan(const tsd_score_args& a, hipStream_t s);

size_t topk_workspace(int rows, int max_len, int k);
int topk_max_len();  // largest max_len topk_select accepts
// The stages of launch_topk: clear the histograms, histogram digit 1, then
// filter + resolve (the first two may be replaced by a scan that builds
// the digit-1 histogram itself).
hipError_t launch_topk_clear(void* ws, int rows, hipStream_t s);
hipError_t launch_topk_hist1(const float* scores, int64_t stride, int rows,
                             const int32_t* row_lens, int max_len, int k,
                             void* ws, hipStream_t s);
hipError_t launch_topk_finish(const float* scores, int64_t stride, int rows,
                              const int32_t* row_lens, int max_len, int k,
                              int32_t* idx, int32_t* count, void* ws,
                              hipStream_t s);
// Rows of at most 32,768 elements (24,576 unless there are many rows or k
// is a large share of a row): the whole selection in one launch, one
// workgroup per row (no workspace).
bool topk_small_fits(int max_len, int rows, int k);
hipError_t launch_topk_small(const float* scores, int64_t stride, int rows,
                             const int32_t* row_lens, int max_len, int k,
                             int32_t* idx, int32_t* count, hipStream_t s);
hipError_t launch_topk(const float* scores, int64_t stride, int rows,
                       const int32_t* row_lens, int max_len, int k,
                       int32_t* idx, int32_t* count, void* ws, bool zeroed,
                       hipStream_t s);

int topk_merge_max_candidates();  // W * kl bound of topk_merge_sharded
hipError_t launch_topk_merge_sharded(const float* scores, int64_t stride,
                                     const int32_t* idx_local,
                                     const int32_t* count_local, int W,
                                     int rows, int kl, int k, int32_t* idx,
                                     int32_t* count, hipStream_t s);

hipError_t launch_kv_append(const tsd_append_args& a, hipStream_t s);
hipError_t launch_index_k_compress(const tsd_compress_args& a, hipStream_t s);
hipError_t launch_expand_blocks(const int32_t* sel, const int32_t* count,
                                int rows, int kb, int Bs,
                                const int32_t* row_lens, int kt, int32_t* tok,
                                int32_t* tok_count, hipStream_t s);

hipError_t launch_sparse_gqa(const tsd_attn_args& a, hipStream_t s);

hipError_t launch_lse_merge(const float* o_part, const float* lse_part,
                            int rows, int C, int D, float* out,
                            float* out_lse, hipStream_t s);

}  // namespace tsd
