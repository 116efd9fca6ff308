// Double-sparsity label scan ("Support double sparsity", sglang PR #1459:
// the label cache holds K at r heavy channels per head; decode scores every
// cached token with it and keeps the heavy tokens):
//   s[b*H_kv+g][t] = sum_j qs[g][j] * label[slot(b,t)][g][j],
//   qs[g][j]       = sum of the group's query heads at channel chan[g][j].
//
// About 1 flop per byte, so this is a plain bandwidth-bound VALU pass. One
// workgroup owns one 64-token page of one request and covers every KV head:
// the page's labels ([64][H_kv][r] 16-bit values) are one contiguous block,
// read with 16-byte loads in order. Scores go through LDS so each
// (request, head) row receives 64 contiguous floats.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHeadChan = 4096;  // H_kv * r held in LDS
constexpr int kMaxScoreLds = 64 * 128;

__global__ __launch_bounds__(kThreads) void ds_scan_kernel(
    const uint16_t* __restrict__ q, bool is_bf16, int H_q, int H_kv, int D,
    const int32_t* __restrict__ chan, int r,
    const uint16_t* __restrict__ label, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const int32_t* __restrict__ seq_lens,
    int64_t num_pages, float* __restrict__ scores, int64_t score_stride,
    int32_t* __restrict__ row_lens_out) {
  __shared__ float qs[kMaxHeadChan];
  __shared__ float sc[kMaxScoreLds];
  const int b = blockIdx.y;
  const int64_t p = blockIdx.x;
  int64_t n = clamp_len(seq_lens[b], pt_stride * kPage);
  n = clamp_len(n, score_stride);
  if (p == 0 && row_lens_out)
    for (int g = threadIdx.x; g < H_kv; g += kThreads)
      row_lens_out[static_cast<int64_t>(b) * H_kv + g] = static_cast<int32_t>(n);
  if (p * kPage >= n) return;
  const int32_t page = page_table[static_cast<int64_t>(b) * pt_stride + p];
  const bool valid = page >= 0 && page < num_pages;
  const int G = H_q / H_kv;
  const int hc = H_kv * r;

  // group query at the heavy channels
  for (int i = threadIdx.x; i < hc; i += kThreads) {
    const int g = i / r;
    const int c = chan[i];
    float acc = 0.f;
    if (c >= 0 && c < D) {
      const uint16_t* qb = q + (static_cast<int64_t>(b) * H_q + g * G) * D + c;
      for (int h = 0; h < G; ++h) acc += half_to_f32(qb[h * D], is_bf16);
    }
    qs[i] = acc;
  }
  __syncthreads();

  const int items = kPage * H_kv;  // (slot s, head g), g fastest
  if (valid) {
    const uint16_t* base = label + static_cast<int64_t>(page) * kPage * hc;
    if ((r & 7) == 0) {
      const int vecs = r >> 3;  // 16-byte vectors per label
      for (int it = threadIdx.x; it < items; it += kThreads) {
        const int g = it % H_kv;
        const uint4* src = reinterpret_cast<const uint4*>(base) +
                           static_cast<int64_t>(it) * vecs;
        const float* qg = qs + g * r;
        float acc = 0.f;
        for (int v = 0; v < vecs; ++v) {
          const uint4 x = src[v];
          const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc += qg[8 * v + 2 * e] *
                   half_to_f32(static_cast<uint16_t>(wds[e] & 0xFFFF), is_bf16);
            acc += qg[8 * v + 2 * e + 1] *
                   half_to_f32(static_cast<uint16_t>(wds[e] >> 16), is_bf16);
          }
        }
        sc[g * kPage + it / H_kv] = acc;
      }
    } else {
      for (int it = threadIdx.x; it < items; it += kThreads) {
        const int g = it % H_kv;
        const uint16_t* src = base + static_cast<int64_t>(it) * r;
        const float* qg = qs + g * r;
        float acc = 0.f;
        for (int j = 0; j < r; ++j) acc += qg[j] * half_to_f32(src[j], is_bf16);
        sc[g * kPage + it / H_kv] = acc;
      }
    }
  }
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int g = it / kPage, s = it % kPage;
    const int64_t t = p * kPage + s;
    if (t < n)
      scores[(static_cast<int64_t>(b) * H_kv + g) * score_stride + t] =
          valid ? sc[it] : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_ds_scan(const tsd_score_args& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(a.pt_stride), static_cast<uint32_t>(a.B));
  hipLaunchKernelGGL(ds_scan_kernel, grid, dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(a.q), a.q_dtype == TSD_BF16,
                     a.H_q, a.H_kv, a.D, a.channel_idx, a.r,
                     static_cast<const uint16_t*>(a.label_pool), a.page_table,
                     a.pt_stride, a.seq_lens, a.num_pages, a.scores,
                     a.score_stride, a.row_lens_out);
  return hipGetLastError();
}

}  // namespace tsd
