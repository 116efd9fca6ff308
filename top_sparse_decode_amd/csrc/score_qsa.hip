// QSA-style index-K scan:
//   s[i][t] = sum_h w[i][h] * max(0, sum_d qi[i][h][d] * ki[slot(b,t)][d]).
// The indexer scores every cached token of the request with a 128-dim FP8
// index key and many index heads ("Context parallelism for QSA attention and
// the sparse indexer", Motivation: index-K store, score, top-k per row).
//
// Per key the contraction is 16 heads x 128 dims = 2048 MACs over 128 bytes,
// 32 flop per HBM byte: more than the FP32 vector units can sustain at HBM
// speed, so each 16-key tile is one v_mfma_scale_f32_16x16x128_f8f6f4 with the
// index heads as M, the keys as N and the 128 dims as K. The kernel stays a
// single streaming pass over the index-K pages: every byte is read once, the
// query rows sit in registers for the whole scan.
//
// Work split: one wave owns one query row and a run of consecutive 64-token
// pages; a page is 4 MFMA tiles of 16 keys. The 16x16 f32 result gives lane
// l the dots of key (l % 16) with heads 4*(l/16) .. 4*(l/16)+3; the weighted
// ReLU is applied per lane and a 3-shuffle reduce-scatter over the 4 lane
// groups leaves lane l with the full score of key l of the page, so a page
// stores 256 contiguous bytes of scores.
#include "device_common.h"
#include "launch.h"
#include "topk_digits.h"

namespace tsd {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kPagesPerWave = 4;
constexpr int kDi = 128;

// 32 bytes of one 128-byte FP8 row in the lane's MFMA operand slot:
// bytes [16*kb, 16*kb + 16) and [64 + 16*kb, 64 + 16*kb + 16). Index heads
// and index keys use the same mapping, so the K-dimension pairing inside the
// instruction matches dims of q with the same dims of k.
TSD_DEVICE v8i load_row_slice(const uint8_t* row, int kb) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * kb);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + 64 + 16 * kb);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

TSD_DEVICE v4f mfma_fp8(v8i a, v8i b) {
  v4f c = {0.f, 0.f, 0.f, 0.f};
  // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0,
                                                          127, 0, 127);
}

// HIST: also accumulate the first top-k radix digit of every written score
// into hist1[row][4096] (LDS-privatised per workgroup, flushed with integer
// atomics). The launch then gives each row a multiple of 4 waves so that a
// workgroup never spans two rows, and no wave leaves before the barriers.
template <bool HIST>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void qsa_scan_kernel(
    const uint8_t* __restrict__ index_q, const float* __restrict__ index_w,
    const uint8_t* __restrict__ index_k, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_pos, int64_t num_pages, int rows,
    int rows_per_req, int H_i, int waves_per_row, float* __restrict__ scores,
    int64_t score_stride, int32_t* __restrict__ row_lens_out,
    uint32_t* __restrict__ hist1, int hist_k) {
  __shared__ uint32_t hist_s[HIST ? kTopkBins1 : 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int row = wave / waves_per_row;
  const bool row_ok = row < rows;
  const int chunk = wave - row * waves_per_row;
  const int b = row_ok ? row / rows_per_req : 0;

  int64_t n = 0;
  if (row_ok) {
    n = seq_lens[b];
    if (q_pos) {
      const int64_t p1 = static_cast<int64_t>(q_pos[row]) + 1;
      n = p1 < n ? p1 : n;
    }
    n = clamp_len(n, pt_stride * kPage);
    n = clamp_len(n, score_stride);
    if (chunk == 0 && lane == 0 && row_lens_out)
      row_lens_out[row] = static_cast<int32_t>(n);
  }
  const int64_t page0 = static_cast<int64_t>(chunk) * kPagesPerWave;
  const bool active = row_ok && page0 * kPage < n;
  const bool do_hist = HIST && row_ok && n > hist_k;
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kTopkBins1; i += kWavesPerBlock * kWave)
      hist_s[i] = 0u;
    __syncthreads();
  } else {
    if (!active) return;
  }

  if (active) {
    const int col = lane & 15;  // MFMA row (head) for A, column (key) for B
    const int kb = lane >> 4;   // which 32-byte slice of the 128 dims

    // A operand: index head `col` of this row (zero for padded heads).
    v8i qa = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < H_i)
      qa = load_row_slice(
          index_q + (static_cast<int64_t>(row) * H_i + col) * kDi, kb);
    // Weights of the 4 heads whose dots this lane receives.
    float w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * kb + v;
      w[v] = h < H_i ? index_w[static_cast<int64_t>(row) * H_i + h] : 0.f;
    }

    const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride;
    float* out = scores + static_cast<int64_t>(row) * score_stride;

    // All of the wave's pages are requested before any is consumed (32 KB
    // of loads in flight per wave), then each page is contracted and
    // reduced.
    v8i kt[kPagesPerWave][4];
    bool live[kPagesPerWave], valid[kPagesPerWave];
#pragma unroll
    for (int pp = 0; pp < kPagesPerWave; ++pp) {
      const int64_t p = page0 + pp;
      live[pp] = p * kPage < n;
      const int32_t page = live[pp] ? pt[p] : -1;
      valid[pp] = page >= 0 && page < num_pages;
      const uint8_t* base =
          index_k + static_cast<int64_t>(valid[pp] ? page : 0) * kPage * kDi;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kt[pp][i] = valid[pp] ? load_row_slice(base + (16 * i + col) * kDi, kb)
                              : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int pp = 0; pp < kPagesPerWave; ++pp) {
      if (!live[pp]) break;
      float part[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4f d = mfma_fp8(qa, kt[pp][i]);
        part[i] = w[0] * fmaxf(d[0], 0.f) + w[1] * fmaxf(d[1], 0.f) +
                  w[2] * fmaxf(d[2], 0.f) + w[3] * fmaxf(d[3], 0.f);
      }
      // Reduce-scatter over the 4 lane groups g = lane / 16: lane (g, j)
      // ends with sum_g' part[g](g', j) = score of key 16*g + j of the page.
      const int g = kb;
      const bool upper = g >= 2;
      const float x_send = upper ? part[0] : part[2];
      const float y_send = upper ? part[1] : part[3];
      const float x_recv = __shfl_xor(x_send, 32, kWave);
      const float y_recv = __shfl_xor(y_send, 32, kWave);
      const float u = (upper ? part[2] : part[0]) + x_recv;
      const float v = (upper ? part[3] : part[1]) + y_recv;
      const bool odd = g & 1;
      const float s_send = odd ? u : v;
      const float s_recv = __shfl_xor(s_send, 16, kWave);
      const float sc = valid[pp] ? (odd ? v : u) + s_recv : -__builtin_inff();

      const int64_t t = (page0 + pp) * kPage + lane;
      if (t < n) {
        out[t] = sc;
        if (do_hist) atomicAdd(&hist_s[topk_digit1(order_key(sc))], 1u);
      }
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    if (do_hist) {  // uniform: the workgroup lies in one row
      uint32_t* g = hist1 + static_cast<int64_t>(row) * kTopkBins1;
      for (int i = threadIdx.x; i < kTopkBins1; i += kWavesPerBlock * kWave) {
        const uint32_t c = hist_s[i];
        if (c) atomicAdd(g + i, c);
      }
    }
  }
}

}  // namespace

hipError_t launch_qsa_scan(const tsd_score_args& a, hipStream_t s,
                           uint32_t* hist1, int hist_k) {
  const int rows = a.B * a.rows_per_req;
  if (rows == 0) return hipSuccess;
  int64_t waves_per_row = (a.pt_stride + kPagesPerWave - 1) / kPagesPerWave;
  if (hist1)  // whole workgroups per row
    waves_per_row = (waves_per_row + kWavesPerBlock - 1) / kWavesPerBlock *
                    kWavesPerBlock;
  const int64_t waves = waves_per_row * rows;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  auto kern = hist1 ? qsa_scan_kernel<true> : qsa_scan_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)),
                     dim3(kWavesPerBlock * kWave), 0, s, a.index_q, a.index_w,
                     a.index_k_pool, a.page_table, a.pt_stride, a.seq_lens,
                     a.q_pos, a.num_pages, rows, a.rows_per_req, a.H_i,
                     static_cast<int>(waves_per_row), a.scores,
                     a.score_stride, a.row_lens_out, hist1, hist_k);
  return hipGetLastError();
}

}  // namespace tsd
