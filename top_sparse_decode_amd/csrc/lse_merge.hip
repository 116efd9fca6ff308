// FP32 log-sum-exp merge of chunk partials ("QSA cache sharding", sglang PR
// #43527, Distributed QSA execution: owner-side partial outputs are combined
// with FP32 log-sum-exp normalisation):
//   M = max_c lse_c, W = sum_c exp(lse_c - M),
//   out = sum_c exp(lse_c - M) * o_c / W, out_lse = M + log W.
// One wave per row; each lane owns D/64 (rounded up) output dimensions, the
// per-chunk weights are computed once per lane from the row's LSEs.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    int rows, int C, int D, float* __restrict__ out,
    float* __restrict__ out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* lse = lse_part + static_cast<int64_t>(row) * C;
  // max over chunks (C <= 64: one chunk per lane)
  const float mine = lane < C ? lse[lane] : -__builtin_inff();
  const float M = wave_max(mine);
  float* o = out + static_cast<int64_t>(row) * D;
  if (M == -__builtin_inff()) {
    for (int d = lane; d < D; d += kWave) o[d] = 0.f;
    if (lane == 0 && out_lse) out_lse[row] = -__builtin_inff();
    return;
  }
  const float wl = lane < C ? expf(mine - M) : 0.f;
  const float W = wave_sum(wl);
  const float inv = 1.f / W;
  const float* op = o_part + static_cast<int64_t>(row) * C * D;
  for (int d = lane; d < D; d += kWave) {
    float acc = 0.f;
    for (int c = 0; c < C; ++c) {
      const float a = __shfl(wl, c, kWave);
      if (a != 0.f) acc += a * op[static_cast<int64_t>(c) * D + d];
    }
    o[d] = acc * inv;
  }
  if (lane == 0 && out_lse) out_lse[row] = M + logf(W);
}

}  // namespace

hipError_t launch_lse_merge(const float* o_part, const float* lse_part,
                            int rows, int C, int D, float* out,
                            float* out_lse, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(lse_merge_kernel, dim3(blocks), dim3(kThreads), 0, s,
                     o_part, lse_part, rows, C, D, out, out_lse);
  return hipGetLastError();
}

}  // namespace tsd
