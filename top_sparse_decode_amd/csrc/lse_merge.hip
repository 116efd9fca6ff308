// FP32 log-sum-exp merge of chunk partials ("QSA cache sharding", sglang PR
// #43527, Distributed QSA execution: owner-side partial outputs are combined
// with FP32 log-sum-exp normalisation):
//   M = max_c lse_c, W = sum_c exp(lse_c - M),
//   out = sum_c exp(lse_c - M) * o_c / W, out_lse = M + log W.
// One workgroup per (row, 128 output dimensions). Every thread owns one
// output dimension and issues the loads of its first 16 chunk partials at
// once, while the first wave turns the row's C <= 64 LSEs (one per lane)
// into normalised weights in LDS, so the merge is a single memory round
// trip for C <= 16.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 128;
constexpr int kPre = 16;  // chunk partials each thread loads up front

__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    int C, int D, float* __restrict__ out, float* __restrict__ out_lse) {
  __shared__ float w_s[64];
  __shared__ float empty_s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int d = blockIdx.y * kThreads + tid;
  const float* op = o_part + static_cast<int64_t>(row) * C * D + d;
  float pre[kPre];  // partials of chunks 0 .. kPre-1, loaded before the weights
#pragma unroll
  for (int c = 0; c < kPre; ++c)
    pre[c] = d < D && c < C ? op[static_cast<int64_t>(c) * D] : 0.f;
  if (tid < kWave) {
    const float* lse = lse_part + static_cast<int64_t>(row) * C;
    const float mine = tid < C ? lse[tid] : -__builtin_inff();
    const float M = wave_max(mine);
    const bool empty = M == -__builtin_inff();
    const float e = (!empty && tid < C) ? expf(mine - M) : 0.f;
    const float W = wave_sum(e);
    if (tid < C) w_s[tid] = empty ? 0.f : e / W;
    if (tid == 0) {
      empty_s = empty ? 1.f : 0.f;
      if (out_lse && blockIdx.y == 0)
        out_lse[row] = empty ? -__builtin_inff() : M + logf(W);
    }
  }
  __syncthreads();
  if (d >= D) return;
  float acc = 0.f;
  if (empty_s == 0.f) {
#pragma unroll
    for (int c = 0; c < kPre; ++c)
      if (c < C) acc += w_s[c] * pre[c];
#pragma unroll 8
    for (int c = kPre; c < C; ++c) acc += w_s[c] * op[static_cast<int64_t>(c) * D];
  }
  out[static_cast<int64_t>(row) * D + d] = acc;
}

}  // namespace

hipError_t launch_lse_merge(const float* o_part, const float* lse_part,
                            int rows, int C, int D, float* out,
                            float* out_lse, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(rows),
            static_cast<uint32_t>((D + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(lse_merge_kernel, grid, dim3(kThreads), 0, s, o_part,
                     lse_part, C, D, out, out_lse);
  return hipGetLastError();
}

}  // namespace tsd
