// Exact global top-k from page-owner shards ("QSA cache sharding", sglang
// PR #43527, Distributed QSA execution: every rank selects over the pages it
// owns, the (score, token id) candidates are exchanged, and one exact top-k
// with token-id tie-breaking is formed from their union).
//
// Shard w owns the logical pages p with p % W == w of a row; its local token
// u is the global token ((u / 64) * W + w) * 64 + u % 64. The global top-k
// is contained in the union of the shards' local top-k lists (a shard holds
// at most k of the global winners, and within a shard the global ranking
// restricted to its tokens is its local ranking), so merging the candidates
// is exact.
//
// One workgroup per row holds the W * kl candidates in registers (16 per
// thread at most). The k-th largest order-preserving score key T is found
// by the same 12/10/10-bit radix select as topk_select; when more
// candidates tie at T than are kept, the kept ties are the lowest global
// tokens, found by a second radix select on the inverted tokens of the
// ties. The kept tokens are then marked in an LDS bitmap over the row's
// global tokens, segment by segment, and a popcount scan writes them in
// ascending order.
#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

namespace tsd {
namespace {

constexpr int kMT = 1024;                 // threads per row
constexpr int kMaxCand = 16384;           // W * kl per row
constexpr int kPer = kMaxCand / kMT;      // candidates per thread
// tokens per bitmap segment: a 1,048,576-token row in one pass (128 KB of
// LDS beside the 16 KB histogram; 512K-token segments took 4.2 us more for
// such a row, the second segment's clear, marks, scan and barriers)
constexpr int kSegBits = 1 << 20;
constexpr int kSegWords = kSegBits / 32;

// The c-th largest (1 <= c <= count of valid values) of the values v[i]
// whose bit i of okb is set, held kPer per thread across the workgroup
// (flags as bits of one word keep them out of scalar lane masks): returns the value
// and the number of values strictly above it. Three radix digits of 12, 10
// and 10 bits, each counted in the LDS histogram `hist` (4096 words,
// 16-byte aligned) and resolved by pick_bin.
TSD_DEVICE void select_kth(const uint32_t (&v)[kPer], uint32_t okb,
                           uint32_t c, uint32_t* hist, uint32_t* lds,
                           BinPick* pick, uint32_t& value, uint32_t& above) {
  for (int i = threadIdx.x; i < kTopkBins1; i += kMT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((okb >> i) & 1u) atomicAdd(&hist[v[i] >> 20], 1u);
  __syncthreads();
  const BinPick p1 = pick_bin<kTopkBins1, kMT>(hist, c, lds, pick);
  for (int i = threadIdx.x; i < kTopkBins2; i += kMT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (((okb >> i) & 1u) && (v[i] >> 20) == p1.bin)
      atomicAdd(&hist[(v[i] >> 10) & 1023u], 1u);
  __syncthreads();
  const BinPick p2 = pick_bin<kTopkBins2, kMT>(hist, c - p1.above, lds, pick);
  const uint32_t pre = (p1.bin << 10) | p2.bin;
  for (int i = threadIdx.x; i < kTopkBins3; i += kMT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (((okb >> i) & 1u) && (v[i] >> 10) == pre) atomicAdd(&hist[v[i] & 1023u], 1u);
  __syncthreads();
  const BinPick p3 =
      pick_bin<kTopkBins3, kMT>(hist, c - p1.above - p2.above, lds, pick);
  value = (pre << 10) | p3.bin;
  above = p1.above + p2.above + p3.above;
}

// Workgroup sum of one value per thread (every thread gets the total).
TSD_DEVICE uint32_t block_sum(uint32_t x, uint32_t* lds) {
  x = wave_sum_u32(x);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < kMT / kWave; ++i) t += lds[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kMT) void topk_merge_sharded_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ idx_local,
    const int32_t* __restrict__ count_local, int W, int rows, int kl, int k,
    int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ __align__(16) uint32_t hist[kTopkBins1];
  __shared__ __align__(16) uint32_t bits[kSegWords];
  __shared__ uint32_t lds[kMT / kWave + 1];
  __shared__ BinPick pick;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;

  // candidates e = tid + i * kMT, entry j of shard w's list (e = w * kl + j)
  uint32_t key[kPer], tok[kPer];
  int32_t u[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kMT;
    u[i] = -1;
    if (e < W * kl) {
      const int w = e / kl, j = e - w * kl;
      const int64_t sr = static_cast<int64_t>(w) * rows + row;
      if (j < count_local[sr]) u[i] = idx_local[sr * kl + j];
    }
  }
  uint32_t okb = 0;  // bit i: candidate i of this thread is valid
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kMT;
    const int w = e / kl;
    const bool ok = u[i] >= 0 && u[i] < stride;
    key[i] = 0u;
    tok[i] = 0u;
    if (ok) {
      const int64_t sr = static_cast<int64_t>(w) * rows + row;
      key[i] = order_key(scores[sr * stride + u[i]]);
      tok[i] = static_cast<uint32_t>(
          (static_cast<int64_t>(u[i] / kPage) * W + w) * kPage + u[i] % kPage);
      okb |= 1u << i;
    }
  }
  const uint32_t total = block_sum(__popc(okb), lds);
  const uint32_t m = total < static_cast<uint32_t>(k) ? total : k;

  // kept: key > T, plus the `need` lowest tokens among key == T
  uint32_t keptb = okb;
  if (m < total) {
    uint32_t T, above;
    select_kth(key, okb, m, hist, lds, &pick, T, above);
    const uint32_t need = m - above;
    uint32_t tieb = 0, inv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      tieb |= static_cast<uint32_t>(((okb >> i) & 1u) && key[i] == T) << i;
      inv[i] = ~tok[i];
    }
    const uint32_t ties = block_sum(__popc(tieb), lds);
    uint32_t G = 0u;  // kept ties: inverted token >= G (all if ties == need)
    if (ties > need) {
      uint32_t gabove;
      select_kth(inv, tieb, need, hist, lds, &pick, G, gabove);
    }
    keptb = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      keptb |= static_cast<uint32_t>(((okb >> i) & 1u) &&
                                     (key[i] > T || (key[i] == T && inv[i] >= G)))
               << i;
  }

  // ascending output through a bitmap over the row's global tokens
  uint32_t tmax = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    tmax = ((keptb >> i) & 1u) && tok[i] + 1 > tmax ? tok[i] + 1 : tmax;
  tmax = wave_butterfly(tmax, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  if ((tid & (kWave - 1)) == 0) lds[tid >> 6] = tmax;
  __syncthreads();
  uint32_t span = 0;
#pragma unroll
  for (int i = 0; i < kMT / kWave; ++i) span = lds[i] > span ? lds[i] : span;
  __syncthreads();
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  uint32_t written = 0;
  for (uint32_t seg = 0; seg < span; seg += kSegBits) {
    for (int i = tid; i < kSegWords / 4; i += kMT)  // 16-byte stores
      reinterpret_cast<uint4*>(bits)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (((keptb >> i) & 1u) && tok[i] >= seg &&
          tok[i] - seg < static_cast<uint32_t>(kSegBits)) {
        const uint32_t r = tok[i] - seg;
        atomicOr(&bits[r >> 5], 1u << (r & 31));
      }
    __syncthreads();
    constexpr int wpt = kSegWords / kMT;
    uint32_t wd[wpt], pc = 0;
#pragma unroll
    for (int j = 0; j < wpt; ++j) {
      wd[j] = bits[tid * wpt + j];
      pc += __popc(wd[j]);
    }
    uint32_t pos = written + block_exclusive_scan<kMT>(pc, lds);
#pragma unroll
    for (int j = 0; j < wpt; ++j) {
      uint32_t word = wd[j];
      while (word) {
        const int b = __ffs(word) - 1;
        word &= word - 1;
        if (pos < m) out[pos] = static_cast<int32_t>(seg + (tid * wpt + j) * 32 + b);
        ++pos;
      }
    }
    if (tid == kMT - 1) lds[kMT / kWave] = pos;
    __syncthreads();
    written = lds[kMT / kWave];
    __syncthreads();
  }
  for (uint32_t j = m + tid; j < static_cast<uint32_t>(k); j += kMT) out[j] = -1;
  if (tid == 0 && count) count[row] = static_cast<int32_t>(m);
}

}  // namespace

int topk_merge_max_candidates() { return kMaxCand; }

hipError_t launch_topk_merge_sharded(const float* scores, int64_t stride,
                                     const int32_t* idx_local,
                                     const int32_t* count_local, int W,
                                     int rows, int kl, int k, int32_t* idx,
                                     int32_t* count, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_merge_sharded_kernel, dim3(static_cast<uint32_t>(rows)),
                     dim3(kMT), 0, s, scores, stride, idx_local, count_local, W,
                     rows, kl, k, idx, count);
  return hipGetLastError();
}

}  // namespace tsd
