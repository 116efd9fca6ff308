// Exact top-k per row with the lowest-index tie-break ("QSA cache sharding",
// sglang PR #43527, Distributed QSA execution: an exact Top-K whose ties are
// broken deterministically by token ID), output in ascending index order.
//
// Scores are mapped to order-preserving 32-bit keys (-0 folded onto +0).
// The threshold key T (the k-th largest) is found by an MSD radix select in
// three digit passes (11 + 11 + 10 bits); each pass builds per-workgroup LDS
// histograms of the rows' elements that match the prefix found so far and
// adds them into one global histogram per row with integer atomics, so the
// counts -- and everything derived from them -- are deterministic. Then each
// wave counts, over its 1024-element slice, the keys above T and equal to T;
// a final pass turns those counts into exclusive offsets and every wave
// compacts its slice in index order with 64-lane ballots: keys above T are
// kept, keys equal to T are kept while their global tie rank is below the
// number of ties still needed. Rows with n <= k keep every index.
//
// Every pass uses the same grid (row, 4096-element chunk), so a chunk's
// scores are re-read by the same XCD and tend to hit its L2.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSub = 1024;                      // elements per wave slice
constexpr int kChunk = kSub * kWavesPerBlock;   // elements per workgroup
constexpr int kBins1 = 2048, kBins2 = 2048, kBins3 = 1024;
constexpr int kHistWords = kBins1 + kBins2 + kBins3;

// Workspace: the three histograms of every row ([rows][5120] words, cleared
// by each call), then the slice counts ([rows][nsub][2] words, always
// written before they are read).
struct RowWs {
  uint32_t* h1;
  uint32_t* h2;
  uint32_t* h3;
  uint32_t* counts;  // [nsub][2]: keys > T, keys == T
};

TSD_DEVICE RowWs row_ws(uint32_t* ws, int row, int nsub, int rows) {
  uint32_t* base = ws + static_cast<int64_t>(row) * kHistWords;
  uint32_t* cnt = ws + static_cast<int64_t>(rows) * kHistWords +
                  static_cast<int64_t>(row) * 2 * nsub;
  return {base, base + kBins1, base + kBins1 + kBins2, cnt};
}

TSD_DEVICE int64_t row_len(const int32_t* row_lens, int row, int64_t cap) {
  return clamp_len(row_lens[row], cap);
}

// Block-wide exclusive scan of one value per thread (256 threads).
TSD_DEVICE uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds4) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v, lane);
  if (lane == kWave - 1) lds4[w] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += lds4[i];
  __syncthreads();
  return before + inc - v;
}

struct BinPick {
  uint32_t bin;
  uint32_t above;  // elements in bins strictly above `bin`
};

// Finds the bin holding the target-th largest element of an LDS histogram:
// above(bin) < target <= above(bin) + hist[bin]. Threads own runs of bins
// from the top down; a block scan of the run totals locates the run.
template <int NB>
TSD_DEVICE BinPick pick_bin(const uint32_t* hist, uint32_t target,
                            uint32_t* lds4, BinPick* result) {
  constexpr int per = NB / kThreads;
  const int t = threadIdx.x;
  const int top = NB - t * per;  // this thread owns bins [top-per, top)
  uint32_t s = 0;
#pragma unroll
  for (int i = 1; i <= per; ++i) s += hist[top - i];
  if (t == 0) *result = BinPick{0u, 0u};
  const uint32_t before = block_exclusive_scan(s, lds4);
  if (before < target && target <= before + s) {
    uint32_t acc = before;
    for (int i = 1; i <= per; ++i) {
      const uint32_t h = hist[top - i];
      if (acc + h >= target) {
        *result = BinPick{static_cast<uint32_t>(top - i), acc};
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  const BinPick r = *result;
  __syncthreads();
  return r;
}

template <int NB>
TSD_DEVICE void load_hist(uint32_t* lds, const uint32_t* g) {
  for (int i = threadIdx.x; i < NB; i += kThreads) lds[i] = g[i];
  __syncthreads();
}

template <int NB>
TSD_DEVICE void zero_hist(uint32_t* lds) {
  for (int i = threadIdx.x; i < NB; i += kThreads) lds[i] = 0u;
  __syncthreads();
}

template <int NB>
TSD_DEVICE void flush_hist(const uint32_t* lds, uint32_t* g) {
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += kThreads) {
    const uint32_t v = lds[i];
    if (v) atomicAdd(g + i, v);
  }
}

// Threshold state shared by the passes after the digits are known.
struct Threshold {
  uint32_t key;   // T
  uint32_t need;  // ties at T to keep
};

TSD_DEVICE Threshold find_threshold(const RowWs& w, int k, uint32_t* hist,
                                    uint32_t* lds4, BinPick* pick) {
  load_hist<kBins1>(hist, w.h1);
  const BinPick p1 = pick_bin<kBins1>(hist, k, lds4, pick);
  load_hist<kBins2>(hist, w.h2);
  const BinPick p2 = pick_bin<kBins2>(hist, k - p1.above, lds4, pick);
  load_hist<kBins3>(hist, w.h3);
  const BinPick p3 =
      pick_bin<kBins3>(hist, k - p1.above - p2.above, lds4, pick);
  Threshold th;
  th.key = (p1.bin << 21) | (p2.bin << 10) | p3.bin;
  th.need = k - p1.above - p2.above - p3.above;
  return th;
}

__global__ __launch_bounds__(kThreads) void topk_clear_kernel(
    uint32_t* __restrict__ ws, int64_t words) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < words) ws[i] = 0u;
}

// Pass 1: histogram of the top 11 key bits.
__global__ __launch_bounds__(kThreads) void topk_hist1_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nsub,
    uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins1];
  const int row = blockIdx.y;
  const int64_t n = row_len(row_lens, row, cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kChunk;
  if (n <= k || start >= n) return;
  const int64_t end = start + kChunk < n ? start + kChunk : n;
  const float* s = scores + row * stride;
  zero_hist<kBins1>(hist);
  for (int64_t i = start + threadIdx.x; i < end; i += kThreads)
    atomicAdd(&hist[order_key(s[i]) >> 21], 1u);
  flush_hist<kBins1>(hist, row_ws(ws, row, nsub, gridDim.y).h1);
}

// Pass 2: histogram of key bits 20..10 among keys whose top digit is the
// threshold digit.
__global__ __launch_bounds__(kThreads) void topk_hist2_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nsub,
    uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t lds4[kWavesPerBlock];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int64_t n = row_len(row_lens, row, cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kChunk;
  if (n <= k || start >= n) return;
  const int64_t end = start + kChunk < n ? start + kChunk : n;
  const RowWs w = row_ws(ws, row, nsub, gridDim.y);
  load_hist<kBins1>(hist, w.h1);
  const BinPick p1 = pick_bin<kBins1>(hist, k, lds4, &pick);
  zero_hist<kBins2>(hist);
  const float* s = scores + row * stride;
  for (int64_t i = start + threadIdx.x; i < end; i += kThreads) {
    const uint32_t key = order_key(s[i]);
    if ((key >> 21) == p1.bin) atomicAdd(&hist[(key >> 10) & 0x7FF], 1u);
  }
  flush_hist<kBins2>(hist, w.h2);
}

// Pass 3: histogram of the low 10 key bits among keys matching the first
// 22 bits of the threshold.
__global__ __launch_bounds__(kThreads) void topk_hist3_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nsub,
    uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t lds4[kWavesPerBlock];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int64_t n = row_len(row_lens, row, cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kChunk;
  if (n <= k || start >= n) return;
  const int64_t end = start + kChunk < n ? start + kChunk : n;
  const RowWs w = row_ws(ws, row, nsub, gridDim.y);
  load_hist<kBins1>(hist, w.h1);
  const BinPick p1 = pick_bin<kBins1>(hist, k, lds4, &pick);
  load_hist<kBins2>(hist, w.h2);
  const BinPick p2 = pick_bin<kBins2>(hist, k - p1.above, lds4, &pick);
  const uint32_t prefix = (p1.bin << 11) | p2.bin;
  zero_hist<kBins3>(hist);
  const float* s = scores + row * stride;
  for (int64_t i = start + threadIdx.x; i < end; i += kThreads) {
    const uint32_t key = order_key(s[i]);
    if ((key >> 10) == prefix) atomicAdd(&hist[key & 0x3FF], 1u);
  }
  flush_hist<kBins3>(hist, w.h3);
}

// Pass 4: per 1024-element wave slice, the number of keys above T and equal
// to T.
__global__ __launch_bounds__(kThreads) void topk_count_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nsub,
    uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t lds4[kWavesPerBlock];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int64_t n = row_len(row_lens, row, cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kChunk;
  if (n <= k || start >= n) return;
  const RowWs w = row_ws(ws, row, nsub, gridDim.y);
  const Threshold th = find_threshold(w, k, hist, lds4, &pick);
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t s0 = static_cast<int64_t>(sub) * kSub;
  const int64_t s1 = s0 + kSub < n ? s0 + kSub : n;
  const float* s = scores + row * stride;
  uint32_t gt = 0, eq = 0;
  for (int64_t i = s0 + lane; i < s1; i += kWave) {
    const uint32_t key = order_key(s[i]);
    gt += key > th.key;
    eq += key == th.key;
  }
  gt = wave_sum_u32(gt);
  eq = wave_sum_u32(eq);
  if (lane == 0 && s0 < n) {
    w.counts[2 * sub] = gt;
    w.counts[2 * sub + 1] = eq;
  }
}

// Pass 5: ordered compaction into idx (and the fast path for n <= k).
__global__ __launch_bounds__(kThreads) void topk_write_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nsub,
    const uint32_t* __restrict__ ws_in, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t lds4[kWavesPerBlock];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int64_t n = row_len(row_lens, row, cap);
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  const int64_t m = n < k ? n : k;
  if (blockIdx.x == 0) {
    for (int64_t j = m + threadIdx.x; j < k; j += kThreads) out[j] = -1;
    if (threadIdx.x == 0 && count) count[row] = static_cast<int32_t>(m);
  }
  const int64_t start = static_cast<int64_t>(blockIdx.x) * kChunk;
  if (start >= n) return;
  const int64_t s0 = static_cast<int64_t>(sub) * kSub;
  const int64_t s1 = s0 + kSub < n ? s0 + kSub : n;
  if (n <= k) {
    for (int64_t i = s0 + lane; i < s1; i += kWave)
      out[i] = static_cast<int32_t>(i);
    return;
  }
  uint32_t* ws = const_cast<uint32_t*>(ws_in);
  const RowWs w = row_ws(ws, row, nsub, gridDim.y);
  const Threshold th = find_threshold(w, k, hist, lds4, &pick);
  if (s0 >= n) return;
  // counts of the slices before this one
  uint32_t gt_before = 0, eq_before = 0;
  for (int j = lane; j < sub; j += kWave) {
    gt_before += w.counts[2 * j];
    eq_before += w.counts[2 * j + 1];
  }
  gt_before = wave_sum_u32(gt_before);
  eq_before = wave_sum_u32(eq_before);
  uint32_t tie_rank = eq_before;
  uint32_t pos = gt_before + (eq_before < th.need ? eq_before : th.need);
  const float* s = scores + row * stride;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = s0; base < s1; base += kWave) {
    const int64_t i = base + lane;
    const uint32_t key = i < s1 ? order_key(s[i]) : 0u;
    const bool in = i < s1;
    const bool is_eq = in && key == th.key;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t my_tie =
        tie_rank + static_cast<uint32_t>(__popcll(eq_mask & lt_mask));
    const bool take = in && (key > th.key || (is_eq && my_tie < th.need));
    const uint64_t take_mask = __ballot(take);
    const uint32_t my_pos =
        pos + static_cast<uint32_t>(__popcll(take_mask & lt_mask));
    if (take && my_pos < static_cast<uint32_t>(k))
      out[my_pos] = static_cast<int32_t>(i);
    tie_rank += static_cast<uint32_t>(__popcll(eq_mask));
    pos += static_cast<uint32_t>(__popcll(take_mask));
  }
}

int nsub_for(int max_len) { return (max_len + kSub - 1) / kSub; }

}  // namespace

size_t topk_workspace(int rows, int max_len, int k) {
  (void)k;
  const int nsub = nsub_for(max_len);
  return static_cast<size_t>(rows) *
         (kHistWords + 2 * static_cast<size_t>(nsub)) * sizeof(uint32_t);
}

hipError_t launch_topk(const float* scores, int64_t stride, int rows,
                       const int32_t* row_lens, int max_len, int k,
                       int32_t* idx, int32_t* count, void* ws_v,
                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nsub = nsub_for(max_len);
  const int64_t cap = max_len < stride ? max_len : stride;
  uint32_t* ws = static_cast<uint32_t*>(ws_v);
  const int64_t words = static_cast<int64_t>(rows) * kHistWords;
  const int64_t cblocks = (words + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(topk_clear_kernel, dim3(static_cast<uint32_t>(cblocks)),
                     dim3(kThreads), 0, s, ws, words);
  const int chunks = max_len > 0 ? (max_len + kChunk - 1) / kChunk : 1;
  dim3 grid(static_cast<uint32_t>(chunks), static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(topk_hist1_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nsub, ws);
  hipLaunchKernelGGL(topk_hist2_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nsub, ws);
  hipLaunchKernelGGL(topk_hist3_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nsub, ws);
  hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nsub, ws);
  hipLaunchKernelGGL(topk_write_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nsub, ws, idx, count);
  return hipGetLastError();
}

}  // namespace tsd
