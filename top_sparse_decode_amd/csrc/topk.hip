// Exact top-k per row with the lowest-index tie-break ("QSA cache sharding",
// sglang PR #43527, Distributed QSA execution: an exact Top-K whose ties are
// broken deterministically by token ID), output in ascending index order.
//
// Scores map to order-preserving 32-bit keys (-0 folded onto +0). The k-th
// largest key T is found by an MSD radix select over digits of 12, 10 and
// 10 bits; all counts are integer atomics, so the result is deterministic.
//   pass 1 (per 4096-element chunk): histogram of digit 1 -> H1[row].
//   pass 2 (per chunk): with the threshold digit b1 known from H1, every key
//          whose digit 1 is >= b1 (above it: certainly kept; equal: a
//          candidate) is compacted in index order into the chunk's list of
//          (index, key) pairs, and the candidates' digit 2 is histogrammed
//          -> H2[row]. Typically 1-3% of a row survives.
//   pass 3 (one workgroup per row): digit 3 of the list keys matching
//          (b1, b2) is histogrammed in LDS, giving T and the number of ties
//          at T to keep. The kept entries are then marked in an LDS bitmap
//          over the row's indices (2^19 indices per segment) and a popcount
//          scan of the bitmap writes them out in ascending order.
// A chunk whose survivors overflow its list is read raw by pass 3 (the same
// entries, recomputed from the scores), so the result never depends on the
// list capacity. Rows with n <= k keep every index.
#include "device_common.h"
#include "launch.h"
#include "topk_digits.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 4096;           // elements per pass-1/2 workgroup
constexpr int kSub = kChunk / kWaves;  // elements per wave
constexpr int kPerThread = kChunk / kThreads;
constexpr int kListCap = 512;          // entries kept per chunk list
constexpr int kB1 = kTopkB1, kB2 = kTopkB2, kB3 = kTopkB3;
constexpr int kBins1 = kTopkBins1, kBins2 = kTopkBins2, kBins3 = kTopkBins3;
constexpr int kShift1 = 32 - kB1, kShift2 = kB3;
constexpr int kRT = 1024;              // pass-3 threads
constexpr int kSegBits = 1 << 19;      // indices per bitmap segment
constexpr int kSegWords = kSegBits / 32;
constexpr int kMaxChunks = 4096;       // max_len <= 2^24

TSD_DEVICE uint32_t digit1(uint32_t key) { return topk_digit1(key); }
TSD_DEVICE uint32_t digit2(uint32_t key) {
  return (key >> kShift2) & (kBins2 - 1);
}
TSD_DEVICE uint32_t prefix12(uint32_t key) { return key >> kShift2; }

struct Ws {
  uint32_t* h1;      // [rows][kBins1]
  uint32_t* h2;      // [rows][kBins2]
  uint32_t* counts;  // [rows][nch]  survivors of each chunk
  uint2* lists;      // [rows][nch][kListCap]  (index, key)
};

__host__ __device__ inline int64_t hist_words(int rows) {
  return static_cast<int64_t>(rows) * (kBins1 + kBins2);
}

__host__ __device__ inline int64_t list_offset_words(int rows, int nch) {
  const int64_t off = hist_words(rows) + static_cast<int64_t>(rows) * nch;
  return (off + 1) & ~static_cast<int64_t>(1);  // 8-byte alignment
}

__host__ __device__ inline Ws make_ws(void* base, int rows, int nch) {
  uint32_t* w = static_cast<uint32_t*>(base);
  Ws ws;
  ws.h1 = w;
  ws.h2 = w + static_cast<int64_t>(rows) * kBins1;
  ws.counts = w + hist_words(rows);
  ws.lists = reinterpret_cast<uint2*>(w + list_offset_words(rows, nch));
  return ws;
}

__host__ __device__ inline int64_t ws_words(int rows, int nch) {
  return list_offset_words(rows, nch) +
         2 * static_cast<int64_t>(rows) * nch * kListCap;
}

// Block-wide exclusive scan of one value per thread.
template <int NT>
TSD_DEVICE uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v, lane);
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += lds[i];
  __syncthreads();
  return before + inc - v;
}

struct BinPick {
  uint32_t bin;
  uint32_t above;  // elements in bins strictly above `bin`
};

// The bin holding the target-th largest element of an LDS histogram:
// above(bin) < target <= above(bin) + hist[bin]. Threads own runs of bins
// from the top down; a block scan of the run totals locates the run. If the
// histogram holds fewer than `target` elements the result is bin 0 with
// everything above it (the callers' bounds checks keep that harmless).
template <int NB, int NT>
TSD_DEVICE BinPick pick_bin(const uint32_t* hist, uint32_t target,
                            uint32_t* lds, BinPick* result) {
  constexpr int per = NB / NT;
  const int t = threadIdx.x;
  const int top = NB - t * per;  // this thread owns bins [top - per, top)
  uint32_t s = 0;
#pragma unroll
  for (int i = 1; i <= per; ++i) s += hist[top - i];
  if (t == 0) *result = BinPick{0u, 0u};
  const uint32_t before = block_exclusive_scan<NT>(s, lds);
  if (before < target && target <= before + s) {
    uint32_t acc = before;
#pragma unroll
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

template <int NB, int NT>
TSD_DEVICE void load_lds(uint32_t* lds, const uint32_t* g) {
  for (int i = threadIdx.x; i < NB; i += NT) lds[i] = g[i];
  __syncthreads();
}

template <int NB, int NT>
TSD_DEVICE void zero_lds(uint32_t* lds) {
  for (int i = threadIdx.x; i < NB; i += NT) lds[i] = 0u;
  __syncthreads();
}

template <int NB, int NT>
TSD_DEVICE void flush_hist(const uint32_t* lds, uint32_t* g) {
  __syncthreads();
  for (int i = threadIdx.x; i < NB; i += NT) {
    const uint32_t v = lds[i];
    if (v) atomicAdd(g + i, v);
  }
}

__global__ __launch_bounds__(kThreads) void topk_clear_kernel(
    uint32_t* __restrict__ ws, int64_t words) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < words) ws[i] = 0u;
}

// Pass 1: histogram of digit 1; a workgroup covers `cpw` consecutive chunks.
__global__ __launch_bounds__(kThreads) void topk_hist1_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    int cpw, void* __restrict__ ws_base) {
  __shared__ uint32_t hist[kBins1];
  const int row = blockIdx.y;
  const int64_t n = clamp_len(row_lens[row], cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * cpw * kChunk;
  if (n <= k || start >= n) return;
  const float* s = scores + row * stride;
  zero_lds<kBins1, kThreads>(hist);
  for (int c = 0; c < cpw; ++c) {
    const int64_t c0 = start + static_cast<int64_t>(c) * kChunk;
    if (c0 >= n) break;
    float v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t i = c0 + threadIdx.x + j * kThreads;
      v[j] = i < n ? s[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t i = c0 + threadIdx.x + j * kThreads;
      if (i < n) atomicAdd(&hist[digit1(order_key(v[j]))], 1u);
    }
  }
  const Ws ws = make_ws(ws_base, gridDim.y, nch);
  flush_hist<kBins1, kThreads>(hist, ws.h1 + static_cast<int64_t>(row) * kBins1);
}

// Pass 2: survivors (digit 1 >= b1) compacted in index order into each
// chunk's list; digit-2 histogram of the candidates (digit 1 == b1). A
// workgroup covers `cpw` consecutive chunks of one row, so the row's digit-1
// threshold is resolved once per workgroup.
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    int cpw, void* __restrict__ ws_base) {
  __shared__ uint32_t hist[kBins1];
  __shared__ uint2 list_s[kWaves][kSub];
  __shared__ uint32_t lds[kWaves];
  __shared__ uint32_t wcount[kWaves];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int64_t n = clamp_len(row_lens[row], cap);
  const int64_t start = static_cast<int64_t>(blockIdx.x) * cpw * kChunk;
  if (n <= k || start >= n) return;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const float* s = scores + row * stride;
  const Ws ws = make_ws(ws_base, gridDim.y, nch);
  load_lds<kBins1, kThreads>(hist, ws.h1 + static_cast<int64_t>(row) * kBins1);
  const BinPick p1 = pick_bin<kBins1, kThreads>(hist, k, lds, &pick);
  zero_lds<kBins2, kThreads>(hist);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t* counts = ws.counts + static_cast<int64_t>(row) * nch;
  for (int cc = 0; cc < cpw; ++cc) {
    const int64_t c0 = start + static_cast<int64_t>(cc) * kChunk;
    if (c0 >= n) break;  // uniform
    const int chunk = static_cast<int>(c0 / kChunk);
    const int64_t sub = c0 + static_cast<int64_t>(w) * kSub;
    float v[kSub / kWave];
#pragma unroll
    for (int r = 0; r < kSub / kWave; ++r) {
      const int64_t i = sub + r * kWave + lane;
      v[r] = i < n ? s[i] : 0.f;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < kSub / kWave; ++r) {
      const int64_t i = sub + r * kWave + lane;
      const uint32_t key = order_key(v[r]);
      const uint32_t d1 = digit1(key);
      const bool keep = i < n && d1 >= p1.bin;
      const uint64_t mask = __ballot(keep);
      if (keep) {
        const uint32_t pos = cnt + static_cast<uint32_t>(__popcll(mask & lt));
        list_s[w][pos] = make_uint2(static_cast<uint32_t>(i), key);
        if (d1 == p1.bin) atomicAdd(&hist[digit2(key)], 1u);
      }
      cnt += static_cast<uint32_t>(__popcll(mask));
    }
    if (lane == 0) wcount[w] = cnt;
    __syncthreads();
    uint32_t total = 0, off[kWaves];
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      off[i] = total;
      total += wcount[i];
    }
    if (threadIdx.x == 0) counts[chunk] = total;
    if (total <= kListCap) {
      uint2* dst =
          ws.lists + (static_cast<int64_t>(row) * nch + chunk) * kListCap;
      for (uint32_t e = threadIdx.x; e < total; e += kThreads) {
        int ww = 0;
#pragma unroll
        for (int i = 1; i < kWaves; ++i) ww += e >= off[i];
        dst[e] = list_s[ww][e - off[ww]];
      }
    }
    __syncthreads();  // list_s and wcount are reused by the next chunk
  }
  flush_hist<kBins2, kThreads>(hist, ws.h2 + static_cast<int64_t>(row) * kBins2);
}

// Survivors of one chunk, 64 per round, in index order: from the chunk's
// list, or recomputed from the raw scores when the list overflowed. Calls
// f(index, key) for every survivor held by this lane.
template <typename F>
TSD_DEVICE void for_survivors(const Ws& ws, const float* s, int row, int nch,
                              int c, uint32_t cnt, int64_t n, uint32_t b1,
                              int lane, F&& f) {
  if (cnt <= kListCap) {
    const uint2* list =
        ws.lists + (static_cast<int64_t>(row) * nch + c) * kListCap;
    for (uint32_t e = lane; e < cnt; e += kWave) {
      const uint2 en = list[e];
      f(static_cast<int64_t>(en.x), en.y);
    }
  } else {
    const int64_t i0 = static_cast<int64_t>(c) * kChunk;
    const int64_t i1 = i0 + kChunk < n ? i0 + kChunk : n;
    for (int64_t i = i0 + lane; i < i1; i += kWave) {
      const uint32_t key = order_key(s[i]);
      if (digit1(key) >= b1) f(i, key);
    }
  }
}

// Pass 3: exact threshold and ordered output, one workgroup per row.
__global__ __launch_bounds__(kRT) void topk_resolve_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    void* __restrict__ ws_base, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ uint32_t cnt_s[kMaxChunks];
  __shared__ uint32_t hist[kBins1];
  __shared__ uint32_t bits[kSegWords];
  __shared__ uint32_t lds[kRT / kWave + 1];  // scan partials + running total
  __shared__ uint32_t misc_s[2];
  __shared__ BinPick pick;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  constexpr int kWavesR = kRT / kWave;
  const int64_t n = clamp_len(row_lens[row], cap);
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  if (n <= k) {
    for (int64_t j = tid; j < k; j += kRT)
      out[j] = j < n ? static_cast<int32_t>(j) : -1;
    if (tid == 0 && count) count[row] = static_cast<int32_t>(n);
    return;
  }
  const Ws ws = make_ws(ws_base, gridDim.x, nch);
  const int nc = static_cast<int>((n + kChunk - 1) / kChunk);
  const float* s = scores + row * stride;
  for (int c = tid; c < nc; c += kRT)
    cnt_s[c] = ws.counts[static_cast<int64_t>(row) * nch + c];

  load_lds<kBins1, kRT>(hist, ws.h1 + static_cast<int64_t>(row) * kBins1);
  const BinPick p1 = pick_bin<kBins1, kRT>(hist, k, lds, &pick);
  load_lds<kBins2, kRT>(hist, ws.h2 + static_cast<int64_t>(row) * kBins2);
  const BinPick p2 = pick_bin<kBins2, kRT>(hist, k - p1.above, lds, &pick);
  const uint32_t pre = (p1.bin << kB2) | p2.bin;  // first 22 bits of T
  const uint32_t need2 = k - p1.above - p2.above;

  // digit 3 of the survivors that match the first 22 bits of T
  zero_lds<kBins3, kRT>(hist);
  for (int c = wave; c < nc; c += kWavesR)
    for_survivors(ws, s, row, nch, c, cnt_s[c], n, p1.bin, lane,
                  [&](int64_t, uint32_t key) {
                    if (prefix12(key) == pre)
                      atomicAdd(&hist[key & (kBins3 - 1)], 1u);
                  });
  __syncthreads();
  const BinPick p3 = pick_bin<kBins3, kRT>(hist, need2, lds, &pick);
  const uint32_t T = (pre << kB3) | p3.bin;
  const uint32_t need = need2 - p3.above;   // ties at T to keep
  const uint32_t ties = hist[p3.bin];       // ties at T in the row
  __syncthreads();

  // With more ties than needed, the kept ties are those with index <= the
  // index of the need-th tie, found segment by segment.
  int64_t tie_cut = n;
  if (ties > need) {
    if (tid == 0) misc_s[0] = 0u;
    uint32_t seen = 0;
    for (int64_t seg = 0; seg < n && tie_cut == n; seg += kSegBits) {
      zero_lds<kSegWords, kRT>(bits);
      const int c0 = static_cast<int>(seg / kChunk);
      const int c1 = static_cast<int>((seg + kSegBits) / kChunk) < nc
                         ? static_cast<int>((seg + kSegBits) / kChunk)
                         : nc;
      for (int c = c0 + wave; c < c1; c += kWavesR)
        for_survivors(ws, s, row, nch, c, cnt_s[c], n, p1.bin, lane,
                      [&](int64_t i, uint32_t key) {
                        if (key == T) {
                          const int64_t r = i - seg;
                          atomicOr(&bits[r >> 5], 1u << (r & 31));
                        }
                      });
      __syncthreads();
      constexpr int wpt = kSegWords / kRT;
      uint32_t pc = 0;
#pragma unroll
      for (int j = 0; j < wpt; ++j) pc += __popc(bits[tid * wpt + j]);
      const uint32_t before = seen + block_exclusive_scan<kRT>(pc, lds);
      if (before < need && need <= before + pc) {
        uint32_t acc = before;
        for (int j = 0; j < wpt; ++j) {
          uint32_t word = bits[tid * wpt + j];
          const uint32_t p = __popc(word);
          if (acc + p >= need) {
            for (uint32_t r = need - acc; r > 1; --r) word &= word - 1;
            misc_s[1] = static_cast<uint32_t>(
                (tid * wpt + j) * 32 + __ffs(word) - 1);
            misc_s[0] = 1u;
            break;
          }
          acc += p;
        }
      }
      if (tid == kRT - 1) lds[kWavesR] = before + pc;  // ties so far
      __syncthreads();
      if (misc_s[0]) tie_cut = seg + misc_s[1];
      seen = lds[kWavesR];
      __syncthreads();
    }
  }

  // mark kept survivors segment by segment and write them in index order
  uint32_t written = 0;
  for (int64_t seg = 0; seg < n; seg += kSegBits) {
    zero_lds<kSegWords, kRT>(bits);
    const int c0 = static_cast<int>(seg / kChunk);
    const int c1 = static_cast<int>((seg + kSegBits) / kChunk) < nc
                       ? static_cast<int>((seg + kSegBits) / kChunk)
                       : nc;
    for (int c = c0 + wave; c < c1; c += kWavesR)
      for_survivors(ws, s, row, nch, c, cnt_s[c], n, p1.bin, lane,
                    [&](int64_t i, uint32_t key) {
                      if (key > T || (key == T && i <= tie_cut)) {
                        const int64_t r = i - seg;
                        atomicOr(&bits[r >> 5], 1u << (r & 31));
                      }
                    });
    __syncthreads();
    constexpr int wpt = kSegWords / kRT;
    uint32_t wd[wpt], pc = 0;
#pragma unroll
    for (int j = 0; j < wpt; ++j) {
      wd[j] = bits[tid * wpt + j];
      pc += __popc(wd[j]);
    }
    uint32_t pos = written + block_exclusive_scan<kRT>(pc, lds);
#pragma unroll
    for (int j = 0; j < wpt; ++j) {
      uint32_t word = wd[j];
      while (word) {
        const int b = __ffs(word) - 1;
        word &= word - 1;
        if (pos < static_cast<uint32_t>(k))
          out[pos] = static_cast<int32_t>(seg + (tid * wpt + j) * 32 + b);
        ++pos;
      }
    }
    if (tid == kRT - 1) lds[kWavesR] = pos;
    __syncthreads();
    written = lds[kWavesR];
    __syncthreads();
  }
  if (tid == 0 && count) count[row] = k;
}

int nch_for(int max_len) { return max_len > 0 ? (max_len + kChunk - 1) / kChunk : 1; }

}  // namespace

size_t topk_workspace(int rows, int max_len, int k) {
  (void)k;
  return static_cast<size_t>(ws_words(rows, nch_for(max_len))) * sizeof(uint32_t);
}

int topk_max_len() { return kChunk * kMaxChunks; }

hipError_t launch_topk_clear(void* ws, int rows, hipStream_t s) {
  const int64_t words = hist_words(rows);
  hipLaunchKernelGGL(topk_clear_kernel,
                     dim3(static_cast<uint32_t>((words + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, static_cast<uint32_t*>(ws), words);
  return hipGetLastError();
}

// Chunks per pass-1/2 workgroup: one, unless the launch would exceed about
// 2,048 workgroups, in which case a workgroup takes consecutive chunks.
int chunks_per_wg(int nch, int rows) {
  const int64_t total = static_cast<int64_t>(nch) * rows;
  int cpw = 1;
  while (total / cpw > 2048 && cpw < nch) cpw *= 2;
  return cpw;
}

hipError_t launch_topk_hist1(const float* scores, int64_t stride, int rows,
                             const int32_t* row_lens, int max_len, int k,
                             void* ws, hipStream_t s) {
  const int nch = nch_for(max_len);
  const int cpw = chunks_per_wg(nch, rows);
  const int64_t cap = max_len < stride ? max_len : stride;
  dim3 grid(static_cast<uint32_t>((nch + cpw - 1) / cpw),
            static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(topk_hist1_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nch, cpw, ws);
  return hipGetLastError();
}

hipError_t launch_topk_finish(const float* scores, int64_t stride, int rows,
                              const int32_t* row_lens, int max_len, int k,
                              int32_t* idx, int32_t* count, void* ws,
                              hipStream_t s) {
  const int nch = nch_for(max_len);
  const int cpw = chunks_per_wg(nch, rows);
  const int64_t cap = max_len < stride ? max_len : stride;
  dim3 grid(static_cast<uint32_t>((nch + cpw - 1) / cpw),
            static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(kThreads), 0, s, scores,
                     stride, row_lens, cap, k, nch, cpw, ws);
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(static_cast<uint32_t>(rows)),
                     dim3(kRT), 0, s, scores, stride, row_lens, cap, k, nch,
                     ws, idx, count);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t stride, int rows,
                       const int32_t* row_lens, int max_len, int k,
                       int32_t* idx, int32_t* count, void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipError_t e = launch_topk_clear(ws, rows, s);
  if (e != hipSuccess) return e;
  e = launch_topk_hist1(scores, stride, rows, row_lens, max_len, k, ws, s);
  if (e != hipSuccess) return e;
  return launch_topk_finish(scores, stride, rows, row_lens, max_len, k, idx,
                            count, ws, s);
}

}  // namespace tsd
