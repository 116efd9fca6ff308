// Pieces of the exact top-k select shared by the top-k kernels and by the
// index scan when it builds the first-digit histogram itself: the radix
// digits, the workspace layout, the histogram flush and the bin pick.
#pragma once

#include "device_common.h"

namespace tsd {

constexpr int kTopkB1 = 12, kTopkB2 = 10, kTopkB3 = 10;  // digit widths (bits)
constexpr int kTopkBins1 = 1 << kTopkB1;
constexpr int kTopkBins2 = 1 << kTopkB2;
constexpr int kTopkBins3 = 1 << kTopkB3;
constexpr int kTopkChunk = 4096;    // elements per filter chunk
constexpr int kTopkListCap = 512;   // entries kept per chunk list

// Digit 1 of a score's order-preserving key.
TSD_DEVICE uint32_t topk_digit1(uint32_t key) { return key >> (32 - kTopkB1); }

// Workspace layout, in 32-bit words from the base:
//   h1    [rows][4096]  digit-1 counts                    (zero on entry)
//   h2    [rows][1024]  digit-2 counts of the candidates  (zero on entry)
//   sel   [rows]        (digit-1 bin, elements above it) as uint2
//   counts[rows][nch]   survivors of each chunk
//   lists [rows][nch][512] (index, key) as uint2, 8-byte aligned
// The first two are zero on entry: a call clears them first unless its
// caller states they are zero already, and every call's last kernel leaves
// its rows of them zero again.
struct TopkWs {
  uint32_t* h1;
  uint32_t* h2;
  uint2* sel;
  uint32_t* counts;
  uint2* lists;
};

__host__ __device__ inline int64_t topk_clear_words(int rows) {
  return static_cast<int64_t>(rows) * (kTopkBins1 + kTopkBins2);
}

__host__ __device__ inline int64_t topk_list_offset_words(int rows, int nch) {
  const int64_t off = topk_clear_words(rows) + 2 * static_cast<int64_t>(rows) +
                      static_cast<int64_t>(rows) * nch;
  return (off + 1) & ~static_cast<int64_t>(1);  // 8-byte alignment
}

__host__ __device__ inline int64_t topk_ws_words(int rows, int nch) {
  return topk_list_offset_words(rows, nch) +
         2 * static_cast<int64_t>(rows) * nch * kTopkListCap;
}

// nch = 0 gives the row-indexed parts only (h1, h2, sel).
__host__ __device__ inline TopkWs topk_ws(void* base, int rows, int nch) {
  uint32_t* w = static_cast<uint32_t*>(base);
  const int64_t r = rows;
  TopkWs ws;
  ws.h1 = w;
  ws.h2 = w + r * kTopkBins1;
  ws.sel = reinterpret_cast<uint2*>(w + topk_clear_words(rows));
  ws.counts = w + topk_clear_words(rows) + 2 * r;
  ws.lists = reinterpret_cast<uint2*>(w + topk_list_offset_words(rows, nch));
  return ws;
}

// Adds a workgroup's LDS digit-1 histogram to a row's h1, nonzero bins only.
template <int NT>
TSD_DEVICE void topk_flush_h1(const uint32_t* hist_s, uint32_t* h1) {
  for (int i = threadIdx.x; i < kTopkBins1; i += NT) {
    const uint32_t c = hist_s[i];
    if (c) atomicAdd(h1 + i, c);
  }
}

// Inclusive-scan based block scan of one value per thread. Every use of
// `lds` writes before the first barrier and reads between the two, so calls
// may follow each other without further synchronisation.
template <int NT>
TSD_DEVICE uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) before += i < w ? lds[i] : 0u;
  __syncthreads();
  return before + inc - v;
}

struct BinPick {
  uint32_t bin;
  uint32_t above;  // elements in bins strictly above `bin`
};

// The bin holding the target-th largest element of a histogram of NB bins
// split over NT threads: above(bin) < target <= above(bin) + hist[bin].
// Thread t owns the run of NB/NT bins [NB - (t+1)*per, NB - t*per) and
// passes it in h[] from the top down (h[i] = hist[NB - t*per - 1 - i]); a
// block scan of the run totals names the one run that contains the target,
// and its owner finds the bin. If the histogram holds fewer than `target`
// elements the result is bin 0 with above = 0 (the callers' bounds keep that
// harmless). Exactly one thread writes *result between the two barriers, so
// consecutive calls need no extra synchronisation. `lds` holds NT/64 words.
template <int NB, int NT>
TSD_DEVICE BinPick pick_bin_runs(const uint32_t (&h)[NB / NT],
                                 uint32_t target, uint32_t* lds,
                                 BinPick* result) {
  constexpr int per = NB / NT;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
  const int base = NB - (t + 1) * per;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) s += h[i];
  const uint32_t inc = wave_inclusive_scan(s);
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  uint32_t before = inc - s;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) before += i < w ? lds[i] : 0u;
  if (before < target && target <= before + s) {
    uint32_t acc = before, bin = 0, above = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (!found && acc + h[i] >= target) {
        bin = static_cast<uint32_t>(base + per - 1 - i);
        above = acc;
        found = true;
      }
      acc += h[i];
    }
    *result = BinPick{bin, above};
  } else if (t == NT - 1 && before + s < target) {
    *result = BinPick{0u, 0u};  // fewer than target elements in all
  }
  __syncthreads();
  return *result;
}

// The same over a 16-byte aligned histogram in LDS (or global memory).
template <int NB, int NT>
TSD_DEVICE BinPick pick_bin(const uint32_t* hist, uint32_t target,
                            uint32_t* lds, BinPick* result) {
  constexpr int per = NB / NT;
  static_assert(per == 1 || per % 4 == 0, "bins per thread");
  const int base = NB - (static_cast<int>(threadIdx.x) + 1) * per;
  uint32_t h[per];
  if constexpr (per == 1) {
    h[0] = hist[base];
  } else {
#pragma unroll
    for (int q = 0; q < per / 4; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(hist + base + 4 * q);
      h[per - 1 - 4 * q] = x.x;
      h[per - 2 - 4 * q] = x.y;
      h[per - 3 - 4 * q] = x.z;
      h[per - 4 - 4 * q] = x.w;
    }
  }
  return pick_bin_runs<NB, NT>(h, target, lds, result);
}

}  // namespace tsd
