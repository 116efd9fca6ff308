// Exact top-k per row with the lowest-index tie-break ("QSA cache sharding",
// sglang PR #43527, Distributed QSA execution: an exact Top-K whose ties are
// broken deterministically by token ID), output in ascending index order.
//
// Scores map to order-preserving 32-bit keys (-0 folded onto +0). The k-th
// largest key T is found by an MSD radix select over digits of 12, 10 and
// 10 bits; all counts are integer atomics, so the result is deterministic.
//   pass 1 (per 4096-element chunk, or inside the index scan): histogram of
//          digit 1 -> H1[row].
//   pass 2 (2 or 4 chunks per workgroup pass): the threshold digit b1 (the bin
//          holding the k-th largest) is resolved from H1; every key whose
//          digit 1 is >= b1 (above it:
//          certainly kept; equal: a candidate) is compacted in index order
//          into the chunk's list of (index, key) pairs, and the candidates'
//          digit 2 is histogrammed -> H2[row]. Typically 1-3% of a row
//          survives.
//   pass 3 (one workgroup per row): the chunk lists, concatenated in chunk
//          order, are the row's survivors in ascending index order. Digit 3
//          of those matching (b1, b2) gives T and the number of ties at T to
//          keep; the kept entries are placed by ballots and one exchange of
//          per-wave totals. When a list overflowed or the survivors exceed
//          what the workgroup holds in registers, the survivors are instead
//          marked in an LDS bitmap over the row's indices (2^19 indices per
//          segment) and written out by a popcount scan.
// A chunk whose survivors overflow its list is read raw by pass 3 (the same
// entries, recomputed from the scores), so the result never depends on the
// list capacity. Rows with n <= k keep every index.
// Short rows (at most 32,768 entries; see topk_small_fits) take a single
// launch instead: one workgroup per row holds the whole row in registers and
// runs the same three digits and the same ordered placement on chip, with no
// workspace.
#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = kTopkChunk;     // elements per pass-1/2 workgroup
constexpr int kPerThread = kChunk / kThreads;
constexpr int kListCap = kTopkListCap;  // entries kept per chunk list
constexpr int kB2 = kTopkB2, kB3 = kTopkB3;
constexpr int kBins1 = kTopkBins1, kBins2 = kTopkBins2, kBins3 = kTopkBins3;
constexpr int kShift2 = kB3;
constexpr int kRT = 1024;              // pass-3 threads
constexpr int kSegBits = 1 << 19;      // indices per bitmap segment
constexpr int kSegWords = kSegBits / 32;
constexpr int kMaxChunks = 4096;       // max_len <= 2^24
constexpr int kStage = 8192;           // survivors the pass-3 fast path holds
constexpr int kPerLane = kStage / kRT; // survivors per lane on that path
constexpr int kBlindRounds = 16;       // list reads per lane on the blind path
constexpr int kSmallMax = 32 * kRT;   // longest rows of the one-workgroup path

TSD_DEVICE uint32_t digit1(uint32_t key) { return topk_digit1(key); }
TSD_DEVICE uint32_t digit2(uint32_t key) {
  return (key >> kShift2) & (kBins2 - 1);
}
TSD_DEVICE uint32_t prefix12(uint32_t key) { return key >> kShift2; }

using Ws = TopkWs;

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
// The first chunk's scores are loaded together with the row length (load i
// reads entry min(i, cap - 1) of the row, cap = min(max_len, stride) >=
// 24,577 here since shorter rows take the one-workgroup path; entries at or
// past the length are not counted).
__global__ __launch_bounds__(kThreads) void topk_hist1_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    int cpw, void* __restrict__ ws_base) {
  __shared__ __align__(16) uint32_t hist[kBins1];
  const int row = blockIdx.y;
  const int32_t len_raw = row_lens[row];
  const int64_t start = static_cast<int64_t>(blockIdx.x) * cpw * kChunk;
  const float* s = scores + row * stride;
  float v[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t i = start + threadIdx.x + j * kThreads;
    v[j] = s[i < cap ? i : cap - 1];
  }
  const int64_t n = clamp_len(len_raw, cap);
  if (n <= k || start >= n) return;
  zero_lds<kBins1, kThreads>(hist);
  for (int c = 0; c < cpw; ++c) {
    const int64_t c0 = start + static_cast<int64_t>(c) * kChunk;
    if (c0 >= n) break;
    if (c > 0) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int64_t i = c0 + threadIdx.x + j * kThreads;
        v[j] = i < n ? s[i] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int64_t i = c0 + threadIdx.x + j * kThreads;
      if (i < n) atomicAdd(&hist[digit1(order_key(v[j]))], 1u);
    }
  }
  const Ws ws = topk_ws(ws_base, gridDim.y, nch);
  __syncthreads();
  topk_flush_h1<kThreads>(hist, ws.h1 + static_cast<int64_t>(row) * kBins1);
}

// Pass 2: survivors (digit 1 >= b1) compacted in index order into each
// chunk's list; digit-2 histogram of the candidates (digit 1 == b1).
// A workgroup of 16 waves takes FC consecutive chunks per pass (16/FC
// waves per chunk) and `passes` consecutive passes: FC = 1 while one chunk
// per workgroup keeps the launch within 256 workgroups, one per CU (1.6 us
// faster on one row of 1,048,576; at 512 workgroups, 8 rows of 262,144, it
// is 2.3 us slower than FC = 2), FC = 2 while the launch stays within about
// 1,024 workgroups (twice the workgroups of FC = 4, 1.6 us faster on 8 rows
// of 262,144), else FC = 4 (fewer, longer passes: 0.3 ms faster on 2,048
// rows of a million). It
// resolves b1 itself from the row's H1 (one uint4 run of 4 bins per thread,
// read while its first scores are in flight); the row's first workgroup
// records (b1, above) for pass 3. Survivors are counted by ballots, the
// per-wave counts exchanged once, and each survivor stored straight to its
// slot in the chunk's list.
constexpr int kFT = 1024;                        // filter threads
constexpr int kFW = kFT / kWave;                 // 16 waves

template <int FC>
__global__ __launch_bounds__(kFT) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    int passes, void* __restrict__ ws_base) {
  __shared__ uint32_t hist[kBins2];
  __shared__ uint32_t wcount[kFW];
  __shared__ uint32_t lds[kFW];
  __shared__ BinPick pick;
  const int row = blockIdx.y;
  const int32_t len_raw = row_lens[row];
  constexpr int kFChunks = FC;                     // chunks per pass
  constexpr int kFWavesPerChunk = kFW / kFChunks;
  constexpr int kFSub = kChunk / kFWavesPerChunk;  // elements per wave
  constexpr int kFPer = kFSub / kWave;             // elements per lane
  constexpr int64_t kSpan = static_cast<int64_t>(kFChunks) * kChunk;
  const int64_t start = static_cast<int64_t>(blockIdx.x) * passes * kSpan;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const int q = w / kFWavesPerChunk, wq = w % kFWavesPerChunk;
  const float* s = scores + row * stride;
  const Ws ws = topk_ws(ws_base, gridDim.y, nch);
  // b1 from the row's H1: thread t holds bins [4096 - 4(t+1), 4096 - 4t).
  // The row length, H1 and the first pass's scores are loaded in that order
  // before any of them is used. The score loads are unconditional and do
  // not wait for the length: load i reads entry min(i, cap - 1), inside the
  // row's [0, cap) of the caller's buffer (cap = min(max_len, stride) >=
  // 24,577 here: shorter rows take the one-workgroup path), and entries at
  // or past the length are masked at use. Loads
  // complete in order, so the early-exit test waits for the length only and
  // the pick's wait for H1 leaves the scores in flight.
  constexpr int per1 = kBins1 / kFT;
  static_assert(per1 == 4, "one uint4 run per thread");
  const uint4 x = *reinterpret_cast<const uint4*>(
      ws.h1 + static_cast<int64_t>(row) * kBins1 + (kBins1 - (tid + 1) * per1));
  float v[kFPer];
  auto load_pass = [&](int64_t p0) {
    const int64_t sub = p0 + static_cast<int64_t>(q) * kChunk +
                        static_cast<int64_t>(wq) * kFSub;
#pragma unroll
    for (int r = 0; r < kFPer; ++r) {
      const int64_t i = sub + r * kWave + lane;
      v[r] = s[i < cap ? i : cap - 1];
    }
  };
  load_pass(start);
  const int64_t n = clamp_len(len_raw, cap);
  if (n <= k || start >= n) return;
  const uint32_t h[per1] = {x.w, x.z, x.y, x.x};  // from the top down
  for (int i = tid; i < kBins2; i += kFT) hist[i] = 0u;  // ordered by the pick
  const BinPick p1 =
      pick_bin_runs<kBins1, kFT>(h, static_cast<uint32_t>(k), lds, &pick);
  if (blockIdx.x == 0 && tid == 0) ws.sel[row] = make_uint2(p1.bin, p1.above);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint32_t* counts = ws.counts + static_cast<int64_t>(row) * nch;
  for (int ps = 0; ps < passes; ++ps) {
    const int64_t p0 = start + static_cast<int64_t>(ps) * kSpan;
    if (p0 >= n) break;  // uniform
    const int64_t c0 = p0 + static_cast<int64_t>(q) * kChunk;
    const int64_t sub = c0 + static_cast<int64_t>(wq) * kFSub;
    uint32_t key[kFPer];
    uint64_t mask[kFPer];
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < kFPer; ++r) {
      const int64_t i = sub + r * kWave + lane;
      key[r] = order_key(v[r]);
      const uint32_t d1 = digit1(key[r]);
      const bool keep = i < n && d1 >= p1.bin;
      mask[r] = __ballot(keep);
      cnt += static_cast<uint32_t>(__popcll(mask[r]));
      if (keep && d1 == p1.bin) atomicAdd(&hist[digit2(key[r])], 1u);
    }
    if (ps + 1 < passes && p0 + kSpan < n) load_pass(p0 + kSpan);
    if (lane == 0) wcount[w] = cnt;
    __syncthreads();
    uint32_t off = 0, total = 0;
#pragma unroll
    for (int j = 0; j < kFWavesPerChunk; ++j) {
      const uint32_t c = wcount[q * kFWavesPerChunk + j];
      off += j < wq ? c : 0u;
      total += c;
    }
    if (c0 < n) {  // uniform per wave; the chunk holds elements
      const int chunk = static_cast<int>(c0 / kChunk);
      if (wq == 0 && lane == 0) counts[chunk] = total;
      if (total <= static_cast<uint32_t>(kListCap)) {
        uint2* dst =
            ws.lists + (static_cast<int64_t>(row) * nch + chunk) * kListCap;
        uint32_t pos = off;
#pragma unroll
        for (int r = 0; r < kFPer; ++r) {
          if ((mask[r] >> lane) & 1ull) {
            const uint32_t pidx =
                pos + static_cast<uint32_t>(__popcll(mask[r] & lt));
            dst[pidx] = make_uint2(static_cast<uint32_t>(sub + r * kWave + lane),
                                   key[r]);
          }
          pos += static_cast<uint32_t>(__popcll(mask[r]));
        }
      }
    }
    __syncthreads();  // wcount is reused by the next pass
  }
  flush_hist<kBins2, kFT>(hist, ws.h2 + static_cast<int64_t>(row) * kBins2);
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
//
// The chunk counts, b1 and H2 are read in one round trip; a block scan turns
// the counts into each chunk's offset in the row's survivor sequence.
// Fast path (no list overflowed, at most kStage survivors): every survivor
// is loaded once into registers, wave-contiguously, while digit 3 is
// histogrammed; after T is known one wave-total exchange gives each wave its
// output base (kept = key > T, plus the first `need` ties in index order)
// and ballots place the kept entries. Otherwise the survivors are re-read
// per pass and ordered through an LDS bitmap over the row's indices.
// Zeroes a row's digit-1 and digit-2 counts once the row's last reader is
// done with them (every path of the resolve ends here), so the next call on
// the workspace may skip the clearing launch.
TSD_DEVICE void clean_row(const Ws& ws, int row) {
  uint4* h1 = reinterpret_cast<uint4*>(ws.h1 + static_cast<int64_t>(row) * kBins1);
  uint4* h2 = reinterpret_cast<uint4*>(ws.h2 + static_cast<int64_t>(row) * kBins2);
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int i = threadIdx.x; i < kBins1 / 4; i += kRT) h1[i] = z;
  for (int i = threadIdx.x; i < kBins2 / 4; i += kRT) h2[i] = z;
}

// Blind plan of the resolve for nch chunks per row: wave w takes chunks
// [w*R, w*R + R) and reads the first E list entries of each; entry p of the
// wave's sequence (p = 64*q + lane in round q) is entry p % E of the wave's
// chunk p / E, so the sequence stays in index order. E is the smallest power
// of two from 16 that holds three times the survivors a chunk keeps on
// average (about 4096*k/max_len), at most the whole list (512 entries) and
// at most kBlindRounds rounds of 64 entries; rounds = 0 when even 16 entries
// per chunk exceed that (no blind path).
struct BlindPlan {
  int rounds, logE;
};
BlindPlan blind_plan(int nch, int k, int max_len) {
  const int R = (nch + kRT / kWave - 1) / (kRT / kWave);
  if (R * 16 > kBlindRounds * kWave) return {0, 4};
  const int64_t want = 3 * (static_cast<int64_t>(kChunk) * k / (max_len > 0 ? max_len : 1));
  int logE = 4;
  while ((1 << logE) < kListCap && (1 << logE) < want &&
         R * (2 << logE) <= kBlindRounds * kWave)
    ++logE;
  return {(R * (1 << logE) + kWave - 1) / kWave, logE};
}

// RB: blind rounds compiled in (2, 4, 8 or 16, at least the blind plan's),
// or 0 for rows with no blind path.
template <int RB>
__global__ __launch_bounds__(kRT) void topk_resolve_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k, int nch,
    int logE, void* __restrict__ ws_base, int32_t* __restrict__ idx,
    int32_t* __restrict__ count) {
  __shared__ uint32_t off_s[kMaxChunks + 1];  // survivors before chunk c
  __shared__ __align__(16) uint32_t hist[kBins3];
  __shared__ __align__(16) uint32_t hist2[kBins2];
  __shared__ uint32_t bits[kSegWords];
  __shared__ uint32_t lds[kRT / kWave + 1];  // scan partials + running total
  __shared__ uint32_t misc_s[2];
  __shared__ BinPick pick;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  constexpr int kWavesR = kRT / kWave;
  const Ws ws = topk_ws(ws_base, gridDim.x, nch);
  // Blind reads, issued with the row length: wave w takes chunks
  // [w*R, w*R + R) and reads the first E entries of each chunk's list and,
  // in lane j, the count of its j-th chunk. Entries past a chunk's count are
  // ignored; when every live chunk holds at most E survivors this is the
  // whole survivor sequence, wave-contiguous, after a single round trip.
  // Round q of a lane covers entry p = 64*q + lane of the wave: entry p % E
  // of its chunk p / E (E = 2^logE from the launcher's blind plan).
  // The row's records are loaded first and every blind read is
  // unconditional (a chunk index past nch reads the last chunk and is
  // masked at use), so the compiler can count the loads in flight and the
  // digit-2 pick below runs while the lists arrive (loads complete in order).
  constexpr bool kBlind = RB > 0;
  constexpr int kRounds = kBlind ? RB : 1;
  const int R = (nch + kWavesR - 1) / kWavesR;
  const int ents = 1 << logE;  // list entries read per chunk
  const uint32_t h2v = ws.h2[static_cast<int64_t>(row) * kBins2 + (kBins2 - 1 - tid)];
  const uint2 sel = ws.sel[row];  // digit-1 bin of the row, from pass 2
  const int64_t n = clamp_len(row_lens[row], cap);
  uint2 bl[kRounds];
  uint32_t cntw = 0;
  if constexpr (kBlind) {
    __builtin_amdgcn_sched_barrier(0);  // keep the records' loads first
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int p = q * kWave + lane;
      int c = wave * R + (p >> logE);
      c = c < nch ? c : nch - 1;
      bl[q] = ws.lists[(static_cast<int64_t>(row) * nch + c) * kListCap +
                       (p & (ents - 1))];
    }
    int c = wave * R + lane;
    c = c < nch ? c : nch - 1;
    cntw = ws.counts[static_cast<int64_t>(row) * nch + c];
  }
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  if (n <= k) {
    for (int64_t j = tid; j < k; j += kRT)
      out[j] = j < n ? static_cast<int32_t>(j) : -1;
    if (tid == 0 && count) count[row] = static_cast<int32_t>(n);
    clean_row(ws, row);
    return;
  }
  const int nc = static_cast<int>((n + kChunk - 1) / kChunk);
  const float* s = scores + row * stride;
  const BinPick p1{sel.x, sel.y};
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));

  bool blind_ok = false;
  BinPick p2b{0u, 0u};
  if constexpr (kBlind) {
    hist[tid] = 0u;  // digit-3 counts; ordered before use by p2's barriers
    const uint32_t h2r[1] = {h2v};
    p2b = pick_bin_runs<kBins2, kRT>(h2r, k - p1.above, lds, &pick);
    const int c = wave * R + lane;
    blind_ok = __ballot(lane < R && c < nc &&
                        cntw > static_cast<uint32_t>(ents)) == 0;
  }
  if (kBlind && __syncthreads_and(blind_ok)) {
    // ---- blind fast path ----
    const BinPick p2 = p2b;
    const uint32_t pre = (p1.bin << kB2) | p2.bin;  // first 22 bits of T
    const uint32_t need2 = k - p1.above - p2.above;
    // per-lane flags of the rounds, one bit per round (ok, above T, at T),
    // balloted again where a wave-wide view is needed
    uint32_t okb = 0;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      const int p = q * kWave + lane;
      const int j = p >> logE;  // the wave's chunk of this entry (< 64)
      const int c = wave * R + j;
      // its count sits in lane j: one lane for the whole round when ents >= 64
      const uint32_t cc = static_cast<uint32_t>(
          ents >= kWave ? __builtin_amdgcn_readlane(static_cast<int>(cntw), (q * kWave) >> logE)
                     : __shfl(static_cast<int>(cntw), j));
      const bool ok = j < R && c < nc && static_cast<uint32_t>(p & (ents - 1)) < cc;
      okb |= static_cast<uint32_t>(ok) << q;
      if (ok && prefix12(bl[q].y) == pre)
        atomicAdd(&hist[bl[q].y & (kBins3 - 1)], 1u);
    }
    __syncthreads();
    const BinPick p3 = pick_bin<kBins3, kRT>(hist, need2, lds, &pick);
    const uint32_t T = (pre << kB3) | p3.bin;
    const uint32_t need = need2 - p3.above;  // ties at T to keep
    uint32_t gtb = 0, eqb = 0, gtl = 0, eql = 0;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      const bool ok = (okb >> q) & 1u;
      const bool gt = ok && bl[q].y > T, eq = ok && bl[q].y == T;
      gtb |= static_cast<uint32_t>(gt) << q;
      eqb |= static_cast<uint32_t>(eq) << q;
      gtl += gt;
      eql += eq;
    }
    const uint32_t gtw = wave_sum_u32(gtl), eqw = wave_sum_u32(eql);
    // per-wave totals packed (ties << 16 | above); each is < 2^16
    if (lane == 0) lds[wave] = (eqw << 16) | gtw;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < kWavesR; ++i) before += i < wave ? lds[i] : 0u;
    uint32_t eqr = before >> 16;  // ties in earlier waves
    uint32_t pos = (before & 0xffffu) + (eqr < need ? eqr : need);
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      const bool is_gt = (gtb >> q) & 1u;
      const bool is_eq = (eqb >> q) & 1u;
      const uint64_t me = __ballot(is_eq);
      const uint32_t rank = eqr + static_cast<uint32_t>(__popcll(me & lt));
      const bool kept = is_gt || (is_eq && rank < need);
      const uint64_t mk = __ballot(kept);
      const uint32_t p = pos + static_cast<uint32_t>(__popcll(mk & lt));
      if (kept && p < static_cast<uint32_t>(k)) out[p] = static_cast<int32_t>(bl[q].x);
      pos += static_cast<uint32_t>(__popcll(mk));
      eqr += static_cast<uint32_t>(__popcll(me));
    }
    if (tid == 0 && count) count[row] = k;
    clean_row(ws, row);
    return;
  }

  // counts of this thread's run of chunks, b1 and H2, all loads in flight
  constexpr int kCpt = kMaxChunks / kRT;
  uint32_t cnt[kCpt];
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
    const int c = tid * kCpt + j;
    cnt[j] = c < nc ? ws.counts[static_cast<int64_t>(row) * nch + c] : 0u;
  }
  const uint32_t* h2 = ws.h2 + static_cast<int64_t>(row) * kBins2;
  for (int i = tid; i < kBins2; i += kRT) hist2[i] = h2[i];
  uint32_t run = 0;
  bool over = false;
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
    run += cnt[j];
    over |= cnt[j] > static_cast<uint32_t>(kListCap);
  }
  {
    // the scan's first barrier also publishes hist2
    uint32_t acc = block_exclusive_scan<kRT>(run, lds);
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const int c = tid * kCpt + j;
      if (c < nc) off_s[c] = acc;
      acc += cnt[j];
    }
    if (tid == kRT - 1) off_s[nc] = acc;  // every chunk lies in some run
  }
  const bool any_over = __syncthreads_or(over);
  const uint32_t total = off_s[nc];
  const bool fast = !any_over && total <= static_cast<uint32_t>(kStage);

  // Fast path: every survivor is loaded once, wave-contiguously, and its
  // loads stay in flight while the digit-2 bin is resolved.
  const uint32_t E = (total + kRT - 1) / kRT;  // rounds per lane
  const uint32_t wbase = static_cast<uint32_t>(wave) * E * kWave;
  uint2 v[kPerLane];
  if (fast) {
    // chunk of each entry: the largest c with off_s[c] <= e, by a
    // branchless binary search run for all of the lane's entries at once
    int cl[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) cl[j] = 0;
    for (int step = 1 << (31 - __clz(nc)); step > 0; step >>= 1) {
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const uint32_t e = wbase + j * kWave + lane;
        const int c = cl[j] + step;
        if (c < nc && off_s[c] <= e) cl[j] = c;
      }
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint32_t e = wbase + j * kWave + lane;
      v[j] = make_uint2(0u, 0u);
      if (static_cast<uint32_t>(j) < E && e < total)
        v[j] = ws.lists[(static_cast<int64_t>(row) * nch + cl[j]) * kListCap +
                        (e - off_s[cl[j]])];
    }
  }
  for (int i = tid; i < kBins3; i += kRT) hist[i] = 0u;  // ordered by p2
  const BinPick p2 = pick_bin<kBins2, kRT>(hist2, k - p1.above, lds, &pick);
  const uint32_t pre = (p1.bin << kB2) | p2.bin;  // first 22 bits of T
  const uint32_t need2 = k - p1.above - p2.above;

  if (fast) {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint32_t e = wbase + j * kWave + lane;
      if (static_cast<uint32_t>(j) < E && e < total &&
          prefix12(v[j].y) == pre)
        atomicAdd(&hist[v[j].y & (kBins3 - 1)], 1u);
    }
    __syncthreads();
    const BinPick p3 = pick_bin<kBins3, kRT>(hist, need2, lds, &pick);
    const uint32_t T = (pre << kB3) | p3.bin;
    const uint32_t need = need2 - p3.above;  // ties at T to keep
    uint64_t mg[kPerLane], me[kPerLane];
    uint32_t gtw = 0, eqw = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const uint32_t e = wbase + j * kWave + lane;
      const bool ok = static_cast<uint32_t>(j) < E && e < total;
      mg[j] = __ballot(ok && v[j].y > T);
      me[j] = __ballot(ok && v[j].y == T);
      gtw += static_cast<uint32_t>(__popcll(mg[j]));
      eqw += static_cast<uint32_t>(__popcll(me[j]));
    }
    // per-wave totals packed (ties << 16 | above); each is <= kStage
    if (lane == 0) lds[wave] = (eqw << 16) | gtw;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < kWavesR; ++i) before += i < wave ? lds[i] : 0u;
    uint32_t eqr = before >> 16;  // ties in earlier waves
    uint32_t pos = (before & 0xffffu) + (eqr < need ? eqr : need);
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const bool is_gt = (mg[j] >> lane) & 1ull;
      const bool is_eq = (me[j] >> lane) & 1ull;
      const uint32_t rank = eqr + static_cast<uint32_t>(__popcll(me[j] & lt));
      const bool kept = is_gt || (is_eq && rank < need);
      const uint64_t mk = __ballot(kept);
      const uint32_t p = pos + static_cast<uint32_t>(__popcll(mk & lt));
      if (kept && p < static_cast<uint32_t>(k)) out[p] = static_cast<int32_t>(v[j].x);
      pos += static_cast<uint32_t>(__popcll(mk));
      eqr += static_cast<uint32_t>(__popcll(me[j]));
    }
    if (tid == 0 && count) count[row] = k;
    clean_row(ws, row);
    return;
  }

  // ---- general path: survivors re-read per pass, ordered by a bitmap ----
  for (int c = wave; c < nc; c += kWavesR)
    for_survivors(ws, s, row, nch, c, off_s[c + 1] - off_s[c], n, p1.bin,
                  lane, [&](int64_t, uint32_t key) {
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
        for_survivors(ws, s, row, nch, c, off_s[c + 1] - off_s[c], n, p1.bin,
                      lane, [&](int64_t i, uint32_t key) {
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
      for_survivors(ws, s, row, nch, c, off_s[c + 1] - off_s[c], n, p1.bin,
                    lane, [&](int64_t i, uint32_t key) {
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
  clean_row(ws, row);
}

// Rows of at most 1,024 * RPT elements: one workgroup per row holds the
// whole row in registers, element r * 1024 + t in round r of thread t, so
// the row is read once and every pass runs on chip. Digits 1, 2 and 3 are
// histogrammed in LDS in turn (each pass over the candidates of the
// previous digits), giving T and the number of ties at T to keep; then the
// (round, wave) blocks of 64 consecutive indices, in index order, are
// ranked by an exclusive scan of their counts above T and at T, and each
// kept entry is stored at (kept before its block) + (kept lanes before it
// in the block).
// Lanes of the last round that lie past the row take key 0, the smallest
// key, in every pass: the k-th largest key is unchanged, none of them is
// above it, and as ties they follow every real tie in index order, of
// which there are at least as many as are kept, so none is kept. Rounds
// wholly past the row are skipped (a uniform branch).
// Digit 1 is counted in four copies of the histogram, lane l adding to copy
// l % 4, each copy starting four banks after the previous (a 16-byte
// aligned pitch, so the pick reads a thread's 4 bins of a copy with one
// 16-byte load instead of four strided words), so lanes of one wave that
// share a bin mostly update different words.
template <int RPT>
__global__ __launch_bounds__(kRT) void topk_small_kernel(
    const float* __restrict__ scores, int64_t stride,
    const int32_t* __restrict__ row_lens, int64_t cap, int k,
    int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  constexpr int kWavesR = kRT / kWave;
  constexpr int kBlocks = RPT * kWavesR;  // (round, wave) blocks
  constexpr int kCopies = 4;
  constexpr int kCopyPitch = kBins1 + 4;
  static_assert(kBlocks <= kRT, "one block count per thread");
  static_assert(kBins1 == 4 * kRT && kBins2 == kRT && kBins3 == kRT, "bins");
  __shared__ __align__(16) uint32_t h1[kCopies * kCopyPitch];
  __shared__ __align__(16) uint32_t h2[kBins2];
  __shared__ __align__(16) uint32_t h3[kBins3];
  __shared__ uint32_t cnt_s[kBlocks];  // (ties << 16 | above) per block
  __shared__ uint32_t lds[kRT / kWave + 1];
  __shared__ BinPick pick;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  // The row's scores are loaded together with its length, not after it:
  // load i reads entry min(i, cap - 1), inside the row's [0, cap) of the
  // caller's [rows, stride] buffer (cap = min(max_len, stride) <= 32,768),
  // and entries at or past the length are masked below. Every load is
  // unconditional, so the first histogram consumes the row while the rest
  // of it is still in flight.
  const float* s = scores + row * stride;
  const int capi = static_cast<int>(cap);
  const int32_t len_raw = row_lens[row];
  uint32_t key[RPT];
  if (capi > 0) {  // uniform; cap = 0 leaves every row empty
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = r * kRT + tid;
      key[r] = __float_as_uint(s[i < capi ? i : capi - 1]);
    }
  }
  const int64_t n = clamp_len(len_raw, cap);
  int32_t* out = idx + static_cast<int64_t>(row) * k;
  if (n <= k) {
    for (int64_t j = tid; j < k; j += kRT)
      out[j] = j < n ? static_cast<int32_t>(j) : -1;
    if (tid == 0 && count) count[row] = static_cast<int32_t>(n);
    return;
  }
  const int n32 = static_cast<int>(n);  // n <= 32,768 here
  // rounds holding elements, a scalar; each pass takes a fresh copy so no
  // per-round condition is kept from one pass to the next
  const int nr = __builtin_amdgcn_readfirstlane((n32 + kRT - 1) / kRT);
  auto rounds = [nr]() {
    int v = nr;
    asm volatile("" : "+s"(v));
    return v;
  };
  for (int i = tid; i < kCopies * kCopyPitch; i += kRT) h1[i] = 0u;
  h2[tid] = 0u;
  h3[tid] = 0u;
  __syncthreads();
  uint32_t* h1c = h1 + (lane & (kCopies - 1)) * kCopyPitch;
  {
    const int nr1 = rounds();
    const int lim = n32 - tid;  // round r of this lane is in the row iff r * 1024 < lim
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const uint32_t live = 0u - static_cast<uint32_t>(r * kRT < lim);
      key[r] = order_key(__uint_as_float(key[r])) & live;
      if (r < nr1) atomicAdd(&h1c[digit1(key[r])], 1u);
    }
  }
  __syncthreads();
  BinPick p1;
  {
    static_assert(kBins1 / kRT == 4, "one 16-byte run of bins per thread and copy");
    uint32_t h[4] = {0u, 0u, 0u, 0u};  // this thread's run of bins, from the top down
    const int base = kBins1 - (tid + 1) * 4;
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(h1 + q * kCopyPitch + base);
      h[0] += x.w;
      h[1] += x.z;
      h[2] += x.y;
      h[3] += x.x;
    }
    p1 = pick_bin_runs<kBins1, kRT>(h, static_cast<uint32_t>(k), lds, &pick);
  }
  {
    const int nr2 = rounds();
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (r < nr2 && digit1(key[r]) == p1.bin) atomicAdd(&h2[digit2(key[r])], 1u);
  }
  __syncthreads();
  const BinPick p2 = pick_bin<kBins2, kRT>(h2, k - p1.above, lds, &pick);
  const uint32_t pre = (p1.bin << kB2) | p2.bin;  // first 22 bits of T
  const uint32_t need2 = k - p1.above - p2.above;
  {
    const int nr3 = rounds();
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (r < nr3 && prefix12(key[r]) == pre) atomicAdd(&h3[key[r] & (kBins3 - 1)], 1u);
  }
  __syncthreads();
  const BinPick p3 = pick_bin<kBins3, kRT>(h3, need2, lds, &pick);
  const uint32_t T = (pre << kB3) | p3.bin;
  const uint32_t need = need2 - p3.above;  // ties at T to keep
  // counts above T and at T of every (round, wave) block, packed as
  // (ties << 16 | above) and scanned once: both totals are at most
  // n <= 32,768, so the low field never carries into the high one
  // lane r of `packed` collects round r's counts, so the wave stores them
  // with one LDS write
  const int nr4 = rounds();
  uint32_t packed = 0u;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const uint32_t g = static_cast<uint32_t>(__popcll(__ballot(key[r] > T)));
    const uint32_t q = static_cast<uint32_t>(__popcll(__ballot(key[r] == T)));
    packed = lane == r ? (r < nr4 ? (q << 16) | g : 0u) : packed;
  }
  if (lane < RPT) cnt_s[lane * kWavesR + wave] = packed;
  __syncthreads();
  {
    const uint32_t v = tid < kBlocks ? cnt_s[tid] : 0u;
    const uint32_t vb = block_exclusive_scan<kRT>(v, lds);
    if (tid < kBlocks) cnt_s[tid] = vb;
  }
  __syncthreads();
  const int pbl = lane < RPT ? static_cast<int>(cnt_s[lane * kWavesR + wave]) : 0;
  const int nr5 = rounds();
  // T again, opaque to the compiler: the comparisons below are recomputed
  // instead of keeping the counting pass's 2 * RPT wave masks live across
  // the scan (they spill)
  uint32_t Tp = T;
  asm volatile("" : "+v"(Tp));
  // set lanes of a wave mask below this lane
  auto below = [](uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
  };
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    if (r >= nr5) continue;
    const uint32_t pb = static_cast<uint32_t>(__builtin_amdgcn_readlane(pbl, r));
    const uint32_t gb = pb & 0xffffu, qb = pb >> 16;
    const bool gt = key[r] > Tp, eq = key[r] == Tp;
    const uint64_t me = __ballot(eq);
    bool kept = gt;
    uint64_t mk = __ballot(gt);
    if (me != 0) {  // uniform; ties at T in this block (rare)
      kept = gt || (eq && qb + below(me) < need);
      mk = __ballot(kept);
    }
    const uint32_t p = gb + (qb < need ? qb : need) + below(mk);
    if (kept && p < static_cast<uint32_t>(k)) out[p] = r * kRT + tid;
  }
  if (tid == 0 && count) count[row] = k;
}

int nch_for(int max_len) { return max_len > 0 ? (max_len + kChunk - 1) / kChunk : 1; }

}  // namespace

size_t topk_workspace(int rows, int max_len, int k) {
  (void)k;
  return static_cast<size_t>(topk_ws_words(rows, nch_for(max_len))) * sizeof(uint32_t);
}

int topk_max_len() { return kChunk * kMaxChunks; }

hipError_t launch_topk_clear(void* ws, int rows, hipStream_t s) {
  const int64_t words = topk_clear_words(rows);
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

// Filter passes per workgroup for FC chunks per pass: one, unless the
// launch would exceed about 1,024 workgroups, in which case a workgroup
// takes consecutive passes.
int filter_passes(int nch, int rows, int fc) {
  const int64_t per_row = (nch + fc - 1) / fc;
  int passes = 1;
  while (per_row * rows / passes > 1024 && passes < per_row) passes *= 2;
  return passes;
}

hipError_t launch_topk_finish(const float* scores, int64_t stride, int rows,
                              const int32_t* row_lens, int max_len, int k,
                              int32_t* idx, int32_t* count, void* ws,
                              hipStream_t s) {
  const int nch = nch_for(max_len);
  const int fc = static_cast<int64_t>(nch) * rows <= 256 ? 1
                 : filter_passes(nch, rows, 2) == 1 ? 2 : 4;
  const int passes = filter_passes(nch, rows, fc);
  const int64_t cap = max_len < stride ? max_len : stride;
  const int64_t per_row = (nch + fc - 1) / fc;
  dim3 grid(static_cast<uint32_t>((per_row + passes - 1) / passes),
            static_cast<uint32_t>(rows));
  hipLaunchKernelGGL(fc == 1 ? topk_filter_kernel<1>
                     : fc == 2 ? topk_filter_kernel<2> : topk_filter_kernel<4>, grid,
                     dim3(kFT), 0, s, scores, stride, row_lens, cap, k, nch,
                     passes, ws);
  const BlindPlan bp = blind_plan(nch, k, max_len);
  const int rb = bp.rounds;
  auto resolve = rb == 0 ? topk_resolve_kernel<0> : rb <= 2 ? topk_resolve_kernel<2>
               : rb <= 4 ? topk_resolve_kernel<4> : rb <= 8 ? topk_resolve_kernel<8>
               : topk_resolve_kernel<16>;
  hipLaunchKernelGGL(resolve, dim3(static_cast<uint32_t>(rows)), dim3(kRT), 0, s,
                     scores, stride, row_lens, cap, k, nch, bp.logE, ws, idx, count);
  return hipGetLastError();
}

// The one-workgroup path where it measured faster than the chunked one:
// rows of up to 24,576 entries; up to 32,768 with at least 64 rows (the
// chunked path's grid is then large) or when a chunk of 4,096 would keep
// about 400 entries or more (its 512-entry lists would overflow).
bool topk_small_fits(int max_len, int rows, int k) {
  if (max_len > kSmallMax) return false;
  if (max_len <= 24 * kRT) return true;
  return rows >= 64 || static_cast<int64_t>(k) * kChunk >= 400ll * max_len;
}

hipError_t launch_topk_small(const float* scores, int64_t stride, int rows,
                             const int32_t* row_lens, int max_len, int k,
                             int32_t* idx, int32_t* count, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t cap = max_len < stride ? max_len : stride;
  // rounds of 1,024 rounded up to a multiple of 4: a round past every row
  // still costs its load and its counting ballots
  const int rpt = (max_len + kRT - 1) / kRT;
  decltype(&topk_small_kernel<4>) kern;
  switch ((rpt + 3) / 4) {
    case 0:
    case 1: kern = topk_small_kernel<4>; break;
    case 2: kern = topk_small_kernel<8>; break;
    case 3: kern = topk_small_kernel<12>; break;
    case 4: kern = topk_small_kernel<16>; break;
    case 5: kern = topk_small_kernel<20>; break;
    case 6: kern = topk_small_kernel<24>; break;
    case 7: kern = topk_small_kernel<28>; break;
    default: kern = topk_small_kernel<32>; break;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(rows)), dim3(kRT), 0, s,
                     scores, stride, row_lens, cap, k, idx, count);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t stride, int rows,
                       const int32_t* row_lens, int max_len, int k,
                       int32_t* idx, int32_t* count, void* ws, bool zeroed,
                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipError_t e = zeroed ? hipSuccess : launch_topk_clear(ws, rows, s);
  if (e != hipSuccess) return e;
  if (topk_small_fits(max_len, rows, k))
    return launch_topk_small(scores, stride, rows, row_lens, max_len, k, idx,
                             count, s);
  e = launch_topk_hist1(scores, stride, rows, row_lens, max_len, k, ws, s);
  if (e != hipSuccess) return e;
  return launch_topk_finish(scores, stride, rows, row_lens, max_len, k, idx,
                            count, ws, s);
}

}  // namespace tsd
