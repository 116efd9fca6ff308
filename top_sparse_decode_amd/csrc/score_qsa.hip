// QSA-style index-K scan:
//   s[i][t] = sum_h w[i][h] * max(0, sum_d qi[i][h][d] * ki[slot(b,t)][d]).
// The indexer scores every cached token of the request with a 128-dim FP8
// index key and many index heads ("Context parallelism for QSA attention and
// the sparse indexer", Motivation: index-K store, score, top-k per row).
//
// Per key the contraction is 16 heads x 128 dims = 2048 MACs over 128 bytes,
// 32 flop per HBM byte: more than the FP32 vector units can sustain at HBM
// speed, so the decode scan runs each 16-key tile on the matrix cores (index
// heads as M, keys as N, the 128 dims as K). It uses the bf16 16x16x32 MFMA
// on exactly widened FP8 values rather than the FP8 16x16x128 MFMA: on this
// part the FP8 instruction drops low-order bits of its products while it
// adds them (measured: up to about 4e-4 of the largest product of a dot),
// while every product of two E4M3 values is exact in the bf16 instruction
// and its FP32 accumulation of the workloads' dots is exact, so the decode
// scores carry only the FP32 rounding of the weighted head sum. The kernel
// stays a single streaming pass over the index-K pages: every byte is read
// once, the query rows sit in registers for the whole scan.
//
// Work split: one wave owns one query row and a run of up to 32 consecutive
// 64-token pages; a page is 4 tiles of 16 keys. The 16x16 f32 result gives lane
// l the dots of key (l % 16) with heads 4*(l/16) .. 4*(l/16)+3; the weighted
// ReLU is applied per lane and a 3-shuffle reduce-scatter over the 4 lane
// groups leaves lane l with the full score of key l of the page, so a page
// stores 256 contiguous bytes of scores.
//
// A page is read as 8 contiguous 1 KB loads (lane l: bytes 16 l .. 16 l + 15
// of each KB, whole 128-byte lines per instruction) and transposed through
// LDS into the operand layout, lane (key c, k-group kb) taking bytes
// 32 kb .. 32 kb + 31 of key c; the query row's lanes take the same bytes, so
// every instruction pairs equal dims. Loads in the operand layout itself (64
// bytes of each of 16 keys per instruction, half of every line) read the
// pages 10-18 % slower on this part.
//
// The chunked-prefill kernel below is a dense contraction that is bound by
// the matrix cores, and it keeps the FP8 instruction at twice the bf16 rate;
// its scores carry that instruction's accumulation error.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

namespace tsd {
namespace {

constexpr int kWavesPerBlock = 4;
// Requests with at least this many query rows use the tiled prefill kernel.
constexpr int kPrefillMinRows = 64;
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

// Weighted ReLU of one lane's 4 heads of an MFMA tile, in a fixed order of
// rounding (written out with fmaf so that no contraction choice of the
// compiler changes it): both index kernels call it.
TSD_DEVICE float weighted_relu4(v4f d, float w0, float w1, float w2, float w3) {
  const float m0 = fmaxf(d[0], 0.f), m1 = fmaxf(d[1], 0.f);
  const float m2 = fmaxf(d[2], 0.f), m3 = fmaxf(d[3], 0.f);
  return fmaf(w3, m3, fmaf(w2, m2, fmaf(w0, m0, w1 * m1)));
}

// Bytes 32 kb .. 32 kb + 31 of a 128-byte FP8 row: the decode scan's
// operand slice, for its query rows (global memory) and its keys (LDS).
TSD_DEVICE v8i load_row_chunk32(const uint8_t* row, int kb) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row + 32 * kb);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + 32 * kb + 16);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// The 32 FP8 codes of a lane's operand slice (as the row loaders pack them)
// widened exactly to bf16 (every E4M3 value is a bf16 value) as the four
// operands of the bf16 16x16x32 MFMA: operand s holds the codes of dwords
// 2s and 2s + 1. Index heads and keys are widened the same way, so each
// instruction still pairs dims of q with the same dims of k.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
struct Bf16Slice {
  v8bf s[4];
};

TSD_DEVICE Bf16Slice widen_fp8(v8i v) {
  Bf16Slice r;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w = static_cast<uint32_t>(v[2 * s + j]);
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
      r.s[s][4 * j + 0] = lo[0];
      r.s[s][4 * j + 1] = lo[1];
      r.s[s][4 * j + 2] = hi[0];
      r.s[s][4 * j + 3] = hi[1];
    }
  return r;
}

// 16 heads x 16 keys x 128 dims on the bf16 MFMA, FP32 accumulation.
TSD_DEVICE v4f mfma_bf16_dot(const Bf16Slice& a, v8i b_fp8) {
  const Bf16Slice b = widen_fp8(b_fp8);
  v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.s[s], b.s[s], c, 0, 0, 0);
  return c;
}

TSD_DEVICE v4f mfma_fp8(v8i a, v8i b) {
  v4f c = {0.f, 0.f, 0.f, 0.f};
  // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0,
                                                          127, 0, 127);
}

// One wave owns G consecutive pages of one row. Pages are contracted in
// pairs with the next pair's loads already in flight (two register sets of
// 2 pages x 8 contiguous 16-byte loads per lane); each page passes through
// the wave's LDS staging rows half a page (32 keys, two tiles) at a time, at
// a 144-byte row pitch, so that the contiguous stores and the operand reads
// (lanes c = 0..15 of one k-group at 36 c mod 64 banks) are conflict-free.
// The wave's scores are staged in LDS and stored in one burst after its
// last page: stores issued between the loads would share the loads'
// completion counter and stall every later wait on them.
//
// HIST: also accumulate the first top-k radix digit of every written score
// into the top-k workspace's digit-1 histograms (LDS-privatised per
// workgroup, flushed with integer atomics). The launch then gives each row
// a multiple of 4 waves so that a workgroup never spans two rows, and no
// wave leaves before the barriers.
//
// The arguments that the first loads' addresses need come first: they fill
// the 14 kernel-argument dwords the hardware preloads into scalar registers,
// so those loads leave without waiting for the argument buffer.
template <int G, bool HIST>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void qsa_scan_kernel(
    int rows, int rows_per_req, int H_i, int waves_per_row,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const uint8_t* __restrict__ index_q,
    const float* __restrict__ index_w, const uint8_t* __restrict__ index_k,
    const int32_t* __restrict__ q_pos, int64_t num_pages,
    float* __restrict__ scores, int64_t score_stride,
    int32_t* __restrict__ row_lens_out, void* __restrict__ topk_base,
    int hist_k) {
  static_assert(G % 4 == 0 && G <= kWave, "pages per wave: one page id per lane");
  constexpr int kStRows = kPage / 2;   // keys staged at a time
  constexpr int kStPitch = kDi + 16;   // LDS bytes per staged key
  __shared__ __align__(16) uint32_t hist_s[HIST ? kTopkBins1 : 4];
  __shared__ float res_s[kWavesPerBlock][G * kPage];
  __shared__ __align__(16) uint8_t kst_s[kWavesPerBlock][kStRows * kStPitch];
  const int lane = threadIdx.x & (kWave - 1);
  // the wave's index is uniform: held in scalar registers, so the row and
  // request divisions run once per wave on the scalar unit
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kWavesPerBlock + wl;
  const int row = wave / waves_per_row;
  const bool row_ok = row < rows;
  const int chunk = wave - row * waves_per_row;
  const int b = row_ok ? row / rows_per_req : 0;
  const int64_t page0 = static_cast<int64_t>(chunk) * G;
  const int col = lane & 15;  // MFMA row (head) for A, column (key) for B
  const int kb = lane >> 4;   // which 32-byte slice of the 128 dims
  const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride;

  // The row's length, the wave's page ids (lane l: page page0 + l, clamped
  // inside the row's pt_stride entries; only those below the length are
  // used), the row's index-query slice and its head weights are all loaded
  // before the length is known, so the key loads wait for one round trip.
  int64_t n = 0;
  int32_t pt_raw = -1;
  v8i qa8 = {0, 0, 0, 0, 0, 0, 0, 0};
  float w[4] = {0.f, 0.f, 0.f, 0.f};
  if (row_ok) {
    n = seq_lens[b];
    const int64_t pi = page0 + lane;
    pt_raw = pt[pi < pt_stride ? pi : pt_stride - 1];
    // A operand: index head `col` of this row (zero for padded heads);
    // the weights of the 4 heads whose dots this lane receives
    if (col < H_i)
      qa8 = load_row_chunk32(
          index_q + (static_cast<int64_t>(row) * H_i + col) * kDi, kb);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * kb + v;
      w[v] = h < H_i ? index_w[static_cast<int64_t>(row) * H_i + h] : 0.f;
    }
    if (q_pos) {
      const int64_t p1 = static_cast<int64_t>(q_pos[row]) + 1;
      n = p1 < n ? p1 : n;
    }
    n = clamp_len(n, pt_stride * kPage);
    n = clamp_len(n, score_stride);
    if (chunk == 0 && lane == 0 && row_lens_out)
      row_lens_out[row] = static_cast<int32_t>(n);
  }
  // live pages of this wave (the last one may be partial)
  int npg = 0;
  if (row_ok && page0 * kPage < n) {
    const int64_t left = (n - page0 * kPage + kPage - 1) / kPage;
    npg = left < G ? static_cast<int>(left) : G;
  }
  const bool do_hist = HIST && row_ok && n > hist_k;
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kTopkBins1; i += kWavesPerBlock * kWave)
      hist_s[i] = 0u;
    __syncthreads();
  } else {
    if (npg == 0) return;
  }

  if (npg > 0) {
    const Bf16Slice qa = widen_fp8(qa8);
    float* res = res_s[wl];
    // every page id of the wave up front, lane l holding page l: a page-id
    // load inside the loop would make each wait on it also drain the other
    // register set's key loads (loads complete in order)
    const int32_t my_page = lane < npg ? pt_raw : -1;

    // loads of wave pages j, j+1. They are unconditional, so the compiler
    // knows how many loads follow the ones it waits for (loads complete in
    // order) and the other register set's loads stay in flight: a page past
    // npg or outside [0, num_pages) reads page 0 (which exists, num_pages >=
    // 1 here) and scores -inf. The index keys are read once per step, so
    // the loads are non-temporal.
    auto load2 = [&](int j, v4u (&kt)[2][8], bool (&valid)[2]) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const bool live = j + d < npg;
        const int32_t page =
            live ? __builtin_amdgcn_readlane(my_page, j + d) : -1;
        valid[d] = page >= 0 && page < num_pages;
        const uint8_t* base =
            index_k + static_cast<int64_t>(valid[d] ? page : 0) * kPage * kDi;
#pragma unroll
        for (int m = 0; m < 8; ++m)  // keys 8m .. 8m + 7, 16 bytes per lane
          kt[d][m] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u*>(base + 1024 * m) + lane);
      }
    };
    uint8_t* kst = kst_s[wl];
    auto score2 = [&](int j, const v4u (&kt)[2][8], const bool (&valid)[2]) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        if (j + d >= npg) break;  // uniform
        float part[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // keys 32h .. 32h + 31
          // LDS operations of one wave run in order: every lane's staged
          // bytes are in place before the operand reads, and the reads are
          // done before the next half overwrites them
#pragma unroll
          for (int m = 0; m < 4; ++m)
            *reinterpret_cast<v4u*>(kst + (8 * m + (lane >> 3)) * kStPitch +
                                    16 * (lane & 7)) = kt[d][4 * h + m];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const v8i kb8 = load_row_chunk32(kst + (16 * i + col) * kStPitch, kb);
            const v4f dd = mfma_bf16_dot(qa, kb8);
            part[2 * h + i] = weighted_relu4(dd, w[0], w[1], w[2], w[3]);
          }
          __builtin_amdgcn_wave_barrier();
        }
        // reduce-scatter over the 4 lane groups: lane l gets key l
        const float red = reduce_scatter4(part);
        const float sc = valid[d] ? red : -__builtin_inff();
        res[(j + d) * kPage + lane] = sc;
        const int64_t t = (page0 + j + d) * kPage + lane;
        if (do_hist && t < n)
          atomicAdd(&hist_s[topk_digit1(order_key(sc))], 1u);
      }
    };
    v4u ka[2][8], kc[2][8];
    bool va[2], vc[2];
    if (num_pages > 0) {
      load2(0, ka, va);
      int j = 0;
#pragma unroll 1
      for (; j + 4 < npg; j += 4) {  // the next 4 pages' loads always in flight
        load2(j + 2, kc, vc);
        score2(j, ka, va);
        load2(j + 4, ka, va);
        score2(j + 2, kc, vc);
      }
      if (j + 2 < npg) load2(j + 2, kc, vc);  // the last 1 to 4 pages
      score2(j, ka, va);
      score2(j + 2, kc, vc);
    } else {  // an empty pool: every page is outside it
#pragma unroll 1
      for (int e = lane; e < npg * kPage; e += kWave) res[e] = -__builtin_inff();
      if (do_hist)
        for (int e = lane; e < npg * kPage; e += kWave)
          if ((page0 * kPage + e) < n)
            atomicAdd(&hist_s[topk_digit1(order_key(-__builtin_inff()))], 1u);
    }
    // the wave's scores are contiguous in the row: one burst of stores
    // (LDS order within the wave makes every lane's staged score visible)
    __builtin_amdgcn_wave_barrier();
    float* out = scores + static_cast<int64_t>(row) * score_stride + page0 * kPage;
    const int64_t cnt64 = n - page0 * kPage;
    const int cnt = cnt64 < npg * kPage ? static_cast<int>(cnt64) : npg * kPage;
#pragma unroll 4
    for (int e = lane; e < cnt; e += kWave) out[e] = res[e];
  }

  if constexpr (HIST) {
    __syncthreads();
    if (do_hist) {  // uniform: the workgroup lies in one row
      const TopkWs ws = topk_ws(topk_base, rows, 0);
      topk_flush_h1<kWavesPerBlock * kWave>(
          hist_s, ws.h1 + static_cast<int64_t>(row) * kTopkBins1);
    }
  }
}

// ---------------------------------------------------------------------------
// Chunked-prefill indexer: many causal query rows of one request against the
// request's index keys -- a dense FP8 contraction (rows x 16 heads) x keys x
// 128 dims with the weighted-ReLU head reduction as epilogue.
//
// A workgroup of 8 waves owns 64 consecutive query rows of one request (8
// per wave, their index heads held as MFMA A operands and their head weights
// in registers, 2 waves per SIMD) and a span of 16,384 keys whose page ids it
// keeps in LDS. The span is walked in blocks of 512 keys (8 pages) that the
// workgroup gathers once into LDS, the next block's loads in flight during
// the current one; every wave then takes each 16-key tile of the block as a
// B operand and issues one MFMA per row, so each key byte read from memory
// feeds 64 rows. The per-row epilogue (weighted_relu4) and the cross-lane
// reduce-scatter are the decode scan's; the dots come from the FP8 MFMA.
// Keys past a row's causal limit are computed but never stored.
constexpr int kPfWaves = 8;
constexpr int kPfRowsPerWave = 8;
constexpr int kPfRows = kPfWaves * kPfRowsPerWave;  // rows per workgroup
constexpr int kPfBlockKeys = 512;                   // keys per LDS block
constexpr int kPfSpanBlocks = 32;                   // blocks per workgroup
constexpr int kPfSpan = kPfBlockKeys * kPfSpanBlocks;
constexpr int kPfPitch = kDi + 16;                  // LDS bytes per key

TSD_DEVICE v8i lds_row_slice(const uint8_t* row, int kb) {
  const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * kb);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + 64 + 16 * kb);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// Gathers the 512 keys of block `key0` (8 pages) into registers: thread tid
// holds 16-byte vectors tid, tid + 512, ... of the block; keys at or past the
// workgroup's longest row, or on an invalid page, read as zeros.
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfVecs = kPfBlockKeys * 8;  // 16-byte vectors per block
constexpr int kPfVecsPerThread = (kPfVecs + kPfThreads - 1) / kPfThreads;
struct PfStage {
  uint4 x[kPfVecsPerThread];
};

// Page ids come from the workgroup's LDS copy of its span's page-table
// entries, so the key loads issue without waiting on earlier memory
// operations (a page-id load from memory would wait on the vector-memory
// counter, which also counts every score store still in flight).
TSD_DEVICE void pf_load(PfStage& st, const uint8_t* __restrict__ index_k,
                        const int32_t* pages_s, int64_t span0, int64_t key0,
                        int64_t n_wg, int tid) {
#pragma unroll
  for (int it = 0; it < kPfVecsPerThread; ++it) {
    const int v = tid + it * kPfThreads;
    const int64_t t = key0 + (v >> 3);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (v < kPfVecs && t < n_wg) {
      const int32_t page = pages_s[(t - span0) / kPage];
      if (page >= 0)
        x = *reinterpret_cast<const uint4*>(
            index_k + (static_cast<int64_t>(page) * kPage + t % kPage) * kDi +
            16 * (v & 7));
    }
    st.x[it] = x;
  }
}

TSD_DEVICE void pf_store(const PfStage& st, uint8_t* keys_s, int tid) {
#pragma unroll
  for (int it = 0; it < kPfVecsPerThread; ++it) {
    const int v = tid + it * kPfThreads;
    if (v < kPfVecs)
      *reinterpret_cast<uint4*>(keys_s + (v >> 3) * kPfPitch + 16 * (v & 7)) =
          st.x[it];
  }
}

__global__ __launch_bounds__(kPfWaves * kWave) void qsa_prefill_kernel(
    const uint8_t* __restrict__ index_q, const float* __restrict__ index_w,
    const uint8_t* __restrict__ index_k, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_pos, int64_t num_pages, int rows_per_req,
    int groups_per_req, int H_i, float* __restrict__ scores,
    int64_t score_stride, int32_t* __restrict__ row_lens_out) {
  // two key blocks: the next one is gathered while the current one is used
  __shared__ __align__(16) uint8_t keys_s[2][kPfBlockKeys * kPfPitch];
  // physical page of each page of the span, -1 past the length or invalid
  __shared__ int32_t pages_s[kPfSpan / kPage];
  __shared__ int64_t nmax_s[kPfWaves], nmin_s[kPfWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y / groups_per_req;
  const int grp_in_req = blockIdx.y - b * groups_per_req;
  const int row0 = grp_in_req * kPfRows;  // first row of the group within b
  const int64_t span0 = static_cast<int64_t>(blockIdx.x) * kPfSpan;
  const int64_t len = clamp_len(clamp_len(seq_lens[b], pt_stride * kPage),
                                score_stride);
  const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride;
  const int col = lane & 15, kb = lane >> 4;

  // this wave's rows: A operands, key counts and, per lane, the weights of
  // the 4 heads its MFMA output rows hold (4*kb .. 4*kb+3)
  v8i qa[kPfRowsPerWave];
  float4 wq[kPfRowsPerWave];
  int32_t nr[kPfRowsPerWave];  // key count of each row (n <= 2^31 - 1)
  int64_t nmax = 0, nmin = INT64_MAX;
#pragma unroll
  for (int i = 0; i < kPfRowsPerWave; ++i) {
    const int rr = row0 + wave * kPfRowsPerWave + i;  // row within request
    const bool ok = rr < rows_per_req;
    const int64_t row = static_cast<int64_t>(b) * rows_per_req + rr;
    int64_t n = 0;
    if (ok) {
      n = len;
      if (q_pos) {
        const int64_t p1 = static_cast<int64_t>(q_pos[row]) + 1;
        n = p1 < n ? (p1 < 0 ? 0 : p1) : n;
      }
      if (blockIdx.x == 0 && lane == 0 && row_lens_out)
        row_lens_out[row] = static_cast<int32_t>(n);
    }
    // n is the same in every lane; keep it scalar so row tests are uniform
    nr[i] = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(n));
    nmax = n > nmax ? n : nmax;
    nmin = n < nmin ? n : nmin;
    qa[i] = (ok && col < H_i)
                ? load_row_slice(index_q + (row * H_i + col) * kDi, kb)
                : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    float w4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      w4[c] = (ok && 4 * kb + c < H_i) ? index_w[row * H_i + 4 * kb + c] : 0.f;
    wq[i] = make_float4(w4[0], w4[1], w4[2], w4[3]);
  }
  if (lane == 0) {
    nmax_s[wave] = nmax;
    nmin_s[wave] = nmin;
  }
  for (int i = tid; i < kPfSpan / kPage; i += kPfThreads) {
    const int64_t t = span0 + static_cast<int64_t>(i) * kPage;
    int32_t page = t < len ? pt[t / kPage] : -1;
    pages_s[i] = page >= 0 && page < num_pages ? page : -1;
  }
  __syncthreads();
  int64_t n_wg = 0;
#pragma unroll
  for (int i = 0; i < kPfWaves; ++i) n_wg = nmax_s[i] > n_wg ? nmax_s[i] : n_wg;
  int nblk = 0;  // blocks of this span below the longest row
  while (nblk < kPfSpanBlocks &&
         span0 + static_cast<int64_t>(nblk) * kPfBlockKeys < n_wg)
    ++nblk;
  if (nblk == 0) return;  // uniform over the workgroup
  int64_t n_min = nmin_s[0];  // shortest row of the workgroup
#pragma unroll
  for (int i = 1; i < kPfWaves; ++i) n_min = nmin_s[i] < n_min ? nmin_s[i] : n_min;
  int nfull = 0;  // leading blocks below every row's key count
  while (nfull < nblk &&
         span0 + static_cast<int64_t>(nfull + 1) * kPfBlockKeys <= n_min)
    ++nfull;

  PfStage st;
  pf_load(st, index_k, pages_s, span0, span0, n_wg, tid);
  pf_store(st, keys_s[0], tid);
  __syncthreads();

  // One block: the next block's loads stay in flight during this block's
  // math. MASKED adds the causal store guard; blocks whose keys all lie
  // below every row's limit store unconditionally, so the number of stores
  // issued after the loads is fixed and waiting for the loads does not wait
  // for the stores as well (loads and stores share one completion counter).
  auto block = [&](int blk, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int cur = blk & 1;
    const int64_t key0 = span0 + static_cast<int64_t>(blk) * kPfBlockKeys;
    const bool more = blk + 1 < nblk;
    if (more)
      pf_load(st, index_k, pages_s, span0, key0 + kPfBlockKeys, n_wg, tid);
    const uint8_t* ks = keys_s[cur];
#pragma unroll 1
    for (int g4 = 0; g4 < kPfBlockKeys / 64; ++g4) {
      const int64_t t = key0 + 64 * g4 + lane;
      v8i kt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kt[i] = lds_row_slice(ks + (64 * g4 + 16 * i + col) * kPfPitch, kb);
      // as in the decode scan, a key on a page outside [0, num_pages)
      // scores -inf (the 64-key group is exactly one page)
      const bool page_ok = pages_s[blk * (kPfBlockKeys / kPage) + g4] >= 0 ||
                           key0 + 64 * g4 >= len;
      // Per row: the four tiles' MFMAs go out back to back into separate
      // accumulators (a scheduling barrier keeps the epilogue behind them),
      // so one MFMA latency is exposed per row instead of one per tile. On
      // this part MFMA and VALU work of one SIMD do not overlap, so issuing
      // the next row's MFMAs ahead of the epilogue gains nothing. Every row
      // computes every tile; causality is enforced by the store guard.
#pragma unroll
      for (int i = 0; i < kPfRowsPerWave; ++i) {
        const float4 wv = wq[i];
        v4f d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = mfma_fp8(qa[i], kt[j]);
        __builtin_amdgcn_sched_barrier(0);
        float part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          part[j] = weighted_relu4(d[j], wv.x, wv.y, wv.z, wv.w);
        const float red = reduce_scatter4(part);
        const float sc = page_ok ? red : -__builtin_inff();
        const int64_t row = static_cast<int64_t>(b) * rows_per_req + row0 +
                            wave * kPfRowsPerWave + i;
        // non-temporal: 8.6 GB of scores per pass, read back by the top-k
        // passes from memory anyway (2 % faster than a plain store)
        if (!MASKED || t < nr[i])
          __builtin_nontemporal_store(sc, scores + row * score_stride + t);
      }
    }
    if (more) pf_store(st, keys_s[cur ^ 1], tid);
    __syncthreads();  // next block landed; this one is no longer read
  };
  int blk = 0;
  for (; blk < nfull; ++blk) block(blk, std::false_type{});
  for (; blk < nblk; ++blk) block(blk, std::true_type{});
}

}  // namespace

hipError_t launch_qsa_scan(const tsd_score_args& a, hipStream_t s,
                           void* topk_ws, int hist_k) {
  const int rows = a.B * a.rows_per_req;
  if (rows == 0) return hipSuccess;
  if (!topk_ws && a.rows_per_req >= kPrefillMinRows) {
    const int64_t keys = a.pt_stride * kPage < a.score_stride
                             ? a.pt_stride * kPage : a.score_stride;
    const int groups = (a.rows_per_req + kPfRows - 1) / kPfRows;
    dim3 grid(static_cast<uint32_t>((keys + kPfSpan - 1) / kPfSpan),
              static_cast<uint32_t>(a.B * groups));
    hipLaunchKernelGGL(qsa_prefill_kernel, grid, dim3(kPfWaves * kWave), 0, s,
                       a.index_q, a.index_w, a.index_k_pool, a.page_table,
                       a.pt_stride, a.seq_lens, a.q_pos, a.num_pages,
                       a.rows_per_req, groups, a.H_i, a.scores, a.score_stride,
                       a.row_lens_out);
    return hipGetLastError();
  }
  // pages per wave: the most (up to 32) that still gives >= 1,024 waves;
  // at 32 a workgroup's LDS (scores, staging rows, histogram: 66 KB) and
  // its 4 waves' registers leave room for two workgroups per CU
  const int64_t pages = a.pt_stride * static_cast<int64_t>(rows);
  int G = 32;
  while (G > 4 && pages / G < 1024) G /= 2;
  int64_t waves_per_row = (a.pt_stride + G - 1) / G;
  if (topk_ws)  // whole workgroups per row
    waves_per_row = (waves_per_row + kWavesPerBlock - 1) / kWavesPerBlock *
                    kWavesPerBlock;
  const int64_t waves = waves_per_row * rows;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  using Kern = void (*)(int, int, int, int, const int32_t*, const int32_t*,
                        int64_t, const uint8_t*, const float*, const uint8_t*,
                        const int32_t*, int64_t, float*, int64_t, int32_t*,
                        void*, int);
  Kern kern;
  if (topk_ws)
    kern = G == 32 ? qsa_scan_kernel<32, true>
         : G == 16 ? qsa_scan_kernel<16, true>
         : G == 8  ? qsa_scan_kernel<8, true> : qsa_scan_kernel<4, true>;
  else
    kern = G == 32 ? qsa_scan_kernel<32, false>
         : G == 16 ? qsa_scan_kernel<16, false>
         : G == 8  ? qsa_scan_kernel<8, false> : qsa_scan_kernel<4, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(blocks)),
                     dim3(kWavesPerBlock * kWave), 0, s, rows, a.rows_per_req,
                     a.H_i, static_cast<int>(waves_per_row), a.seq_lens,
                     a.page_table, a.pt_stride, a.index_q, a.index_w,
                     a.index_k_pool, a.q_pos, a.num_pages, a.scores,
                     a.score_stride, a.row_lens_out, topk_ws, hist_k);
  return hipGetLastError();
}

}  // namespace tsd
