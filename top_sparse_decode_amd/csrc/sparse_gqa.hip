// Sparse GQA decode attention over the selected tokens, split into chunks
// with FP32 partial outputs and log-sum-exps ("QSA cache sharding", sglang
// PR #43527, Distributed QSA execution: sparse attention over the selected
// tokens, partial outputs merged by FP32 log-sum-exp; "Context parallelism
// for QSA attention and the sparse indexer": a sparse GQA call per block).
//
// One workgroup (8 waves for FP8 rows, 4 for 16-bit rows) per (request b,
// KV head g, chunk c) handles the G query heads of the group over the
// chunk's run of the ascending selection list (every token 0 .. len-1 for a
// request at or below the sparse-decode threshold), one tile of tokens at a
// time (128 tokens for FP8 rows, 64 for 16-bit rows, so a tile's K and V
// fit LDS):
//   1. the tile's slots are resolved from the page table; an index outside
//      [0, len) or a page outside [0, num_pages) is masked and never read;
//   2. the K and V rows are gathered into LDS with 16-byte loads (a token's
//      row is contiguous in the token-major pool), masked rows zero-filled;
//   3. logits S = Q K^T on MFMA: v_mfma_f32_16x16x32_{bf16,f16} with the
//      group's query heads as M (padded to 16), 16 tokens as N and 32 head
//      dims per instruction as K. FP8 K is widened exactly to the query's
//      16-bit type, so the products are exact and accumulate in FP32;
//   4. an online softmax (base 2) per head updates the running max and sum;
//      the page's V scale is folded into the probabilities;
//   5. O += P V on MFMA, each wave owning 128 / waves output dimensions of
//      every head: for 16-bit caches on v_mfma_f32_16x16x32_{bf16,f16} with
//      P as the sum of two 16-bit parts (within 2^-17 of P) and V as stored;
//      for FP8 caches with P rounded once to bf16 and V widened exactly.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <int ENC>
struct Tile {
  static constexpr int kEsz = ENC == TSD_FP8_E4M3 ? 1 : 2;
  static constexpr int kTokens = ENC == TSD_FP8_E4M3 ? 128 : 64;
  static constexpr int kRowBytes = kD * kEsz;
  static constexpr int kPitch = kRowBytes + 16;      // LDS row pitch (bytes)
  // V rows: the P.V step reads, per lane group, 8 consecutive rows of one
  // column range, the groups 8 rows apart. 32 more bytes after every 8 rows
  // keep the groups off each other's banks (8 rows of a 16-byte aligned
  // pitch span a multiple of 32 banks). 16-bit rows are 288 bytes apart, 8
  // banks mod 32, so the 4 rows one 16-lane transpose load touches lie in
  // disjoint banks.
  static constexpr int kVPitch = ENC == TSD_FP8_E4M3 ? kPitch : kRowBytes + 32;
  static constexpr int kVPad = 32;
  static constexpr int kVBytes = kTokens * kVPitch + (kTokens / 8) * kVPad;
  static constexpr __host__ __device__ int vrow(int t) { return t * kVPitch + (t >> 3) * kVPad; }
  // waves per workgroup: an FP8 tile is short on arithmetic per byte, so
  // twice the waves split each phase of a tile (one 16-token block per wave,
  // 16 output dimensions per wave)
  static constexpr int kWaves = ENC == TSD_FP8_E4M3 ? 8 : 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlocks = kTokens / 16 / kWaves;  // 16-token blocks per wave
  static constexpr int kDW = kD / kWaves;  // output dimensions per wave
  static constexpr int kJ = kDW / 16;      // 16-wide MFMA column blocks per wave
  // logits / probs pitch (floats): 16-byte aligned rows for the 8-wide P
  // reads of the P.V step
  static constexpr int kZPitch = kTokens + 4;
};

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two FP8 E4M3 codes (the low or, with HI, the high half of w) widened to a pair of
// 16-bit values (QBF: bf16, else fp16) by the hardware converter at scale
// 1; exact, since every E4M3 value is a bf16 and an fp16 value.
template <bool QBF, bool HI>
TSD_DEVICE uint32_t widen2(uint32_t w) {
  if constexpr (QBF)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// 8 consecutive 16-bit values (as raw bits) starting at element `e0` of a
// K row in LDS, in the encoding of the query (QBF: bf16, else fp16).
template <int ENC, bool QBF>
TSD_DEVICE uint4 k8_as_q(const uint8_t* row, int e0) {
  if constexpr (ENC == TSD_FP8_E4M3) {
    const uint2 raw = *reinterpret_cast<const uint2*>(row + e0);
    return make_uint4(widen2<QBF, false>(raw.x), widen2<QBF, true>(raw.x),
                      widen2<QBF, false>(raw.y), widen2<QBF, true>(raw.y));
  } else {
    return *reinterpret_cast<const uint4*>(row + 2 * e0);
  }
}

typedef short v4s __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose load of 16-bit elements (ds_read_b64_tr_b16): within
// each 16-lane group, lane i receives element i % 4 of the 8-byte segments
// that lanes 4m + i / 4 point at, for m = 0 .. 3.
TSD_DEVICE v4s lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(p));
}

template <bool QBF>
TSD_DEVICE v4f mfma_qk(uint4 a, uint4 b, v4f c) {
  if constexpr (QBF) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
}

// The arguments that the first loads' addresses need come first: they fill
// the 14 kernel-argument dwords the hardware preloads into scalar registers,
// so those loads leave without waiting for the argument buffer.
template <int ENC, bool QBF>
__global__ __launch_bounds__(Tile<ENC>::kThreads) void sparse_gqa_kernel(
    int H_q, int H_kv, int H_sel, int k, int C, int lbs,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ count, const uint16_t* __restrict__ q,
    int64_t pt_stride, const int32_t* __restrict__ page_table,
    int64_t num_pages, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, float softmax_scale, int dense_len,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  using T = Tile<ENC>;
  constexpr int NT = T::kTokens;
  constexpr int kThreads = T::kThreads, kWavesW = T::kWaves;
  constexpr bool fp8 = ENC == TSD_FP8_E4M3;
  __shared__ __align__(16) uint8_t k_s[NT * T::kPitch];
  __shared__ __align__(16) uint8_t v_s[T::kVBytes];
  __shared__ float zp_s[16 * T::kZPitch];  // logits, then probabilities
  __shared__ int64_t slot_s[NT];
  __shared__ float ks_s[NT], vs_s[NT];
  __shared__ float m_s[16], l_s[16], alpha_s[16];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = H_q / H_kv;
  const int h0 = g * G;
  const int srow = H_sel == 1 ? 0 : g;
  const int32_t* sel = idx + (static_cast<int64_t>(b) * H_sel + srow) * k;
  // Entries are token indices (lbs = 0) or ascending indices of blocks of
  // 2^lbs tokens, position p of the selection then being token
  // sel[p >> lbs] * 2^lbs + p % 2^lbs (only a last block can be partial).
  // The chunk bounds depend on the selection's length m, which is the full
  // capacity for every row long enough: the first tile's entries for that m
  // (and, for blocks, the last entry) are loaded together with the length
  // and the count, from the request's row of idx (allocated for every
  // request), and kept wherever they match the real bounds.
  const int bsz = 1 << lbs;
  // capacity in tokens, at most 4,096 * 64, so (c + 1) * cap fits 32 bits
  const int cap = k << lbs;
  auto token_at = [&](int64_t p) -> int64_t {
    if (lbs == 0) return sel[p];
    return static_cast<int64_t>(sel[p >> lbs]) * bsz + (p & (bsz - 1));
  };
  const int lo_s = c * cap / C;
  const int hi_s = (c + 1) * cap / C;
  int64_t t_spec = -1;
  if (tid < NT && lo_s + tid < hi_s) t_spec = token_at(lo_s + tid);
  const int32_t last_spec = lbs > 0 ? sel[k - 1] : -1;
  const int64_t n = clamp_len(seq_lens[b], pt_stride * kPage);
  // at or below the sparse-decode threshold the selection is every token
  const bool dense = n <= dense_len;
  int64_t m = n;
  if (!dense) {
    const int64_t cnt = clamp_len(count[static_cast<int64_t>(b) * H_sel + srow], k);
    m = cnt << lbs;
    if (lbs > 0 && cnt > 0) {  // drop the part of the last block past len
      const int32_t last = cnt == k ? last_spec : sel[cnt - 1];
      const int64_t over = (static_cast<int64_t>(last) + 1) * bsz - n;
      m -= over < 0 ? 0 : (over > bsz ? bsz : over);
    }
  }
  int64_t lo, hi;
  if (m <= (1 << 24)) {  // 32-bit division whenever (c + 1) * m fits
    const int mi = static_cast<int>(m);
    lo = c * mi / C;
    hi = (c + 1) * mi / C;
  } else {
    lo = c * m / C;
    hi = (c + 1) * m / C;
  }
  const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride;
  const float zscale = softmax_scale * kLog2e;

  const int col = lane & 15;   // MFMA row (A) / column (B) index
  const int grp = lane >> 4;   // MFMA k-group / output row group

  // Q operand: head `col` of the group, dims 32*grp .. 32*grp+31 in four
  // 8-wide steps; rows past G are zero.
  uint4 qa[4];
  {
    const bool live = col < G;
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + (static_cast<int64_t>(b) * H_q + h0 + (live ? col : 0)) * kD +
        32 * grp);
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = live ? qp[s] : make_uint4(0, 0, 0, 0);
  }
  if (tid < 16) {
    m_s[tid] = -__builtin_inff();
    l_s[tid] = 0.f;
  }
  // PV accumulators: O[4*grp + v][kDW*wave + 16*j + col]
  v4f acc[T::kJ];
#pragma unroll
  for (int j = 0; j < T::kJ; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t base = lo; base < hi; base += NT) {
    const int tn = static_cast<int>(hi - base < NT ? hi - base : NT);
    // 1. resolve slots; the page-scale loads stay in flight and are stored
    // to LDS after the K/V gather has been issued (the barrier waits for LDS
    // operations only)
    float ksc = 0.f, vsc = 0.f;
    if (tid < NT) {
      int64_t slot = -1;
      if (tid < tn) {
        const bool spec = !dense && base == lo_s && lo_s + tid < hi_s;
        const int64_t t = dense ? base + tid : (spec ? t_spec : token_at(base + tid));
        if (t >= 0 && t < n) {
          const int32_t page = pt[t / kPage];
          if (page >= 0 && page < num_pages) {
            slot = static_cast<int64_t>(page) * kPage + t % kPage;
            ksc = fp8 ? k_scale[page] : 1.f;
            vsc = fp8 ? v_scale[page] : 1.f;
          }
        }
      }
      slot_s[tid] = slot;
    }
    __syncthreads();
    // 2. gather K and V rows (16-byte vectors; masked rows become zeros):
    // every load of the tile is issued before the first LDS store
    constexpr int vpr = T::kRowBytes / 16;
    constexpr int kIt = NT * vpr / kThreads;
    static_assert(NT * vpr % kThreads == 0, "gather split");
    uint4 kx[kIt], vx[kIt];
    int64_t slots[kIt];  // all LDS reads first: one wait covers them
#pragma unroll
    for (int it = 0; it < kIt; ++it) slots[it] = slot_s[(tid + it * kThreads) / vpr];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int i = tid + it * kThreads;
      const int v = i % vpr;
      const int64_t slot = slots[it];
      kx[it] = make_uint4(0, 0, 0, 0);
      vx[it] = make_uint4(0, 0, 0, 0);
      if (slot >= 0) {
        const int64_t off = (slot * H_kv + g) * T::kRowBytes + 16 * v;
        kx[it] = *reinterpret_cast<const uint4*>(k_pool + off);
        vx[it] = *reinterpret_cast<const uint4*>(v_pool + off);
      }
    }
    if (tid < NT) {
      ks_s[tid] = ksc;
      vs_s[tid] = vsc;
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int i = tid + it * kThreads;
      const int j = i / vpr, v = i % vpr;
      *reinterpret_cast<uint4*>(k_s + j * T::kPitch + 16 * v) = kx[it];
      *reinterpret_cast<uint4*>(v_s + T::vrow(j) + 16 * v) = vx[it];
    }
    __syncthreads();
    // 3. logits on MFMA: wave owns tokens [16*kBlocks*wave, +16*kBlocks);
    // a block wholly past the tile's tokens skips its MFMAs (a uniform
    // branch) and only writes -inf
#pragma unroll
    for (int blk = 0; blk < T::kBlocks; ++blk) {
      const int t0 = 16 * (T::kBlocks * wave + blk);
      const uint8_t* krow = k_s + (t0 + col) * T::kPitch;
      v4f s = {0.f, 0.f, 0.f, 0.f};
      if (t0 < tn) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
          s = mfma_qk<QBF>(qa[st], k8_as_q<ENC, QBF>(krow, 32 * grp + 8 * st), s);
      }
      const int t = t0 + col;
      const bool live = t < tn && slot_s[t] >= 0;
      const float f = zscale * ks_s[t];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        zp_s[(4 * grp + v) * T::kZPitch + t] = live ? s[v] * f : -__builtin_inff();
    }
    __syncthreads();
    // 4. online softmax per head (base 2): wave handles heads wave + W*i
#pragma unroll
    for (int i = 0; i < 16 / kWavesW; ++i) {
      const int hh = wave + kWavesW * i;
      if (hh < G) {
        float z[NT / 64];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < NT / 64; ++r) {
          z[r] = zp_s[hh * T::kZPitch + lane + 64 * r];
          tmax = fmaxf(tmax, z[r]);
        }
        tmax = wave_max(tmax);
        const float m_old = m_s[hh];
        const float m_new = fmaxf(m_old, tmax);
        float psum = 0.f, alpha = 1.f;
        if (m_new != -__builtin_inff()) {
          alpha = m_old == -__builtin_inff() ? 0.f : exp2f(m_old - m_new);
#pragma unroll
          for (int r = 0; r < NT / 64; ++r) {
            const float p = z[r] == -__builtin_inff() ? 0.f : exp2f(z[r] - m_new);
            psum += p;
            zp_s[hh * T::kZPitch + lane + 64 * r] = p * vs_s[lane + 64 * r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < NT / 64; ++r)
            zp_s[hh * T::kZPitch + lane + 64 * r] = 0.f;
        }
        psum = wave_sum(psum);
        if (lane == 0) {
          m_s[hh] = m_new;
          l_s[hh] = l_s[hh] * alpha + psum;
          alpha_s[hh] = alpha;
        }
      }
    }
    __syncthreads();
    // 5. O += P V on FP32 MFMA, 4 tokens per instruction
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * grp + v;
      const float a = hh < G ? alpha_s[hh] : 0.f;
#pragma unroll
      for (int j = 0; j < T::kJ; ++j) acc[j][v] *= a;
    }
    const bool arow = col < G;
    if constexpr (fp8) {
      // bf16 MFMA, 32 tokens per instruction: A = P x V-scale rounded once
      // to bf16 (heads x tokens), B = the FP8 V codes widened exactly
      // (tokens x dims); lane group grp supplies tokens 8*grp .. 8*grp+7
#pragma unroll
      for (int ks = 0; ks < NT / 32; ++ks) {
        if (32 * ks >= tn) break;  // uniform: only zero probabilities left
        const int t0 = 32 * ks + 8 * grp;
        v8bf pa;
        if (arow) {
          const float4 p0 = *reinterpret_cast<const float4*>(zp_s + col * T::kZPitch + t0);
          const float4 p1 = *reinterpret_cast<const float4*>(zp_s + col * T::kZPitch + t0 + 4);
          pa = v8bf{static_cast<__bf16>(p0.x), static_cast<__bf16>(p0.y),
                    static_cast<__bf16>(p0.z), static_cast<__bf16>(p0.w),
                    static_cast<__bf16>(p1.x), static_cast<__bf16>(p1.y),
                    static_cast<__bf16>(p1.z), static_cast<__bf16>(p1.w)};
        } else {
          pa = v8bf{};
        }
#pragma unroll
        for (int j = 0; j < T::kJ; ++j) {
          const uint8_t* vc = v_s + T::vrow(t0) + T::kDW * wave + 16 * j + col;
          uint32_t w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            w[h] = static_cast<uint32_t>(vc[(4 * h + 0) * T::kPitch]) |
                   static_cast<uint32_t>(vc[(4 * h + 1) * T::kPitch]) << 8 |
                   static_cast<uint32_t>(vc[(4 * h + 2) * T::kPitch]) << 16 |
                   static_cast<uint32_t>(vc[(4 * h + 3) * T::kPitch]) << 24;
          // the FP8 V codes widened exactly to bf16
          const uint4 bv = make_uint4(widen2<true, false>(w[0]), widen2<true, true>(w[0]),
                                      widen2<true, false>(w[1]), widen2<true, true>(w[1]));
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              pa, __builtin_bit_cast(v8bf, bv), acc[j], 0, 0, 0);
        }
      }
    } else {
      // MFMA of the cache's 16-bit type, 32 tokens per instruction: A = P
      // as the sum of two 16-bit parts (hi = P rounded, lo = the remainder
      // rounded; their sum is within 2^-17 of P relative for bf16, 2^-21
      // for fp16, plus 2^-25 absolute for fp16 subnormals), B = the V rows
      // as stored (tokens x dims); lane group grp supplies tokens
      // 8*grp .. 8*grp+7
#pragma unroll
      for (int ks = 0; ks < NT / 32; ++ks) {
        if (32 * ks >= tn) break;  // uniform: only zero probabilities left
        const int t0 = 32 * ks + 8 * grp;
        uint4 ph = make_uint4(0u, 0u, 0u, 0u), pl = make_uint4(0u, 0u, 0u, 0u);
        if (arow) {
          const float4 p0 = *reinterpret_cast<const float4*>(zp_s + col * T::kZPitch + t0);
          const float4 p1 = *reinterpret_cast<const float4*>(zp_s + col * T::kZPitch + t0 + 4);
          const float pf[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t h2[2], l2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float x = pf[2 * i + e];
              if constexpr (QBF) {
                const __bf16 hb = static_cast<__bf16>(x);
                const __bf16 lb = static_cast<__bf16>(x - static_cast<float>(hb));
                h2[e] = __builtin_bit_cast(uint16_t, hb);
                l2[e] = __builtin_bit_cast(uint16_t, lb);
              } else {
                const _Float16 hh = static_cast<_Float16>(x);
                const _Float16 lh = static_cast<_Float16>(x - static_cast<float>(hh));
                h2[e] = __builtin_bit_cast(uint16_t, hh);
                l2[e] = __builtin_bit_cast(uint16_t, lh);
              }
            }
            hw[i] = h2[0] | (h2[1] << 16);
            lw[i] = l2[0] | (l2[1] << 16);
          }
          ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        // B by LDS transpose loads: lane L of a 16-lane group points at row
        // t + L/4, columns d + 4*(L%4) .. +3, and receives column d + L of
        // rows t .. t+3; two loads give tokens t0 .. t0+7 of one dimension
        const int q = col;  // the lane's index in its group of 16
#pragma unroll
        for (int j = 0; j < T::kJ; ++j) {
          const uint8_t* vb = v_s + 2 * (T::kDW * wave + 16 * j + 4 * (q & 3));
          const v4s lo = lds_read_tr16(vb + T::vrow(t0 + (q >> 2)));
          const v4s hi = lds_read_tr16(vb + T::vrow(t0 + 4 + (q >> 2)));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          const uint4 bv = make_uint4(l2.x, l2.y, h2.x, h2.y);
          acc[j] = mfma_qk<QBF>(ph, bv, acc[j]);
          acc[j] = mfma_qk<QBF>(pl, bv, acc[j]);
        }
      }
    }
    __syncthreads();
  }

  // finalize: O / l and lse (natural log)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int hh = 4 * grp + v;
    if (hh < G) {
      const float l = l_s[hh];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* o = o_part + ((static_cast<int64_t>(b) * H_q + h0 + hh) * C + c) * kD;
#pragma unroll
      for (int j = 0; j < T::kJ; ++j) o[T::kDW * wave + 16 * j + col] = acc[j][v] * inv;
    }
  }
  if (tid < G) {
    const float l = l_s[tid];
    lse_part[(static_cast<int64_t>(b) * H_q + h0 + tid) * C + c] =
        l > 0.f ? (m_s[tid] + log2f(l)) * kLn2 : -__builtin_inff();
  }
}

template <int ENC, bool QBF>
hipError_t launch_enc(const tsd_attn_args& a, hipStream_t s) {
  dim3 grid(static_cast<uint32_t>(a.chunks), static_cast<uint32_t>(a.H_kv),
            static_cast<uint32_t>(a.B));
  const int lbs = a.idx_block > 1 ? __builtin_ctz(static_cast<unsigned>(a.idx_block)) : 0;
  hipLaunchKernelGGL((sparse_gqa_kernel<ENC, QBF>), grid, dim3(Tile<ENC>::kThreads), 0,
                     s, a.H_q, a.H_kv, a.H_sel, a.k, a.chunks, lbs, a.idx,
                     a.seq_lens, a.count, static_cast<const uint16_t*>(a.q),
                     a.pt_stride, a.page_table, a.num_pages,
                     static_cast<const uint8_t*>(a.k_pool),
                     static_cast<const uint8_t*>(a.v_pool), a.k_scale,
                     a.v_scale, a.softmax_scale, a.dense_len, a.o_part,
                     a.lse_part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_gqa(const tsd_attn_args& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const bool qbf = a.q_dtype == TSD_BF16;
  switch (a.kv_dtype) {
    case TSD_FP8_E4M3:
      return qbf ? launch_enc<TSD_FP8_E4M3, true>(a, s)
                 : launch_enc<TSD_FP8_E4M3, false>(a, s);
    case TSD_BF16: return launch_enc<TSD_BF16, true>(a, s);
    default: return launch_enc<TSD_FP16, false>(a, s);
  }
}

}  // namespace tsd
