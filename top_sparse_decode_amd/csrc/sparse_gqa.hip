// Sparse GQA decode attention over the selected tokens, split into chunks
// with FP32 partial outputs and log-sum-exps ("QSA cache sharding", sglang
// PR #43527, Distributed QSA execution: sparse attention over the selected
// tokens, partial outputs merged by FP32 log-sum-exp; "Context parallelism
// for QSA attention and the sparse indexer": a sparse GQA call per block).
//
// One workgroup per (request b, KV head g, chunk c) handles the G query
// heads of the group over the chunk's run of the ascending selection list,
// 64 tokens at a time:
//   1. the tile's slots are resolved from the page table (an index outside
//      [0, len) or a page outside [0, num_pages) is masked, never read);
//   2. the 64 K rows and V rows are gathered into LDS with 16-byte loads
//      (a token's row is contiguous in the token-major pool);
//   3. lane j of each wave forms z = scale * q_h . Khat_j for its heads;
//   4. an online softmax (base-2 internally) updates the running max and
//      sum per head, the V page scale is folded into the probabilities;
//   5. each thread accumulates one output dimension of up to 8 heads.
// FP8 K/V are decoded by the hardware converter and scaled by their page's
// f32 scale; BF16/FP16 are widened exactly. All arithmetic is FP32.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kD = 128;
constexpr int kTile = 64;
constexpr int kMaxG = 16;
constexpr int kMaxRowBytes = kD * 2;
constexpr int kRowPitch = kMaxRowBytes + 16;  // LDS pitch, breaks bank aliasing
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int ENC>
struct Enc {
  static constexpr int kBytes = ENC == TSD_FP8_E4M3 ? 1 : 2;
  static constexpr int kPer16 = 16 / kBytes;  // elements per 16 bytes
};

// 16 bytes of a K or V row -> Enc<ENC>::kPer16 floats.
template <int ENC>
TSD_DEVICE void decode16(const uint4 x, float* out) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (ENC == TSD_FP8_E4M3) {
#pragma unroll
    for (int e = 0; e < 4; ++e) fp8x4_to_f32(w[e], out + 4 * e);
  } else {
    constexpr bool bf = ENC == TSD_BF16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = half_to_f32(static_cast<uint16_t>(w[e] & 0xFFFF), bf);
      out[2 * e + 1] = half_to_f32(static_cast<uint16_t>(w[e] >> 16), bf);
    }
  }
}

template <int ENC>
TSD_DEVICE float elem(const uint8_t* row, int d) {
  if constexpr (ENC == TSD_FP8_E4M3) {
    const uint32_t b = row[d];
    return fp8x2_to_f32<false>(b).x;
  } else {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[d];
    return half_to_f32(h, ENC == TSD_BF16);
  }
}

template <int ENC>
__global__ __launch_bounds__(kThreads) void sparse_gqa_kernel(
    const uint16_t* __restrict__ q, int q_enc, int H_q, int H_kv,
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool,
    const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const int32_t* __restrict__ seq_lens,
    int64_t num_pages, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ count, int H_sel, int k, int C,
    float softmax_scale, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  __shared__ float q_s[kMaxG][kD];
  __shared__ __align__(16) uint8_t k_s[kTile * kRowPitch];
  __shared__ __align__(16) uint8_t v_s[kTile * kRowPitch];
  __shared__ float p_s[kMaxG][kTile];
  __shared__ int64_t slot_s[kTile];
  __shared__ float ks_s[kTile], vs_s[kTile];
  __shared__ float m_s[kMaxG], l_s[kMaxG], alpha_s[kMaxG];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = H_q / H_kv;
  const int h0 = g * G;
  const int srow = H_sel == 1 ? 0 : g;
  int64_t m = count[static_cast<int64_t>(b) * H_sel + srow];
  m = clamp_len(m, k);
  const int64_t lo = c * m / C, hi = (c + 1) * m / C;
  const int64_t n = clamp_len(seq_lens[b], pt_stride * kPage);
  const int32_t* sel = idx + (static_cast<int64_t>(b) * H_sel + srow) * k;
  const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride;
  constexpr bool fp8 = ENC == TSD_FP8_E4M3;
  constexpr int esz = Enc<ENC>::kBytes;
  constexpr int row_bytes = kD * esz;
  const float zscale = softmax_scale * kLog2e;

  for (int i = tid; i < G * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    q_s[hh][d] = half_to_f32(q[(static_cast<int64_t>(b) * H_q + h0 + hh) * kD + d],
                             q_enc == TSD_BF16);
  }
  if (tid < G) {
    m_s[tid] = -__builtin_inff();
    l_s[tid] = 0.f;
  }
  // output ownership: dimension d of heads hs, hs + 2, ...
  const int od = tid % kD, hs = tid / kD;
  float acc[kMaxG / 2];
#pragma unroll
  for (int i = 0; i < kMaxG / 2; ++i) acc[i] = 0.f;
  __syncthreads();

  for (int64_t base = lo; base < hi; base += kTile) {
    const int tn = static_cast<int>(hi - base < kTile ? hi - base : kTile);
    // 1. resolve slots
    if (tid < kTile) {
      int64_t slot = -1;
      float ks = 0.f, vs = 0.f;
      if (tid < tn) {
        const int64_t t = sel[base + tid];
        if (t >= 0 && t < n) {
          const int32_t page = pt[t / kPage];
          if (page >= 0 && page < num_pages) {
            slot = static_cast<int64_t>(page) * kPage + t % kPage;
            ks = fp8 ? k_scale[page] : 1.f;
            vs = fp8 ? v_scale[page] : 1.f;
          }
        }
      }
      slot_s[tid] = slot;
      ks_s[tid] = ks;
      vs_s[tid] = vs;
    }
    __syncthreads();
    // 2. gather K and V rows
    constexpr int vec_per_row = row_bytes / 16;
    for (int i = tid; i < kTile * vec_per_row; i += kThreads) {
      const int j = i / vec_per_row, v = i % vec_per_row;
      const int64_t slot = slot_s[j];
      if (slot >= 0) {
        const int64_t off = (slot * H_kv + g) * row_bytes + 16 * v;
        *reinterpret_cast<uint4*>(k_s + j * kRowPitch + 16 * v) =
            *reinterpret_cast<const uint4*>(k_pool + off);
        *reinterpret_cast<uint4*>(v_s + j * kRowPitch + 16 * v) =
            *reinterpret_cast<const uint4*>(v_pool + off);
      }
    }
    __syncthreads();
    // 3. logits: lane j, heads wave, wave + 4, ...
    {
      float z[kMaxG / 4];
#pragma unroll
      for (int i = 0; i < kMaxG / 4; ++i) z[i] = 0.f;
      const bool live = lane < tn && slot_s[lane] >= 0;
      if (live) {
        const uint8_t* kr = k_s + lane * kRowPitch;
#pragma unroll 2
        for (int off = 0; off < row_bytes; off += 16) {
          constexpr int cnt = Enc<ENC>::kPer16;
          float kv[cnt];
          decode16<ENC>(*reinterpret_cast<const uint4*>(kr + off), kv);
          const int d0 = off / esz;
#pragma unroll
          for (int i = 0; i < kMaxG / 4; ++i) {
            const int hh = wave + 4 * i;
            if (hh < G) {
              float s = 0.f;
#pragma unroll
              for (int e = 0; e < cnt; ++e) s += q_s[hh][d0 + e] * kv[e];
              z[i] += s;
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kMaxG / 4; ++i) {
        const int hh = wave + 4 * i;
        if (hh < G)
          p_s[hh][lane] = live ? z[i] * ks_s[lane] * zscale : -__builtin_inff();
      }
    }
    __syncthreads();
    // 4. online softmax per head (base 2)
#pragma unroll
    for (int i = 0; i < kMaxG / 4; ++i) {
      const int hh = wave + 4 * i;
      if (hh < G) {
        const float z = p_s[hh][lane];
        const float tmax = wave_max(z);
        const float m_old = m_s[hh];
        const float m_new = fmaxf(m_old, tmax);
        float p = 0.f, alpha = 1.f;
        if (m_new != -__builtin_inff()) {
          p = z == -__builtin_inff() ? 0.f : exp2f(z - m_new);
          alpha = m_old == -__builtin_inff() ? 0.f : exp2f(m_old - m_new);
        }
        const float psum = wave_sum(p);
        p_s[hh][lane] = p * vs_s[lane];
        if (lane == 0) {
          m_s[hh] = m_new;
          l_s[hh] = l_s[hh] * alpha + psum;
          alpha_s[hh] = alpha;
        }
      }
    }
    __syncthreads();
    // 5. weighted values
    {
#pragma unroll
      for (int i = 0; i < kMaxG / 2; ++i) {
        const int hh = hs + 2 * i;
        if (hh < G) acc[i] *= alpha_s[hh];
      }
      for (int j = 0; j < tn; ++j) {
        if (slot_s[j] < 0) continue;
        const float v = elem<ENC>(v_s + j * kRowPitch, od);
#pragma unroll
        for (int i = 0; i < kMaxG / 2; ++i) {
          const int hh = hs + 2 * i;
          if (hh < G) acc[i] += p_s[hh][j] * v;
        }
      }
    }
    __syncthreads();
  }

  // finalize
#pragma unroll
  for (int i = 0; i < kMaxG / 2; ++i) {
    const int hh = hs + 2 * i;
    if (hh < G) {
      const float l = l_s[hh];
      const float o = l > 0.f ? acc[i] / l : 0.f;
      o_part[((static_cast<int64_t>(b) * H_q + h0 + hh) * C + c) * kD + od] = o;
    }
  }
  if (tid < G) {
    const float l = l_s[tid];
    lse_part[(static_cast<int64_t>(b) * H_q + h0 + tid) * C + c] =
        l > 0.f ? (m_s[tid] + log2f(l)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_sparse_gqa(const tsd_attn_args& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(a.chunks), static_cast<uint32_t>(a.H_kv),
            static_cast<uint32_t>(a.B));
  auto kern = a.kv_dtype == TSD_FP8_E4M3 ? sparse_gqa_kernel<TSD_FP8_E4M3>
              : a.kv_dtype == TSD_BF16   ? sparse_gqa_kernel<TSD_BF16>
                                         : sparse_gqa_kernel<TSD_FP16>;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(a.q), a.q_dtype, a.H_q,
                     a.H_kv, static_cast<const uint8_t*>(a.k_pool),
                     static_cast<const uint8_t*>(a.v_pool), a.k_scale,
                     a.v_scale, a.page_table, a.pt_stride, a.seq_lens,
                     a.num_pages, a.idx, a.count, a.H_sel, a.k, a.chunks,
                     a.softmax_scale, a.o_part, a.lse_part);
  return hipGetLastError();
}

}  // namespace tsd
