// Cache append: the rows of newly appended tokens into the paged pools
// ("Support double sparsity", forward_extend: the label cache is K gathered
// at the heavy channels and is written with every new token; "Context
// parallelism for QSA attention and the sparse indexer", Motivation: the
// indexer stores raw index-K for every token).
//
// One workgroup per (request, logical page touched by the request's new
// tokens). A workgroup whose page is started by this call (no token of the
// page precedes the first new position) reduces the amax of the K and V
// values it writes and stores the page scales amax / 448; every workgroup
// then encodes with its page's scale. The FP8 codes come from the gfx950
// converter (round to nearest even) after clamping to +-448, which is the
// saturating encode.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kAT = 256;
constexpr float kFp8Max = 448.f;
constexpr float kAppendHeadroom = 4.f;

TSD_DEVICE float clamp448(float x) { return fminf(fmaxf(x, -kFp8Max), kFp8Max); }

// Four f32 values -> four E4M3 codes in one dword (byte i = value i).
TSD_DEVICE uint32_t fp8x4_encode(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return static_cast<uint32_t>(w);
}

// Four consecutive 16-bit values as f32.
TSD_DEVICE void half4_to_f32(uint2 raw, bool bf, float* f) {
  f[0] = half_to_f32(static_cast<uint16_t>(raw.x & 0xffffu), bf);
  f[1] = half_to_f32(static_cast<uint16_t>(raw.x >> 16), bf);
  f[2] = half_to_f32(static_cast<uint16_t>(raw.y & 0xffffu), bf);
  f[3] = half_to_f32(static_cast<uint16_t>(raw.y >> 16), bf);
}

// Workgroup max of one non-negative value per thread, broadcast.
TSD_DEVICE float block_max(float x, float* lds) {
  x = wave_max(x);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kAT / kWave; ++i) m = fmaxf(m, lds[i]);
  __syncthreads();
  return m;
}

__global__ __launch_bounds__(kAT) void kv_append_kernel(tsd_append_args a) {
  __shared__ float lds[kAT / kWave];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t pos = a.positions[b];
  int64_t n = a.n_new[b];
  n = n < 0 ? 0 : (n > a.max_new ? a.max_new : n);
  const int64_t tlo = pos < 0 ? 0 : pos;
  const int64_t cap = a.pt_stride * kPage;
  const int64_t thi = pos + n < cap ? pos + n : cap;
  if (tlo >= thi) return;  // uniform over the workgroup
  const int64_t lp = tlo / kPage + blockIdx.x;
  const int64_t t0 = lp * kPage > tlo ? lp * kPage : tlo;
  const int64_t t1 = lp * kPage + kPage < thi ? lp * kPage + kPage : thi;
  if (t0 >= t1) return;
  const int32_t page = a.page_table[static_cast<int64_t>(b) * a.pt_stride + lp];
  if (page < 0 || page >= a.num_pages) return;
  const int nt = static_cast<int>(t1 - t0);            // tokens on this page
  const int64_t slot0 = static_cast<int64_t>(page) * kPage + (t0 - lp * kPage);
  const int64_t src0 = static_cast<int64_t>(b) * a.max_new + (t0 - pos);
  const bool bf = a.new_dtype == TSD_BF16;
  const int row = a.H_kv * a.D;                        // elements per token

  if (a.k_new) {
    const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + src0 * row;
    const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + src0 * row;
    const int nvec = nt * row / 4;                     // 4 elements per step
    if (a.kv_dtype == TSD_FP8_E4M3) {
      float sk, sv;
      if (lp * kPage >= pos) {  // started by this call: scale from its values
        float ka = 0.f, va = 0.f;
        for (int i = tid; i < nvec; i += kAT) {
          float f[4], g[4];
          half4_to_f32(reinterpret_cast<const uint2*>(kn)[i], bf, f);
          half4_to_f32(reinterpret_cast<const uint2*>(vn)[i], bf, g);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ka = fmaxf(ka, fabsf(f[j]));
            va = fmaxf(va, fabsf(g[j]));
          }
        }
        ka = block_max(ka, lds);
        va = block_max(va, lds);
        // a page this call does not fill keeps two binades of headroom for
        // the tokens later calls append (a power of two: exact, and FP8
        // precision is relative, so only values below 2^-6 of the range
        // lose bits)
        const float room = nt == kPage ? 1.f : kAppendHeadroom;
        sk = ka > 0.f ? ka / kFp8Max * room : 1.f;
        sv = va > 0.f ? va / kFp8Max * room : 1.f;
        if (tid == 0) {
          a.k_scale[page] = sk;
          a.v_scale[page] = sv;
        }
      } else {
        sk = a.k_scale[page];
        sv = a.v_scale[page];
      }
      uint32_t* kp = reinterpret_cast<uint32_t*>(
          static_cast<uint8_t*>(a.k_pool) + slot0 * row);
      uint32_t* vp = reinterpret_cast<uint32_t*>(
          static_cast<uint8_t*>(a.v_pool) + slot0 * row);
      for (int i = tid; i < nvec; i += kAT) {
        float f[4], g[4];
        half4_to_f32(reinterpret_cast<const uint2*>(kn)[i], bf, f);
        half4_to_f32(reinterpret_cast<const uint2*>(vn)[i], bf, g);
        kp[i] = fp8x4_encode(f[0] / sk, f[1] / sk, f[2] / sk, f[3] / sk);
        vp[i] = fp8x4_encode(g[0] / sv, g[1] / sv, g[2] / sv, g[3] / sv);
      }
    } else {  // 16-bit pool in the new rows' encoding: a copy
      uint2* kp = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.k_pool) + slot0 * row);
      uint2* vp = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.v_pool) + slot0 * row);
      for (int i = tid; i < nvec; i += kAT) {
        kp[i] = reinterpret_cast<const uint2*>(kn)[i];
        vp[i] = reinterpret_cast<const uint2*>(vn)[i];
      }
    }
  }

  if (a.channel_idx) {  // label: K at each KV head's heavy channels
    const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + src0 * row;
    uint16_t* lp_ = static_cast<uint16_t*>(a.label_pool) + slot0 * a.H_kv * a.r;
    const int per_tok = a.H_kv * a.r;
    for (int i = tid; i < nt * per_tok; i += kAT) {
      const int tok = i / per_tok, gj = i - tok * per_tok;
      const int g = gj / a.r;
      const int32_t ch = a.channel_idx[gj];  // outside [0, D): stores 0
      lp_[i] = ch >= 0 && ch < a.D ? kn[static_cast<int64_t>(tok) * row + g * a.D + ch]
                                   : static_cast<uint16_t>(0);
    }
  }

  if (a.index_k_new) {  // FP8 index-K, unit scale
    uint32_t* ip = reinterpret_cast<uint32_t*>(
        static_cast<uint8_t*>(a.index_k_pool) + slot0 * a.D_i);
    const int nvec = nt * a.D_i / 4;
    const int64_t isrc = src0 * a.D_i / 4;
    for (int i = tid; i < nvec; i += kAT) {
      float f[4];
      if (a.index_dtype == TSD_F32) {
        const float4 x = reinterpret_cast<const float4*>(a.index_k_new)[isrc + i];
        f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
      } else {
        half4_to_f32(reinterpret_cast<const uint2*>(a.index_k_new)[isrc + i],
                     a.index_dtype == TSD_BF16, f);
      }
      ip[i] = fp8x4_encode(f[0], f[1], f[2], f[3]);
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const tsd_append_args& a, hipStream_t s) {
  if (a.B == 0 || a.max_new == 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((a.max_new + kPage - 1) / kPage + 1),
            static_cast<uint32_t>(a.B));
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(kAT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tsd
