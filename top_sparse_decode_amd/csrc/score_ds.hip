// Double-sparsity label scan ("Support double sparsity", sglang PR #1459:
// the label cache holds K at r heavy channels per head; decode scores every
// cached token with it and keeps the heavy tokens):
//   s[b*H_kv+g][t] = sum_j qs[g][j] * label[slot(b,t)][g][j],
//   qs[g][j]       = sum of the group's query heads at channel chan[g][j].
//
// About 1 flop per byte, so this is a plain bandwidth-bound VALU pass. The
// labels of a page ([64][H_kv][r] 16-bit values) are one contiguous block.
//
// ds_scan_vec_kernel (r a multiple of 8, 16-byte aligned pool): one
// workgroup owns a run of pages of one request. It computes qs once, keeps
// the run's page ids in LDS, and streams the pages as 32 KB sub-blocks (8
// 16-byte loads per thread), the next sub-block's loads in flight while the
// current one is summed; the loads are unconditional (a page outside the
// pool reads page 0 and scores -inf), so the compiler can count them, and
// non-temporal (every label is read once). Where the launch would give one
// page per workgroup anyway and the page splits into whole-token sub-blocks,
// each workgroup takes one sub-block and keeps a single register buffer,
// which raises the workgroups per CU from 5 to 8. A
// label spans VPI = r/8 consecutive vectors, held by VPI consecutive lanes
// whose partial dots are added by lane exchanges; when every lane always
// meets the same head and channels (256/VPI a multiple of H_kv) its slice of
// qs sits in registers. A page's scores are staged in LDS and stored as 64
// contiguous floats per (request, head) row.
//
// In the one-sub-block form, where each thread forms at most EC channels of the
// group query from at most EG query heads (EC, EG = 1, 4 or 2, 1), the row
// length, the thread's channel ids and the unit's page id are loaded
// together; then the thread's query values at those channels, then the
// unit's labels, all unconditional (clamped indices, masked at use). Loads
// complete in order, so forming the group query waits for the query values
// only and the labels are already in flight: the labels leave after one
// dependent round trip instead of three (length, channels, query).
//
// The vector kernel's arguments that its first loads need come first, in
// the 14 kernel-argument dwords the hardware preloads into scalar registers.
//
// ds_scan_kernel: the general form, one workgroup per page.
#include "device_common.h"
#include "launch.h"

namespace tsd {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxHeadChan = 4096;  // H_kv * r held in LDS
// Scores staged in LDS as [head][token] rows of kScPitch floats: the
// lanes of one wave store one token's scores of many heads, which a
// 64-float pitch would put in one bank (a many-way conflict); 65 spreads
// them over distinct banks.
constexpr int kScPitch = kPage + 1;
constexpr int kMaxScoreLds = kScPitch * 128;
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <bool B>
struct Bool {
  static constexpr bool value = B;
};

// Sum over aligned groups of N lanes (N a power of two, at most 16) by DPP
// moves: quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row
// mirrors (after the quad steps the 4 lanes of a quad hold equal values, so
// a mirror pairs every lane with an equal partner in the other half). Each
// lane adds its partner's value to its own, as a lane exchange would.
template <int CTRL>
TSD_DEVICE float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int N>
TSD_DEVICE float group_sum(float v) {
  static_assert(N >= 1 && N <= 16 && (N & (N - 1)) == 0, "group size");
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);
  if constexpr (N >= 16) v += dpp_mov<0x140>(v);
  return v;
}

__global__ __launch_bounds__(kThreads) void ds_scan_kernel(
    const uint16_t* __restrict__ q, bool is_bf16, int H_q, int H_kv, int D,
    const int32_t* __restrict__ chan, int r,
    const uint16_t* __restrict__ label, const int32_t* __restrict__ page_table,
    int64_t pt_stride, const int32_t* __restrict__ seq_lens,
    int64_t num_pages, float* __restrict__ scores, int64_t score_stride,
    int32_t* __restrict__ row_lens_out) {
  __shared__ float qs[kMaxHeadChan];
  __shared__ float sc[kMaxScoreLds];
  const int b = blockIdx.y;
  const int64_t p = blockIdx.x;
  int64_t n = clamp_len(seq_lens[b], pt_stride * kPage);
  n = clamp_len(n, score_stride);
  if (p == 0 && row_lens_out)
    for (int g = threadIdx.x; g < H_kv; g += kThreads)
      row_lens_out[static_cast<int64_t>(b) * H_kv + g] = static_cast<int32_t>(n);
  if (p * kPage >= n) return;
  const int32_t page = page_table[static_cast<int64_t>(b) * pt_stride + p];
  const bool valid = page >= 0 && page < num_pages;
  const int G = H_q / H_kv;
  const int hc = H_kv * r;

  // group query at the heavy channels
  for (int i = threadIdx.x; i < hc; i += kThreads) {
    const int g = i / r;
    const int c = chan[i];
    float acc = 0.f;
    if (c >= 0 && c < D) {
      const uint16_t* qb = q + (static_cast<int64_t>(b) * H_q + g * G) * D + c;
      for (int h = 0; h < G; ++h) acc += half_to_f32(qb[h * D], is_bf16);
    }
    qs[i] = acc;
  }
  __syncthreads();

  const int items = kPage * H_kv;  // (slot s, head g), g fastest
  if (valid) {
    const uint16_t* base = label + static_cast<int64_t>(page) * kPage * hc;
    if ((r & 7) == 0 && (reinterpret_cast<uintptr_t>(label) & 15u) == 0) {
      const int vecs = r >> 3;  // 16-byte vectors per label
      for (int it = threadIdx.x; it < items; it += kThreads) {
        const int g = it % H_kv;
        const uint4* src = reinterpret_cast<const uint4*>(base) +
                           static_cast<int64_t>(it) * vecs;
        const float* qg = qs + g * r;
        float acc = 0.f;
        for (int v = 0; v < vecs; ++v) {
          const uint4 x = src[v];
          const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc += qg[8 * v + 2 * e] *
                   half_to_f32(static_cast<uint16_t>(wds[e] & 0xFFFF), is_bf16);
            acc += qg[8 * v + 2 * e + 1] *
                   half_to_f32(static_cast<uint16_t>(wds[e] >> 16), is_bf16);
          }
        }
        sc[g * kScPitch + it / H_kv] = acc;
      }
    } else {
      for (int it = threadIdx.x; it < items; it += kThreads) {
        const int g = it % H_kv;
        const uint16_t* src = base + static_cast<int64_t>(it) * r;
        const float* qg = qs + g * r;
        float acc = 0.f;
        for (int j = 0; j < r; ++j) acc += qg[j] * half_to_f32(src[j], is_bf16);
        sc[g * kScPitch + it / H_kv] = acc;
      }
    }
  }
  __syncthreads();
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int g = it / kPage, s = it % kPage;
    const int64_t t = p * kPage + s;
    if (t < n)
      scores[(static_cast<int64_t>(b) * H_kv + g) * score_stride + t] =
          valid ? sc[g * kScPitch + s] : -__builtin_inff();
  }
}

constexpr int kSubVec = kThreads * 8;  // 16-byte vectors per sub-block

// ONE: every workgroup streams a single unit, sub-block blockIdx.x % SB of
// page blockIdx.x / SB (SB a power of two, so a unit holds 64 / SB whole
// tokens), with no second register buffer, so more workgroups fit a CU.
template <int VPI, bool QREG, bool ONE, int EC, int EG>
__global__ __launch_bounds__(kThreads) void ds_scan_vec_kernel(
    int H_kv, int r, int H_q, int D, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ chan, const int32_t* __restrict__ page_table,
    int64_t pt_stride, int P, bool is_bf16, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ label, int64_t num_pages,
    float* __restrict__ scores, int64_t score_stride,
    int32_t* __restrict__ row_lens_out) {
  extern __shared__ __align__(16) float dyn_s[];
  const int hc = H_kv * r;
  float* qs = dyn_s;                              // [hc]
  float* sc = dyn_s + hc;                         // [2][H_kv][kScPitch]
  int32_t* pages_s = reinterpret_cast<int32_t*>(sc + 2 * kScPitch * H_kv);  // [P]
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int VP = 8 * hc;                          // vectors per page
  const int SB = (VP + kSubVec - 1) / kSubVec;    // sub-blocks per page
  const int64_t pp0 = ONE ? blockIdx.x / SB : static_cast<int64_t>(blockIdx.x) * P;
  const int sub0 = ONE ? static_cast<int>(blockIdx.x % SB) : 0;
  const int tpu = kPage / SB;                     // ONE: tokens of the unit
  constexpr bool EARLY = ONE && EC > 0;  // see the one-unit form above
  uint4 xe[8];  // EARLY: the unit's labels, loaded in the prologue
  int64_t n;
  int npg = 1;
  const int G = H_q / H_kv;
  if constexpr (EARLY) {
    const int32_t len_raw = seq_lens[b];
    int32_t ch[EC];
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int i = tid + j * kThreads;
      ch[j] = chan[i < hc ? i : hc - 1];
    }
    const int32_t pe = page_table[static_cast<int64_t>(b) * pt_stride + pp0];
    n = clamp_len(len_raw, pt_stride * kPage);
    n = clamp_len(n, score_stride);
    if (blockIdx.x == 0 && row_lens_out)
      for (int g = tid; g < H_kv; g += kThreads)
        row_lens_out[static_cast<int64_t>(b) * H_kv + g] = static_cast<int32_t>(n);
    if (pp0 * kPage + sub0 * tpu >= n) return;  // uniform
    uint16_t qraw[EC][EG];
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int i0 = tid + j * kThreads;
      const int i = i0 < hc ? i0 : hc - 1;
      const int g = i / r;
      const int c = ch[j] >= 0 && ch[j] < D ? ch[j] : 0;
#pragma unroll
      for (int h = 0; h < EG; ++h)
        qraw[j][h] = q[(static_cast<int64_t>(b) * H_q + g * G + (h < G ? h : 0)) * D + c];
    }
    __builtin_amdgcn_sched_barrier(0);  // the labels are issued after the query
    const bool pv = pe >= 0 && pe < num_pages;
    const uint4* be = reinterpret_cast<const uint4*>(label) +
                      static_cast<int64_t>(pv ? pe : 0) * VP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int vv = sub0 * kSubVec + i * kThreads + tid;
      vv = vv < VP ? vv : VP - 1;
      const v4u tt = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(be + vv));
      xe[i] = make_uint4(tt.x, tt.y, tt.z, tt.w);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int i = tid + j * kThreads;
      if (i < hc) {
        float acc = 0.f;
        if (ch[j] >= 0 && ch[j] < D)
          for (int h = 0; h < G; ++h) acc += half_to_f32(qraw[j][h], is_bf16);
        qs[i] = acc;
      }
    }
    if (tid == 0) pages_s[0] = pv ? pe : -1;
    __syncthreads();
  } else {
  n = clamp_len(seq_lens[b], pt_stride * kPage);
  n = clamp_len(n, score_stride);
  if (blockIdx.x == 0 && row_lens_out)
    for (int g = tid; g < H_kv; g += kThreads)
      row_lens_out[static_cast<int64_t>(b) * H_kv + g] = static_cast<int32_t>(n);
  if (pp0 * kPage + sub0 * tpu >= n) return;  // uniform
  const int64_t left = (n - pp0 * kPage + kPage - 1) / kPage;
  npg = ONE ? 1 : (left < P ? static_cast<int>(left) : P);
  for (int i = tid; i < hc; i += kThreads) {  // group query at the channels
    const int g = i / r;
    const int c = chan[i];
    float acc = 0.f;
    if (c >= 0 && c < D) {
      const uint16_t* qb = q + (static_cast<int64_t>(b) * H_q + g * G) * D + c;
      for (int h = 0; h < G; ++h) acc += half_to_f32(qb[h * D], is_bf16);
    }
    qs[i] = acc;
  }
  for (int i = tid; i < npg; i += kThreads) {
    const int32_t page = page_table[static_cast<int64_t>(b) * pt_stride + pp0 + i];
    pages_s[i] = page >= 0 && page < num_pages ? page : -1;
  }
  __syncthreads();

  }
  const int units = ONE ? 1 : npg * SB;
  const int part = tid % VPI;                     // this lane's label vector
  float qr[8];  // QREG: this lane's slice of qs (head (tid / VPI) % H_kv)
  auto load_unit = [&](int u, uint4 (&x)[8]) {
    const int pg = ONE ? 0 : u / SB, sub = ONE ? sub0 : u - pg * SB;
    int32_t page = pages_s[pg];
    page = page < 0 ? 0 : page;                   // invalid: page 0, masked
    const uint4* base = reinterpret_cast<const uint4*>(label) +
                        static_cast<int64_t>(page) * VP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int vv = sub * kSubVec + i * kThreads + tid;
      vv = vv < VP ? vv : VP - 1;
      const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(base + vv));
      x[i] = make_uint4(t.x, t.y, t.z, t.w);
    }
  };
  // A vector's (token, head) item is vv / VPI, head fastest; a lane's
  // successive vectors lie kThreads / VPI items apart, so its head and token
  // follow from its first item by a uniform step and a carry (no division
  // per vector). The 16-bit type is fixed per call (BF), not per element.
  constexpr int kIpv = kThreads / VPI;
  const int dg = kIpv % H_kv, dt = kIpv / H_kv;
  auto sum_unit = [&](auto bf, int u, const uint4 (&x)[8]) {
    constexpr bool BF = decltype(bf)::value;
    const int pg = ONE ? 0 : u / SB, sub = ONE ? sub0 : u - pg * SB;
    const bool ok = pages_s[pg] >= 0;
    float* scp = sc + (pg & 1) * kScPitch * H_kv;
    const int it0 = (sub * kSubVec + tid) / VPI;
    int g = it0 % H_kv, tok = it0 / H_kv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int vv = sub * kSubVec + i * kThreads + tid;
      float w[8];
      const uint32_t wd[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF) {
          w[2 * e] = __uint_as_float(wd[e] << 16);
          w[2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
        } else {
          w[2 * e] = fp16_to_f32(static_cast<uint16_t>(wd[e] & 0xFFFF));
          w[2 * e + 1] = fp16_to_f32(static_cast<uint16_t>(wd[e] >> 16));
        }
      }
      float acc = 0.f;
      if constexpr (QREG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += qr[e] * w[e];
      } else {
        const float* qg = qs + g * r + part * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += qg[e] * w[e];
      }
      acc = group_sum<VPI>(acc);
      if (part == 0 && vv < VP)
        scp[g * kScPitch + tok] = ok ? acc : -__builtin_inff();
      g += dg;
      tok += dt;
      if (g >= H_kv) {
        g -= H_kv;
        ++tok;
      }
    }
  };
  auto sum_any = [&](int u, const uint4 (&x)[8]) {
    if (is_bf16)
      sum_unit(Bool<true>{}, u, x);
    else
      sum_unit(Bool<false>{}, u, x);
  };
  uint4 xa[8];
  if constexpr (EARLY) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = xe[i];
  } else {
    load_unit(0, xa);
  }
  if constexpr (QREG) {  // this lane always meets head (tid / VPI) % H_kv
    const int g = (tid / VPI) % H_kv;
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[e] = qs[g * r + part * 8 + e];
  }
  if constexpr (ONE) {
    sum_any(0, xa);
    __syncthreads();
    for (int it = tid; it < tpu * H_kv; it += kThreads) {
      const int g = it / tpu, sl = sub0 * tpu + it % tpu;
      const int64_t t = pp0 * kPage + sl;
      if (t < n) scores[(static_cast<int64_t>(b) * H_kv + g) * score_stride + t] = sc[g * kScPitch + sl];
    }
    return;
  } else {
  uint4 xb[8];
  for (int u = 0; u < units; u += 2) {
    if (u + 1 < units) load_unit(u + 1, xb);
    sum_any(u, xa);
    if (u + 2 < units) load_unit(u + 2, xa);
    if (u + 1 < units) sum_any(u + 1, xb);
    // a page is complete after its last sub-block: store its scores
    for (int d = 0; d < 2; ++d) {
      const int uu = u + d;
      if (uu >= units || (uu + 1) % SB != 0) continue;  // uniform
      __syncthreads();
      const int pg = uu / SB;
      const float* scp = sc + (pg & 1) * kScPitch * H_kv;
      for (int it = tid; it < kPage * H_kv; it += kThreads) {
        const int g = it / kPage, sl = it % kPage;
        const int64_t t = (pp0 + pg) * kPage + sl;
        if (t < n) scores[(static_cast<int64_t>(b) * H_kv + g) * score_stride + t] = scp[g * kScPitch + sl];
      }
      __syncthreads();  // the buffer is written again two pages later
    }
  }
  }
}

template <int VPI, bool QREG, bool ONE>
void launch_vec3(const tsd_score_args& a, dim3 grid, size_t lds, int P, hipStream_t s) {
  // the early-label prologue where a thread's share of the group query is
  // at most 1 channel x 4 heads or 2 channels x 1 head
  const int hc = a.H_kv * a.r, G = a.H_q / a.H_kv;
  auto kern = ds_scan_vec_kernel<VPI, QREG, ONE, 0, 0>;
  if (ONE && hc <= 256 && G <= 4) kern = ds_scan_vec_kernel<VPI, QREG, ONE, 1, 4>;
  else if (ONE && hc <= 512 && G <= 1) kern = ds_scan_vec_kernel<VPI, QREG, ONE, 2, 1>;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a.H_kv, a.r, a.H_q,
                     a.D, a.seq_lens, a.channel_idx, a.page_table, a.pt_stride, P,
                     a.q_dtype == TSD_BF16, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.label_pool), a.num_pages,
                     a.scores, a.score_stride, a.row_lens_out);
}

// Runs of P pages per workgroup, P for about 1,536 workgroups or more; where
// that is one page per workgroup and the page's sub-blocks split its tokens
// evenly, one sub-block per workgroup instead.
template <int VPI>
bool launch_vec(const tsd_score_args& a, hipStream_t s) {
  const int hc = a.H_kv * a.r;
  const int64_t total_pages = a.pt_stride * a.B;
  int P = static_cast<int>(total_pages / 1536);
  P = P < 1 ? 1 : (P > 64 ? 64 : P);
  const int SB = (8 * hc + kSubVec - 1) / kSubVec;
  // a unit then holds 64 / SB whole tokens: the page is one sub-block, or a
  // power-of-two number of full ones
  const bool one = P == 1 && (SB == 1 || ((8 * hc) % kSubVec == 0 &&
                                          (SB & (SB - 1)) == 0 && SB <= kPage));
  const size_t lds = static_cast<size_t>(hc + 2 * kScPitch * a.H_kv + P) * 4;
  dim3 grid(static_cast<uint32_t>(one ? a.pt_stride * SB : (a.pt_stride + P - 1) / P),
            static_cast<uint32_t>(a.B));
  const bool qreg = (kThreads / VPI) % a.H_kv == 0;
  if (qreg && one) launch_vec3<VPI, true, true>(a, grid, lds, P, s);
  else if (qreg) launch_vec3<VPI, true, false>(a, grid, lds, P, s);
  else if (one) launch_vec3<VPI, false, true>(a, grid, lds, P, s);
  else launch_vec3<VPI, false, false>(a, grid, lds, P, s);
  return true;
}

}  // namespace

hipError_t launch_ds_scan(const tsd_score_args& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.label_pool) & 15u) == 0;
  if (aligned && a.num_pages > 0 && a.r % 8 == 0) {
    switch (a.r / 8) {
      case 1: launch_vec<1>(a, s); return hipGetLastError();
      case 2: launch_vec<2>(a, s); return hipGetLastError();
      case 4: launch_vec<4>(a, s); return hipGetLastError();
      case 8: launch_vec<8>(a, s); return hipGetLastError();
      case 16: launch_vec<16>(a, s); return hipGetLastError();
      default: break;  // r = 24, 40, ...: the general kernel
    }
  }
  dim3 grid(static_cast<uint32_t>(a.pt_stride), static_cast<uint32_t>(a.B));
  hipLaunchKernelGGL(ds_scan_kernel, grid, dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(a.q), a.q_dtype == TSD_BF16,
                     a.H_q, a.H_kv, a.D, a.channel_idx, a.r,
                     static_cast<const uint16_t*>(a.label_pool), a.page_table,
                     a.pt_stride, a.seq_lens, a.num_pages, a.scores,
                     a.score_stride, a.row_lens_out);
  return hipGetLastError();
}

}  // namespace tsd
