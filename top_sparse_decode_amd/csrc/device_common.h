// Device helpers shared by the gfx950 kernels of libtsd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TSD_DEVICE __device__ __forceinline__

namespace tsd {

constexpr int kWave = 64;
constexpr int kPage = 64;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Two OCP E4M3 values held in bytes (2*HI, 2*HI+1) of a dword, converted by
// the gfx950 hardware converter (OCP encoding on this target).
template <bool HI>
TSD_DEVICE float2 fp8x2_to_f32(uint32_t w) {
  auto r = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  return make_float2(r[0], r[1]);
}

// Four E4M3 values of one dword.
TSD_DEVICE void fp8x4_to_f32(uint32_t w, float* out) {
  float2 a = fp8x2_to_f32<false>(w);
  float2 b = fp8x2_to_f32<true>(w);
  out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
}

TSD_DEVICE float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

TSD_DEVICE float fp16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// 16-bit element -> f32 for the two 16-bit encodings (is_bf16 selects).
TSD_DEVICE float half_to_f32(uint16_t h, bool is_bf16) {
  return is_bf16 ? bf16_to_f32(h) : fp16_to_f32(h);
}

// Order-preserving map f32 -> u32 (larger float -> larger key); -0 is
// folded onto +0 first so that the two compare equal, as floats do.
TSD_DEVICE uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Butterfly over the 64 lanes of a wave: DPP moves within each 16-lane row
// (quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors),
// then the gfx950 lane swaps across rows (permlane16_swap) and halves
// (permlane32_swap). Every lane returns the combination of all 64.
template <typename Op>
TSD_DEVICE uint32_t wave_butterfly(uint32_t v, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                0, static_cast<int>(v), 0xB1, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                0, static_cast<int>(v), 0x4E, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                0, static_cast<int>(v), 0x141, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                0, static_cast<int>(v), 0x140, 0xf, 0xf, false)));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}

TSD_DEVICE float wave_max(float v) {
  return __uint_as_float(wave_butterfly(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

TSD_DEVICE float wave_sum(float v) {
  return __uint_as_float(wave_butterfly(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

TSD_DEVICE uint32_t wave_sum_u32(uint32_t v) {
  return wave_butterfly(v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive prefix sum across the 64 lanes of a wave, on DPP lane moves:
// shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted past the
// row start read 0), then lane 15 of rows 0 and 2 is added into rows 1 and
// 3 (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).
TSD_DEVICE uint32_t wave_inclusive_scan(uint32_t v) {
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false));
  return v;
}

// Reduce-scatter of four 16x16 MFMA tiles over the 4 lane groups of a wave:
// lane l = 16*g + j holds part[i] = its partial for key j of tile i; the
// result in lane l is sum over the 4 groups of part[g] at key j, i.e. the
// total for key 16*g + j. Done with the gfx950 lane-swap instructions:
// permlane32_swap(a, b) gives ([a_lo, b_lo], [a_hi, b_hi]) over the two
// 32-lane halves, permlane16_swap the same over 16-lane rows.
TSD_DEVICE float reduce_scatter4(const float part[4]) {
  const auto r02 = __builtin_amdgcn_permlane32_swap(
      __float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
  const auto r13 = __builtin_amdgcn_permlane32_swap(
      __float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
  // lower half: tiles 0 and 1 over groups {g, g+2}; upper half: tiles 2, 3
  const float u = __uint_as_float(r02[0]) + __uint_as_float(r02[1]);
  const float v = __uint_as_float(r13[0]) + __uint_as_float(r13[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(
      __float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Clamp a device-side length to [0, cap].
TSD_DEVICE int64_t clamp_len(int64_t n, int64_t cap) {
  return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace tsd
