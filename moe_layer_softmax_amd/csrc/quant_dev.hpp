// quant_dev.hpp -- device-side element conversions (OCP e4m3, OCP MX v1.0 e2m1 / E8M0), shared by
// the quantiser kernels and the GEMM epilogues that re-quantise the intermediate activations.
#pragma once

#include "common.hpp"

namespace moe {

// fp32 -> e4m3 (bias 7, no infinities, max 448): round to nearest even, saturate to +-448, keep the
// sign bit (a negative value rounding to zero gives negative zero).
__device__ __forceinline__ uint8_t e4m3_rne_sat(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint8_t sign = static_cast<uint8_t>((u >> 24) & 0x80u);
  const float a = fabsf(q);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                                     // below 2^-6: steps of 2^-9
    return sign | static_cast<uint8_t>(rintf(a * 512.0f));  // exact scaling; 8 -> 2^-6
  }
  uint32_t ua = __float_as_uint(a);
  ua += 0x7FFFFu + ((ua >> 20) & 1u);                      // round the mantissa to 3 bits (RNE)
  ua &= 0xFFF00000u;
  const int e = static_cast<int>(ua >> 23) - 127;
  const uint32_t m = (ua >> 20) & 7u;
  return sign | static_cast<uint8_t>(((e + 7) << 3) | m);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const int ef = (c >> 3) & 15, m = c & 7;
  float v = (ef == 0) ? ldexpf(static_cast<float>(m), -9) : ldexpf(1.0f + m * 0.125f, ef - 7);
  return (c & 0x80) ? -v : v;
}

// fp32 -> e2m1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6): nearest, ties to the even code, saturate.
__device__ __forceinline__ uint8_t e2m1_rne_sat(float y) {
  const uint8_t sign = static_cast<uint8_t>((__float_as_uint(y) >> 28) & 8u);
  const float a = fabsf(y);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return sign | c;
}

// Four fp32 values -> four e4m3 codes (value i in byte i) by the hardware conversion. Clamping the
// operands to +-448 first makes its round-to-nearest-even saturate as e4m3_rne_sat does; the two
// agree bit for bit (checked on the MI355X over every grid value, every tie and its neighbours,
// subnormals, +-0 and 440-620, at scales 2^-30 .. 2^30).
__device__ __forceinline__ uint32_t e4m3x4_rne_sat(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return static_cast<uint32_t>(w);
}

// Eight fp32 values -> eight e2m1 codes (value i in bits 4i .. 4i + 3) by the hardware conversion
// with a unit scale, which saturates itself and agrees with e2m1_rne_sat bit for bit (same check).
__device__ __forceinline__ uint32_t e2m1x8_rne_sat(const float* v) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
}

// Eight e2m1 codes (element i in bits 4i .. 4i + 3) times s as eight bf16 values (16 bytes). With s
// an e4m3 value every product is exact in fp32 and in bf16, so the upper half of each fp32 pattern
// is the bf16 value.
template <int B>
__device__ __forceinline__ int e2m1_pair_times(uint32_t w, float s) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);   // byte B: 2B, 2B + 1
  const float lo = v[0] * s, hi = v[1] * s;
  return static_cast<int>(__builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u));
}
__device__ __forceinline__ i32x4 e2m1x8_times(uint32_t w, float s) {
  return i32x4{e2m1_pair_times<0>(w, s), e2m1_pair_times<1>(w, s), e2m1_pair_times<2>(w, s),
               e2m1_pair_times<3>(w, s)};
}

// The same as fp16 (8 values, 16 bytes): q * s is exact in fp16 as well (at most 6 significant bits
// in [2^-10, 2688], inside fp16's normal range), and one packed fp16 multiply scales two elements.
// s must be exact in fp16 (an e4m3 value is).
template <int B>
__device__ __forceinline__ int e2m1_pair_times_f16(uint32_t w, f16x2 s2) {
  const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B) * s2;   // byte B: 2B, 2B + 1
  return __builtin_bit_cast(int, v);
}
__device__ __forceinline__ i32x4 e2m1x8_times_f16(uint32_t w, float s) {
  const _Float16 h = static_cast<_Float16>(s);
  const f16x2 s2 = f16x2{h, h};
  return i32x4{e2m1_pair_times_f16<0>(w, s2), e2m1_pair_times_f16<1>(w, s2),
               e2m1_pair_times_f16<2>(w, s2), e2m1_pair_times_f16<3>(w, s2)};
}

// shared exponent of an MX block: floor(log2(amax)) minus the element format's largest exponent
// (2 for e2m1, 8 for e4m3), clamped to [-127, 127]; -127 for amax = 0
template <int EMAX = 2>
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (amax == 0.0f) return -127;
  int ex;
  frexpf(amax, &ex);
  int e = ex - 1 - EMAX;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

}  // namespace moe
