// Device helpers shared by the gfx950 kernels of the scaled FP8 GEMM library.
//
// Format facts used here (OCP OFP8 E4M3 "fn", the operand format the JAX/Triton
// Blackwell FP8 GEMM post prefers; OCP MX v1.0 E8M0 for the MXFP8 scales named in
// "Hopper/Blackwell architecture features" §12.6.1):
//   * e4m3fn has no infinity; its largest finite magnitude is 448.
//   * gfx950's v_cvt_pk_fp8_f32 rounds to nearest even onto OCP e4m3fn, including
//     subnormals and ties, but turns magnitudes above 464 into NaN, so every value
//     is clamped to [-448, 448] first (448 is what round-then-saturate gives).
//   * e5m2 (the post's second FP8 format; OCP OFP8 E5M2) has infinities; its
//     largest finite magnitude is 57344.  v_cvt_pk_bf8_f32 converts onto it, and
//     values are clamped to [-57344, 57344] first, so the quantisers saturate
//     instead of producing infinity.
//   * e2m1 (FP4, the MXFP4 element; OCP MX v1.0) has magnitudes 0, 0.5, 1, 1.5, 2,
//     3, 4, 6 and no infinity or NaN; it is encoded here in software (round to a
//     multiple of the binade's spacing with v_rndne, saturating at 6).
//   * e2m3 and e3m2 (FP6, the MXFP6 elements; OCP MX v1.0) have largest
//     magnitudes 7.5 and 28 and no infinity or NaN; they are encoded in software
//     like e2m1.
//   * E8M0 code c encodes 2^(c-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace fp8gemm {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;


__device__ __forceinline__ float clamp448(float v) {
  return fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
}

// Four fp32 values -> four e4m3fn codes packed little-endian into 32 bits
// (round to nearest even, saturating, sign of zero kept).
__device__ __forceinline__ uint32_t encode4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return (uint32_t)w;
}

// Four fp32 values -> four e5m2 codes packed little-endian into 32 bits (round to
// nearest even, saturating at 57344, sign of zero kept).
__device__ __forceinline__ uint32_t encode4_e5m2(float a, float b, float c, float d) {
  auto clamp = [](float v) { return fminf(fmaxf(v, -kE5M2Max), kE5M2Max); };
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp(a), clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp(c), clamp(d), w, true);
  return (uint32_t)w;
}

// One fp32 value -> e2m1 code (bits 0-3): round to nearest even onto the grid of
// spacing 0.5 below 2, 1 below 4 and 2 above (multiplications by powers of two
// and rintf, all exact), saturating at 6; the sign goes to bit 3, so -0 gives
// 0x8.  The code of the rounded magnitude r: 2r for r < 1 (0 or 0.5); else the
// exponent field plus one, doubled, with the top mantissa bit as the last bit.
__device__ __forceinline__ uint32_t encode_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  const float up = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);   // 1 / spacing
  const float dn = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);   // spacing
  const float r = fminf(rintf(a * up) * dn, 6.0f);
  const uint32_t b = __float_as_uint(r);
  const uint32_t mag = r < 1.0f ? (uint32_t)(r * 2.0f)
                                : ((((b >> 23) - 126u) << 1) | ((b >> 22) & 1u));
  return sign | mag;
}

// Four fp32 values -> four e2m1 codes in 16 bits, the first in bits 0-3.
__device__ __forceinline__ uint32_t encode4_e2m1(float a, float b, float c, float d) {
  return encode_e2m1(a) | (encode_e2m1(b) << 4) | (encode_e2m1(c) << 8) | (encode_e2m1(d) << 12);
}

// One fp32 value -> FP6 code (bits 0-5): e2m3 (bias 1, 3 mantissa bits, largest
// 7.5) or e3m2 (bias 3, 2 mantissa bits, largest 28), round to nearest even,
// saturating; the sign goes to bit 5, so -0 gives 0x20.  The magnitude is
// rounded to a multiple of its binade's spacing 2^(E - mantissa bits), E =
// floor(log2 |v|) from the binary32 exponent, no smaller than the smallest
// normal exponent 1 - bias (the subnormal spacing continues below it): a
// multiplication by the power of two 1 / spacing, rintf, and the inverse
// multiplication, all exact.  The code of the rounded magnitude r: r / spacing
// below the smallest normal; else the exponent field (exponent + bias) and the
// top mantissa bits of r.
template <int FMT>
__device__ __forceinline__ uint32_t encode_fp6(float v) {
  constexpr int kBias = FMT == kE2M3 ? 1 : 3;
  constexpr int kMb = FMT == kE2M3 ? 3 : 2;
  constexpr float kMax = FMT == kE2M3 ? 7.5f : 28.0f;
  constexpr float kMinNormal = FMT == kE2M3 ? 1.0f : 0.25f;
  constexpr float kSubScale = FMT == kE2M3 ? 8.0f : 16.0f;    // 1 / subnormal spacing
  const uint32_t sign = (__float_as_uint(v) >> 26) & 0x20u;
  const float a = fabsf(v);
  int e = (int)(__float_as_uint(a) >> 23) - 127;
  e = e < 1 - kBias ? 1 - kBias : e;                     // in [1 - bias, 128]
  const float up = __uint_as_float((uint32_t)(127 + kMb - e) << 23);   // 1 / spacing
  const float dn = __uint_as_float((uint32_t)(127 - kMb + e) << 23);   // spacing
  const float r = fminf(rintf(a * up) * dn, kMax);
  const uint32_t b = __float_as_uint(r);
  const uint32_t mag = r < kMinNormal
                           ? (uint32_t)(r * kSubScale)
                           : ((((b >> 23) - 127u + kBias) << kMb) | ((b >> (23 - kMb)) & ((1u << kMb) - 1)));
  return sign | mag;
}

// Four fp32 values -> four FP6 codes in the low 24 bits, the first in bits 0-5.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_fp6(float a, float b, float c, float d) {
  return encode_fp6<FMT>(a) | (encode_fp6<FMT>(b) << 6) | (encode_fp6<FMT>(c) << 12) |
         (encode_fp6<FMT>(d) << 18);
}

template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  return FMT == kE5M2 ? encode4_e5m2(a, b, c, d) : encode4_e4m3(a, b, c, d);
}

template <int FMT>
constexpr float elem_max() {
  return FMT == kE5M2 ? kE5M2Max : kE4M3Max;
}

// E8M0 code of a 32-element block from its largest magnitude: floor(log2 amax)
// read from the binary32 exponent field, minus the element format's largest
// exponent (8 for e4m3, 15 for e5m2, 2 for e2m1 and e2m3, 4 for e3m2), biased by
// 127 and clamped to [0, 254]; an
// all-zero block gets 127.
template <int FMT = kE4M3>
__device__ __forceinline__ uint32_t mx_code_from_amax(float amax) {
  if (amax == 0.0f) return 127u;
  int ef = (int)(__float_as_uint(amax) >> 23);  // amax >= 0: no sign bit
  int code = ef - (FMT == kE5M2 ? 15 : (FMT == kE2M1 || FMT == kE2M3) ? 2 : FMT == kE3M2 ? 4 : 8);
  return (uint32_t)(code < 0 ? 0 : code);
}

// Largest value over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Largest value over the `width` lanes of an aligned lane group (width <= 64).
__device__ __forceinline__ float group_max(float v, int width) {
  for (int off = width >> 1; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// fp32 -> output element, round to nearest even.
template <typename OutT>
__device__ __forceinline__ OutT to_out(float v);

template <>
__device__ __forceinline__ _Float16 to_out<_Float16>(float v) {
  return (_Float16)v;
}
template <>
__device__ __forceinline__ __bf16 to_out<__bf16>(float v) {
  return (__bf16)v;
}

// bf16 output whose magnitudes the epilogue also folds into maxima (the first
// half of the requantised output): stored exactly as __bf16.
struct bf16_max {
  uint16_t bits;
};
template <typename OutT>
constexpr bool kTrackMax = std::is_same<OutT, bf16_max>::value;

template <>
__device__ __forceinline__ bf16_max to_out<bf16_max>(float v) {
  return __builtin_bit_cast(bf16_max, (__bf16)v);
}

// Largest magnitude of the bf16 values packed in n 32-bit words (two per word).
__device__ __forceinline__ float absmax_bf16(const uint32_t* w, int n) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i)
    a = fmaxf(a, fmaxf(fabsf(__uint_as_float(w[i] << 16)),
                       fabsf(__uint_as_float(w[i] & 0xffff0000u))));
  return a;
}

// Four consecutive outputs packed into 8 bytes.
template <typename OutT>
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  OutT o[4] = {to_out<OutT>(a), to_out<OutT>(b), to_out<OutT>(c), to_out<OutT>(d)};
  uint2 r;
  __builtin_memcpy(&r, o, 8);
  return r;
}

}  // namespace fp8gemm
