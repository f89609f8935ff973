// Shared device helpers for the gfx950 microscaling kernels.
//
// Format facts used here (definitions restated from the pages, see mxq.h):
//  * MXFP8: 32 E4M3 values share one E8M0 (power-of-two) scale.
//  * NVFP4: E2M1 values, one E4M3 scale per 16 values, one FP32 scale per scope.
//
// gfx950 conversion instructions used, and the behaviour relied upon (checked
// exhaustively on MI355X against the CPU definitions over every finite BF16
// input and scales 2^-127 .. 2^127):
//  * v_cvt_scalef32_pk_fp8_bf16 / _f32 (x, scale): OCP E4M3 of x / scale with
//    round-to-nearest-even, sign of zero kept, E4M3 subnormals produced. Out of
//    range inputs are NOT saturated (some give NaN): callers guarantee
//    |x / scale| <= 448 (the MXFP8 round-up scale does) or clamp first.
//  * v_cvt_scalef32_pk_fp4_f32 (x, scale): E2M1 of x / scale, round-to-nearest-
//    even, saturating to +-6, sign of zero kept.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;
constexpr float kFltMax = 3.40282346638528859812e+38f;

// ---------------------------------------------------------------------------
// Lane exchanges
// ---------------------------------------------------------------------------
// DPP quad permutations: exchange with lane ^ 1 and lane ^ 2 inside groups of 4.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, 64);
}

// Packed maximum of two pairs of unsigned 16-bit integers (sign-cleared BF16
// bit patterns order like their magnitudes).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  us2 x, y;
  __builtin_memcpy(&x, &a, 4);
  __builtin_memcpy(&y, &b, 4);
  us2 m = __builtin_elementwise_max(x, y);
  uint32_t r;
  __builtin_memcpy(&r, &m, 4);
  return r;
}
__device__ __forceinline__ uint32_t max_halves(uint32_t v) {
  uint32_t lo = v & 0xFFFFu, hi = v >> 16;
  return lo > hi ? lo : hi;
}

// ---------------------------------------------------------------------------
// MXFP8 scale selection
// ---------------------------------------------------------------------------
// E8M0 code for a block whose largest magnitude has sign-cleared BF16 bits
// `amax_bits`: the smallest power of two 2^e with amax <= 448 * 2^e, as
// s = clamp(e + 127, 0, 254). With amax = (1 + M/128) * 2^(E-127):
// e = E - 127 - 8 when M <= 96 (mantissa <= 1.75), else E - 127 - 7. Zero and
// BF16-subnormal maxima clamp to s = 0; the largest BF16 gives s = 247.
__device__ __forceinline__ uint32_t e8m0_from_bf16_amax(uint32_t amax_bits) {
  int E = (int)((amax_bits >> 7) & 0xFF);
  int M = (int)(amax_bits & 0x7F);
  int s = E - 8 + (M > 96 ? 1 : 0);
  return (uint32_t)(s < 0 ? 0 : s);
}
// The same rule for MXFP4 blocks (E2M1 maximum 6 = 1.5 * 2^2): the smallest 2^e with
// amax <= 6 * 2^e, s = clamp(e + 127, 0, 254): e = E - 127 - 2 when M <= 64
// (mantissa <= 1.5), else E - 127 - 1.
__device__ __forceinline__ uint32_t e8m0_from_bf16_amax_e2m1(uint32_t amax_bits) {
  int E = (int)((amax_bits >> 7) & 0xFF);
  int M = (int)(amax_bits & 0x7F);
  int s = E - 2 + (M > 64 ? 1 : 0);
  return (uint32_t)(s < 0 ? 0 : s);
}
// 2^(127-s) as a float (exact); s = 254 gives the subnormal 2^-127.
__device__ __forceinline__ float e8m0_inverse(uint32_t s) {
  return __uint_as_float(s <= 253 ? (254u - s) << 23 : 0x00400000u);
}
// 2^(s-127) as a float; s = 0 gives the subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
}

// Two BF16 values (one dword, element 0 in the low half) -> two E4M3 bytes,
// written into the low (hi = false) or high (hi = true) 16 bits of `old`.
__device__ __forceinline__ uint32_t cvt_fp8x2_bf16(uint32_t old, uint32_t bf2, float scale, bool hi) {
  v2s o;
  __builtin_memcpy(&o, &old, 4);
  v2bf v;
  __builtin_memcpy(&v, &bf2, 4);
  o = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, v, scale, true)
         : __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, v, scale, false);
  uint32_t r;
  __builtin_memcpy(&r, &o, 4);
  return r;
}
__device__ __forceinline__ uint32_t cvt_fp8x2_f32(uint32_t old, float a, float b, float scale, bool hi) {
  v2s o;
  __builtin_memcpy(&o, &old, 4);
  o = hi ? __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, true)
         : __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, a, b, scale, false);
  uint32_t r;
  __builtin_memcpy(&r, &o, 4);
  return r;
}
// Two FP32 values -> one byte of two E2M1 nibbles (a in the low nibble) placed
// at byte `sel` (0..3) of `old`; scale 1.0 converts the values as given.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_f32(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// 16-byte global load with the non-temporal (streaming) hint, for inputs read once:
// measured on MI355X to lift read-heavy streams (a 268 MB BF16 input read once by the
// MXFP8 quantizer: 4.5 -> 5.6 TB/s); plain loads otherwise.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_stream16f(const float* p) {
  const uint4 v = load_stream16(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// BF16 element j (0/1) of a dword, widened to FP32 exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// FP32 -> BF16 bits, round-to-nearest-even (finite inputs; overflow -> Inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two FP32 -> two BF16 (RNE), element a in the low half: gfx950's packed convert. An
// exhaustive check over every non-NaN binary32 input (denormals included, in the
// library's denormal-preserving mode) matched f32_to_bf16_rne bit for bit.
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  v2f_t f;
  f.x = a;
  f.y = b;
  const v2bf_t h = __builtin_convertvector(f, v2bf_t);
  uint32_t o;
  __builtin_memcpy(&o, &h, 4);
  return o;
}
// Byte SEL of w (two E2M1 codes, low nibble first) -> two FP32 values, exact (hardware
// decode with scale 2^0; checked against e2m1_to_f32 on all 256 bytes).
template <int SEL>
__device__ __forceinline__ v2f_t e2m1x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// E4M3 byte -> FP32 (exact). Codes 0x7F/0xFF (NaN) never occur in our data.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;  // m * 2^-9
  return (c & 0x80) ? -mag : mag;
}
// E2M1 nibble -> FP32 (exact).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  uint32_t e = (c >> 1) & 3, m = c & 1;
  float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
  return (c & 8) ? -mag : mag;
}

}  // namespace mxq
