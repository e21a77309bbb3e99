// Device-side building blocks shared by the NVFP4 kernels (gfx950 only).
//
// NVFP4 element and scale encodings are the OCP Microscaling Formats v1.0
// FP4 E2M1 and FP8 E4M3 types (the pages name NVFP4 without defining its
// bits).  Every helper here is exact unless its comment says otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace nvfp4 {

constexpr int kWave = 64;
constexpr float kQuantRange = 2688.0f;  // 6 (largest E2M1) * 448 (largest E4M3)

// ---------------------------------------------------------------------------
// Decoders
// ---------------------------------------------------------------------------

// E4M3 byte -> fp32, exact.  Normal: 2^(e-7) (1 + m/8); subnormal: m 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                      : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// Two E2M1 codes in byte `sel` (0..3) of `word` -> fp16 pair {low nibble,
// high nibble}, exact (gfx950 v_cvt_scalef32_pk_f16_fp4 with unit scale).
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_to_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

// Eight E2M1 codes (one 32-bit word, element 0 in the low nibble) times an
// fp16 block scale -> eight fp16 values.  Every e2m1*e4m3 product has at most
// 6 significant bits and lies in [2^-10, 2688], so it is exact in fp16.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t word, f16x2 s2) {
  const f16x2 p0 = e2m1x2_to_f16<0>(word) * s2;
  const f16x2 p1 = e2m1x2_to_f16<1>(word) * s2;
  const f16x2 p2 = e2m1x2_to_f16<2>(word) * s2;
  const f16x2 p3 = e2m1x2_to_f16<3>(word) * s2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Two E4M3 block scales (bytes 0 and 1 of `w`) -> fp16 pairs {s0, s0} and
// {s1, s1}.  E4M3 values have 4 significant bits and lie in [2^-9, 448], so
// the conversion (gfx950 v_cvt_scalef32_pk_f16_fp8, unit scale) is exact.
__device__ __forceinline__ void e4m3x2_to_f16_pairs(uint32_t w, f16x2 &s0, f16x2 &s1) {
  const f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  s0[0] = s[0]; s0[1] = s[0];
  s1[0] = s[1]; s1[1] = s[1];
}

// ---------------------------------------------------------------------------
// Encoders (round to nearest, ties to even, saturating)
// ---------------------------------------------------------------------------

// Nearest E4M3 code of a finite v >= 0; v >= 448 gives 0x7E.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0x1p-6f) {
    // subnormal range: code = m with value m 2^-9; m == 8 is 2^-6 = 0x08
    return (uint32_t)__builtin_rintf(v * 512.0f);
  }
  const uint32_t bits = __float_as_uint(v);
  const uint32_t r = bits + 0x7FFFFu + ((bits >> 20) & 1u);  // RNE to 3 mantissa bits
  return (r >> 20) - (120u << 3);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Exponent of a finite non-zero |v| (floor(log2 |v|)), 0 for v == 0.
__device__ __forceinline__ int exponent_of(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int e = (int)((b >> 23) & 255u);
  if (e == 0) return -118 - __clz(b & 0x7FFFFFu);  // fp32 subnormal: 2^(31-clz-149)
  return e - 127;
}

// ---------------------------------------------------------------------------
// Wavefront reductions (deterministic butterfly order)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// One 16-element NVFP4 block quantisation (fp32 steps in a fixed order)
// ---------------------------------------------------------------------------

struct Block16 {
  uint32_t lo, hi;   // packed codes, element 2i in the low nibble of byte i
  uint32_t scale;    // E4M3 code
  float sdec;        // decoded block scale
};

// amax_b / (6 g) -> E4M3, then code = E2M1(x * (1 / (e4m3 * g))).
// g must be > 0.  Contraction into FMAs is disabled: each step is one
// correctly rounded fp32 operation.
__device__ __forceinline__ Block16 quantize_block16(const float (&x)[16], float g) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(x[i]));
  const float six_g = 6.0f * g;
  const float s_f = amax / six_g;
  Block16 b;
  b.scale = e4m3_rne_sat(s_f);
  b.sdec = e4m3_to_f32(b.scale);
  const float denom = b.sdec * g;
  b.lo = 0u;
  b.hi = 0u;
  if (denom > 0.0f) {
    const float inv = 1.0f / denom;
    // gfx950's packed fp32 -> E2M1 converter with unit scale: the nearest
    // E2M1 value, ties to even, |v| > 6 -> 6, the sign bit kept (a negative
    // value rounding to zero gives code 0x8); operand 0 goes to the low
    // nibble of byte SEL.  (Checked on the device against these rules for
    // every multiple of 1/128 in [-9.4, 9.4], the tie points, zeros,
    // denormals and huge values.)
#define NVFP4_ENC(W, SEL, A, B) \
  W = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(W, (A) * inv, (B) * inv, 1.0f, SEL)
    NVFP4_ENC(b.lo, 0, x[0], x[1]);
    NVFP4_ENC(b.lo, 1, x[2], x[3]);
    NVFP4_ENC(b.lo, 2, x[4], x[5]);
    NVFP4_ENC(b.lo, 3, x[6], x[7]);
    NVFP4_ENC(b.hi, 0, x[8], x[9]);
    NVFP4_ENC(b.hi, 1, x[10], x[11]);
    NVFP4_ENC(b.hi, 2, x[12], x[13]);
    NVFP4_ENC(b.hi, 3, x[14], x[15]);
#undef NVFP4_ENC
  }
  return b;
}

// Tensor decode scale from its absolute maximum: amax / 2688, or 1 for zero.
__device__ __forceinline__ float global_from_amax(float amax) {
#pragma clang fp contract(off)
  return amax > 0.0f ? amax / kQuantRange : 1.0f;
}

}  // namespace nvfp4
