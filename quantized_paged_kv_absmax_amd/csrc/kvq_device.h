// kvq_device.h — device-side element codecs and small helpers for gfx950.
//
// Encode rules (quantise a float32 x with scale s; x / s is IEEE correctly
// rounded — hipcc's default, never -ffast-math):
//   INT8  q = clamp(RNE(x / s), -127, 127), NaN -> 0
//         (the INT8 KV cache of the sm86 summary; RNE and the symmetric range
//          are this library's reading)
//   FP8   OCP e4m3 / e5m2 nearest value of x / s, ties to even, saturating to
//         the largest finite value, NaN -> NaN code (the fp8_e4m3 / fp8_e5m2
//         cache dtypes of vLLM PR 4893, description item 1)
//   INT4  per row: s = (max - min) / 15, zp = RNE(-min / s), q = clamp(RNE(x / s)
//         + zp, 0, 15) (vLLM issue 4025, methods item 1: scale + zero point)
// Decode happens inside the attention kernel (decode.hip) as an exact conversion
// of the codes to fp16 / bf16 MFMA operands, with the scales applied to the
// float32 products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// DT_INT4H: INT4 codes of the Hadamard-rotated row (keys only)
enum : int { DT_BF16 = 0, DT_INT8 = 1, DT_E4M3 = 2, DT_E5M2 = 3, DT_INT4 = 4, DT_F32 = 5, DT_INT4H = 6 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest even (NaN -> quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// encoders
// ---------------------------------------------------------------------------

// x / s as the correctly rounded float32 quotient, from r = 1 / s (one division
// per scale instead of one per element): q0 = x r is within an ulp of x / s, the
// residual x - q0 s is exact through fma, and one correction step q0 + r (x - q0 s)
// rounds to the correctly rounded quotient (Markstein's theorem, given r
// correctly rounded and no underflow or overflow in the steps).  Scales outside
// [2^-60, 2^60] divide.  Where |q0| lies outside [2^-60, 2^60] the uncorrected
// q0 is kept: there every encoder below gives the same code for q0 as for x / s
// (0, or a saturated code), and inside it, with such scales, no step underflows
// for any quotient whose code can differ from 0.
struct Quot {
  float s, r;
  bool fast;
  __device__ __forceinline__ explicit Quot(float scale) : s(scale) {
    const float a = fabsf(scale);
    fast = a >= 0x1p-60f && a <= 0x1p60f;
    r = 1.0f / scale;
  }
  __device__ __forceinline__ float operator()(float x) const {
    if (!fast) return x / s;
    const float q0 = x * r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
    const float a = fabsf(q0);
    return (a >= 0x1p-60f && a <= 0x1p60f) ? q1 : q0;
  }
};

// INT8 code of a quotient t: RNE, clamped to [-127, 127]; NaN -> 0
__device__ __forceinline__ uint32_t enc_int8(float t) {
  if (t != t) return 0u;
  t = fminf(fmaxf(rintf(t), -127.0f), 127.0f);
  return (uint32_t)(int32_t)t & 0xffu;
}

template <int DT> struct Fp8Fmt;
template <> struct Fp8Fmt<DT_E4M3> { static constexpr float kMax = 448.0f; };
template <> struct Fp8Fmt<DT_E5M2> { static constexpr float kMax = 57344.0f; };

// OCP fp8 codes of four float32 values (byte i from t[i]): nearest code, ties
// to even, saturating at the largest finite code (infinities included), and a
// NaN becomes 0x7f with its sign.  The hardware conversion rounds to nearest
// even; clamping its input to +-max first makes it saturate, and NaN inputs are
// patched.  Equal to that definition on every float32 input, both formats.
template <int DT>
__device__ __forceinline__ uint32_t enc_fp8x4(const float (&t)[4]) {
  constexpr float M = Fp8Fmt<DT>::kMax;
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(t[i], -M), M);
  uint32_t w;
  if constexpr (DT == DT_E4M3) {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)w, true);
  } else {
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], (int)w, true);
  }
  if ((t[0] != t[0]) | (t[1] != t[1]) | (t[2] != t[2]) | (t[3] != t[3])) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t[i] != t[i]) {
        const uint32_t code = ((__float_as_uint(t[i]) >> 24) & 0x80u) | 0x7fu;
        w = (w & ~(0xffu << (8 * i))) | (code << (8 * i));
      }
    }
  }
  return w;
}

// ---------------------------------------------------------------------------
// byte permutes and fp16 magic-number conversions (exact)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// halves (1024 + b0, 1024 + b1) from bytes 0,1 (sel 0x04010400) or 2,3 (sel 0x04030402)
// of x: the byte becomes the low mantissa byte of an fp16 with exponent 2^10.
constexpr uint32_t kMagic64 = 0x64646464u;
// the same with bf16 128 (0x4300): halves (128 + b0, 128 + b1), exact for b < 128
constexpr uint32_t kMagic43 = 0x43434343u;
constexpr uint32_t kSelLo = 0x04010400u;
constexpr uint32_t kSelHi = 0x04030402u;

// fp8 e4m3 pair (bytes 0,1 or 2,3 of w) -> two fp16 (exact; NaN stays NaN)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------


// max / sum of v over the lane pairs (l, l ^ 16), or (l, l ^ 32), through the
// gfx950 row-swap instructions instead of the LDS crossbar.  Swapping v with
// itself, v_permlane16_swap leaves rows (r0, r0, r2, r2) in one result and
// (r1, r1, r3, r3) in the other; v_permlane32_swap leaves (lo, lo) and (hi, hi).
// Both lanes of a pair combine the two values in the same order.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float shfl_f(float v, int src) { return __shfl(v, src, 64); }

}  // namespace kvq
