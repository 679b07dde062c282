// kvq_rows.h — row helpers shared by the cache write / convert kernels and the
// one-call decode step's new-token write: one row of head_dim values is held by
// LPR = head_dim / 8 aligned consecutive lanes, 8 values each (x[i] = element
// 8 j + i of the row, j the lane's place in its group); cross-lane moves stay
// inside the group.  The encoders (INT8 / FP8 with a tensor or head scale, INT4
// with the row's own scale and zero point) and the Hadamard rotation of rotated
// keys.
#pragma once

#include <type_traits>

#include "kvq_device.h"

namespace kvq {

namespace {

// ---------------------------------------------------------------------------
// cross-lane moves inside the aligned group of LPR lanes that holds a row
// ---------------------------------------------------------------------------

// the value of lane (this lane xor M), for M = 1, 2 (DPP quad permutes) and
// 4, 8 (LDS-crossbar swizzles, no address operand)
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  // quad permutes read a valid lane everywhere, so no old value is needed
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, true);
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, true);
  else if constexpr (M == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);   // swap groups of 4
  else return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x201F);                        // swap groups of 8
}
template <int M>
__device__ __forceinline__ double xor_lane(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xor_lane<M>((uint32_t)u), hi = xor_lane<M>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// max / min over the row's LPR lanes (8 or 16, aligned), by DPP moves: within
// quads, then half-rows (lane i with 7 - i), then rows (i with 15 - i)
template <int LPR>
__device__ __forceinline__ void row_min_max(float& mn, float& mx) {
  static_assert(LPR == 8 || LPR == 16, "lanes per row");
  // every control below reads a valid lane of the same row: no old value needed
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, true));
  };
  using Xor1 = std::integral_constant<int, 0xB1>;   // quad_perm [1, 0, 3, 2]
  using Xor2 = std::integral_constant<int, 0x4E>;   // quad_perm [2, 3, 0, 1]
  using HalfMirror = std::integral_constant<int, 0x141>;
  using Mirror = std::integral_constant<int, 0x140>;
  mn = fminf(mn, dpp(mn, Xor1{}));
  mx = fmaxf(mx, dpp(mx, Xor1{}));
  mn = fminf(mn, dpp(mn, Xor2{}));
  mx = fmaxf(mx, dpp(mx, Xor2{}));
  mn = fminf(mn, dpp(mn, HalfMirror{}));
  mx = fmaxf(mx, dpp(mx, HalfMirror{}));
  if constexpr (LPR == 16) {
    mn = fminf(mn, dpp(mn, Mirror{}));
    mx = fmaxf(mx, dpp(mx, Mirror{}));
  }
}

// ---------------------------------------------------------------------------
// encoders of the 8 values a lane holds (x[i] = element 8 j + i of the row)
// ---------------------------------------------------------------------------

// INT8 / FP8 codes with the tensor's (or head's) scale s: 8 bytes
template <int DT>
__device__ __forceinline__ uint2 encode_8bit(const float (&x)[8], float s) {
  const Quot qt(s);
  float t[2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i / 4][i % 4] = qt(x[i]);
  uint32_t lo = 0, hi = 0;
  if constexpr (DT == DT_INT8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= enc_int8(t[0][i]) << (8 * i);
      hi |= enc_int8(t[1][i]) << (8 * i);
    }
  } else {
    lo = enc_fp8x4<DT>(t[0]);
    hi = enc_fp8x4<DT>(t[1]);
  }
  return make_uint2(lo, hi);
}

// fl(a / 15), correctly rounded: one Markstein step from the correctly rounded
// reciprocal of 15 (0x3D888889) when a is large enough for no step to
// underflow; a true division otherwise.  Infinite or NaN a gives inf or NaN.
__device__ __forceinline__ float div15(float a) {
  if (!(fabsf(a) >= 0x1p-100f) || !(fabsf(a) <= 0x1p100f)) return a / 15.0f;
  const float r = __uint_as_float(0x3D888889u);
  const float q0 = a * r;
  return __builtin_fmaf(__builtin_fmaf(-q0, 15.0f, a), r, q0);
}

// INT4 asymmetric codes of the row: s = (max - min) / 15 (|min| or 1 for a
// constant row), zp = RNE(-min / s) (+0 when zero), q = clamp(RNE(x / s) + zp,
// 0, 15), every
// quotient the correctly rounded float32 one; NaN elements are left out of
// min / max and get code 0.  Returns the 8 nibbles (even element low); the
// row's (s, zp) in *s_out, *zp_out.
template <int LPR>
__device__ __forceinline__ uint32_t encode_int4(const float (&x)[8], float* s_out, float* zp_out) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
  row_min_max<LPR>(mn, mx);
  float sc = div15(mx - mn);
  if (sc == 0.0f || !(fabsf(sc) <= 3.402823466e38f)) sc = (mn != 0.0f) ? fabsf(mn) : 1.0f;
  const Quot qt(sc);
  // + 0: a zero zero point is +0 whichever zero the row minimum came out as
  // (the minimum of a row holding both -0 and +0 depends on the order)
  const float zp = rintf(qt(-mn)) + 0.0f;
  float q[8];
  if (qt.fast) {
    // with a normal scale only the upper half of the quotient's range test is
    // kept: below 2^-60 both the corrected and the uncorrected quotient round to
    // 0, so the code is the same; above 2^60 (an infinite x among them, whose
    // correction would be inf - inf) the uncorrected one saturates the code
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = x[i] * qt.r;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, sc, x[i]), qt.r, q0);
      q[i] = rintf(fabsf(q0) <= 0x1p60f ? q1 : q0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = rintf(x[i] / sc);
  }
  // codes in [0, 15] (fmaxf takes a NaN to 0); pairs (even, odd) as the exact
  // byte value even + 16 odd
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float e = fminf(fmaxf(q[i] + zp, 0.0f), 15.0f);
    const float o = fminf(fmaxf(q[i + 1] + zp, 0.0f), 15.0f);
    packed = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(o, 16.0f, e), i / 2, packed);
  }
  *s_out = sc;
  *zp_out = zp;
  return packed;
}

// A float32 whose rounding to bf16 (nearest even) equals the rounding of the
// float64 v itself.  The hardware narrows v to the nearest float32 f (ties to
// even, subnormals kept); rounding f to bf16 then equals rounding v except where
// f lies exactly halfway between two bf16 values while v does not.  f is within
// half a float32 ulp of v, so no such halfway point lies strictly between them:
// moving f one float32 ulp toward v makes the final rounding go v's way.
// Overflow then rounds to the infinity the direct rounding gives; NaN stays NaN.
__device__ __forceinline__ float f64_to_f32_for_bf16(double v) {
  const float f = (float)v;
  uint32_t u = __float_as_uint(f);
  if ((u & 0xffffu) == 0x8000u) {
    const double fd = (double)f;
    if (fd != v && v == v) u += (fabs(v) > fabs(fd)) ? 1u : 0xffffffffu;
  }
  return __uint_as_float(u);
}

// The unnormalised Walsh-Hadamard transform of a row held by LPR aligned lanes,
// 8 values each (x[i] = element 8 j + i): y = H x with H[i][k] =
// (-1)^popcount(i & k), by the butterfly (stages h = 1, 2, 4 inside the lane,
// then h = 8 .. D/2 between lanes j and j ^ (h / 8); the pair at (i, i + h)
// becomes (a + b, a - b)) in float64, where every sum is exact while the row's
// magnitudes span less than 2^38 (bf16 values carry 8 significant bits; D <=
// 128 terms add 7 more), then rounded once to bf16 (returned as float32).  An
// exact zero comes out as +0.
template <int M>
__device__ __forceinline__ void hadamard_lane_stage(double (&y)[8], int j) {
  // the lower lane of a pair keeps y + other, the upper other - y: one fma with
  // a factor of +-1, rounded once like the add or subtraction it stands for
  // (zeros included: x + (-x) is +0 either way)
  const double sgn = (j & M) ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double other = xor_lane<M>(y[i]);
    y[i] = __builtin_fma(sgn, y[i], other);
  }
}
template <int LPR>
__device__ __forceinline__ void hadamard_row(float (&x)[8], int j) {
  double y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = (double)x[i];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & h)) {
        const double a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  hadamard_lane_stage<1>(y, j);
  hadamard_lane_stage<2>(y, j);
  hadamard_lane_stage<4>(y, j);
  if constexpr (LPR == 16) hadamard_lane_stage<8>(y, j);
  // float64 -> float32 with the bf16 double-rounding case fixed, then the pair
  // to bf16 by the hardware conversion (nearest even) and back to float32
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const float a = f64_to_f32_for_bf16(y[i] + 0.0), b = f64_to_f32_for_bf16(y[i + 1] + 0.0);
    const bf16x2n v = {(__bf16)a, (__bf16)b};
    const uint32_t w = __builtin_bit_cast(uint32_t, v);
    x[i] = __uint_as_float(w << 16);
    x[i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}

}  // namespace

}  // namespace kvq
