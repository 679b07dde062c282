// cache_write.hip — fused quantise-and-scatter of K/V rows into the paged cache
// (vLLM issue 4025, methods item 2) and conversion of an existing bf16 paged
// cache (methods item 1).
//
// One row = head_dim bf16 values of one (token, KV head).  A row is handled by
// D/8 consecutive lanes, each loading 16 bytes (8 values) and storing 8 codes
// (8 bytes; 4 bytes for INT4).  INT4 finds the row's min / max with xor
// moves inside the lane group, and the group's first lane stores the (scale,
// zero point) pair.  Blocks in y = 0 encode K, y = 1 encode V, so a launch
// streams both tensors; each workgroup switches once on its side's element
// format into a path specialised for it.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kThreads = 256;

struct RowSide {
  const uint16_t* src;      // bf16 rows
  uint8_t* pages;
  const float* scale;       // [1] or [Hkv] or null
  int scale_per_head;
  float* meta;              // int4 (scale, zp)
  int dtype;
};

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

// this lane's 16 source bytes of a row, and the row's scale
struct RowIn {
  uint4 raw;
  float s;
};

template <int D, int DT>
__device__ __forceinline__ RowIn load_row(const RowSide& sd, const uint16_t* src_row, int h, int j) {
  RowIn in;
  in.raw = *reinterpret_cast<const uint4*>(src_row + 8 * j);
  if constexpr (DT == DT_INT8 || DT == DT_E4M3 || DT == DT_E5M2)
    in.s = sd.scale ? sd.scale[sd.scale_per_head ? h : 0] : 1.0f;
  else
    in.s = 1.0f;
  return in;
}

// encode the lane's 8 values of a row and store them at row dst_row_idx of the pages
template <int D, int DT>
__device__ __forceinline__ void store_row(const RowSide& sd, const RowIn& in, int64_t dst_row_idx, int j) {
  constexpr int LPR = D / 8;
  const uint4 raw = in.raw;
  if constexpr (DT == DT_BF16) {
    *reinterpret_cast<uint4*>(sd.pages + dst_row_idx * (2 * D) + 16 * j) = raw;
  } else {
    float x[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
    if constexpr (DT == DT_INT4 || DT == DT_INT4H) {
      if constexpr (DT == DT_INT4H) hadamard_row<LPR>(x, j);
      float sc, zp;
      const uint32_t packed = encode_int4<LPR>(x, &sc, &zp);
      *reinterpret_cast<uint32_t*>(sd.pages + dst_row_idx * (D / 2) + 4 * j) = packed;
      if (j == 0) *reinterpret_cast<float2*>(sd.meta + dst_row_idx * 2) = make_float2(sc, zp);
    } else {
      *reinterpret_cast<uint2*>(sd.pages + dst_row_idx * D + 8 * j) = encode_8bit<DT>(x, in.s);
    }
  }
}

// Each lane takes kRowsPerLane rows (kRowsPerLane x 16 bytes in flight before any
// encode); the rows of one pass are consecutive, the passes of a workgroup too.
constexpr int kRowsPerLane = 4;

// rows of a workgroup for the cache write, format DT known at compile time
template <int D, bool R32, int DT>
__device__ __forceinline__ void write_rows(const RowSide& sd, const int64_t* slots, int64_t T, int Hkv,
                                           int64_t num_slots, int32_t* err) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;  // rows per pass
  const int j = threadIdx.x % LPR;
  const int64_t rows = T * Hkv;
  const int64_t row0 = (int64_t)blockIdx.x * RPB * kRowsPerLane + threadIdx.x / LPR;
  // every row's source, scale and slot loads go out before the first store
  RowIn in[kRowsPerLane];
  int64_t slot[kRowsPerLane];
  int hh[kRowsPerLane];
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t row = row0 + (int64_t)u * RPB;
    const int64_t rr = row < rows ? row : rows - 1;
    int64_t t;
    int h;
    if constexpr (R32) {
      t = (int64_t)((uint32_t)rr / (uint32_t)Hkv);
      h = (int)((uint32_t)rr - (uint32_t)t * (uint32_t)Hkv);
    } else {
      t = rr / Hkv;
      h = (int)(rr % Hkv);
    }
    in[u] = load_row<D, DT>(sd, sd.src + rr * D, h, j);
    slot[u] = row < rows ? slots[t] : -1;
    hh[u] = h;
  }
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t sl = slot[u];
    if (sl < 0) continue;                       // uniform over the row's lanes
    if (sl >= num_slots) {
      if (err && blockIdx.y == 0 && hh[u] == 0 && j == 0) atomicAdd(err, 1);
      continue;
    }
    const int64_t blk = sl / 16, off = sl % 16;
    store_row<D, DT>(sd, in[u], (blk * Hkv + hh[u]) * 16 + off, j);
  }
}

// R32: the row count fits 31 bits, so (token, head) come from a 32-bit division.
// Workgroups in y = 0 write K, y = 1 V; the format switch is uniform over a
// workgroup, so each takes one specialised path.
template <int D, bool R32>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(RowSide k, RowSide v, const int64_t* slots,
                                                               int64_t T, int Hkv, int64_t num_slots,
                                                               int32_t* err) {
  const RowSide& sd = (blockIdx.y == 0) ? k : v;
  switch (sd.dtype) {
    case DT_BF16: write_rows<D, R32, DT_BF16>(sd, slots, T, Hkv, num_slots, err); break;
    case DT_INT8: write_rows<D, R32, DT_INT8>(sd, slots, T, Hkv, num_slots, err); break;
    case DT_E4M3: write_rows<D, R32, DT_E4M3>(sd, slots, T, Hkv, num_slots, err); break;
    case DT_E5M2: write_rows<D, R32, DT_E5M2>(sd, slots, T, Hkv, num_slots, err); break;
    case DT_INT4: write_rows<D, R32, DT_INT4>(sd, slots, T, Hkv, num_slots, err); break;
    case DT_INT4H: write_rows<D, R32, DT_INT4H>(sd, slots, T, Hkv, num_slots, err); break;
    default: break;
  }
}

template <int D, int DT>
__device__ __forceinline__ void convert_rows(const RowSide& sd, int first_block, int n_blocks, int Hkv) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int j = threadIdx.x % LPR;
  const int64_t rows = (int64_t)n_blocks * Hkv * 16;                 // rows of the block range
  const int64_t r0 = (int64_t)blockIdx.x * RPB * kRowsPerLane + threadIdx.x / LPR;
  RowIn in[kRowsPerLane];
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t r = min(r0 + (int64_t)u * RPB, rows - 1);
    const int64_t dst = (int64_t)first_block * Hkv * 16 + r;        // same slot in source and dest
    in[u] = load_row<D, DT>(sd, sd.src + dst * D, (int)((dst / 16) % Hkv), j);
  }
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t r = r0 + (int64_t)u * RPB;
    if (r >= rows) break;                       // uniform over the row's lanes
    store_row<D, DT>(sd, in[u], (int64_t)first_block * Hkv * 16 + r, j);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void convert_kernel(RowSide k, RowSide v, int first_block, int n_blocks,
                                                           int Hkv) {
  const RowSide& sd = (blockIdx.y == 0) ? k : v;
  switch (sd.dtype) {
    case DT_BF16: convert_rows<D, DT_BF16>(sd, first_block, n_blocks, Hkv); break;
    case DT_INT8: convert_rows<D, DT_INT8>(sd, first_block, n_blocks, Hkv); break;
    case DT_E4M3: convert_rows<D, DT_E4M3>(sd, first_block, n_blocks, Hkv); break;
    case DT_E5M2: convert_rows<D, DT_E5M2>(sd, first_block, n_blocks, Hkv); break;
    case DT_INT4: convert_rows<D, DT_INT4>(sd, first_block, n_blocks, Hkv); break;
    case DT_INT4H: convert_rows<D, DT_INT4H>(sd, first_block, n_blocks, Hkv); break;
    default: break;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void hadamard_kernel(const uint16_t* x, int64_t rows, uint16_t* out) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int j = threadIdx.x % LPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  if (r >= rows) return;   // whole rows: a row's lanes leave together
  const uint4 raw = *reinterpret_cast<const uint4*>(x + r * D + 8 * j);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  hadamard_row<LPR>(v, j);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(out + r * D + 8 * j) = make_uint4(o[0], o[1], o[2], o[3]);
}

RowSide side(const CacheView& c, bool is_k, const uint16_t* src) {
  RowSide s;
  s.src = src;
  s.pages = is_k ? c.k_pages : c.v_pages;
  s.scale = is_k ? c.k_scale : c.v_scale;
  s.scale_per_head = (is_k ? c.k_gran : c.v_gran) == 1;
  s.meta = is_k ? c.k_meta : c.v_meta;
  s.dtype = is_k ? c.k_dtype : c.v_dtype;
  return s;
}

}  // namespace

hipError_t launch_cache_write(const CacheView& c, const uint16_t* k_new, const uint16_t* v_new,
                              const int64_t* slots, int64_t T, int32_t* err, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const RowSide k = side(c, true, k_new), v = side(c, false, v_new);
  const int64_t rows = T * c.num_kv_heads;
  const int64_t num_slots = (int64_t)c.num_blocks * 16;
  const bool r32 = rows <= 0x7fffffff;
  if (c.head_dim == 128) {
    constexpr int per = kThreads / 16 * kRowsPerLane;
    dim3 grid((unsigned)((rows + per - 1) / per), 2);
    if (r32)
      hipLaunchKernelGGL((cache_write_kernel<128, true>), grid, dim3(kThreads), 0, s, k, v, slots, T,
                         c.num_kv_heads, num_slots, err);
    else
      hipLaunchKernelGGL((cache_write_kernel<128, false>), grid, dim3(kThreads), 0, s, k, v, slots, T,
                         c.num_kv_heads, num_slots, err);
  } else {
    constexpr int per = kThreads / 8 * kRowsPerLane;
    dim3 grid((unsigned)((rows + per - 1) / per), 2);
    if (r32)
      hipLaunchKernelGGL((cache_write_kernel<64, true>), grid, dim3(kThreads), 0, s, k, v, slots, T,
                         c.num_kv_heads, num_slots, err);
    else
      hipLaunchKernelGGL((cache_write_kernel<64, false>), grid, dim3(kThreads), 0, s, k, v, slots, T,
                         c.num_kv_heads, num_slots, err);
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const uint16_t* x, int64_t rows, int D, uint16_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int rpb = kThreads / (D / 8);
  dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (D == 128) hipLaunchKernelGGL(hadamard_kernel<128>, grid, dim3(kThreads), 0, s, x, rows, out);
  else hipLaunchKernelGGL(hadamard_kernel<64>, grid, dim3(kThreads), 0, s, x, rows, out);
  return hipGetLastError();
}

hipError_t launch_convert(const CacheView& c, const uint16_t* k_src, const uint16_t* v_src, int first_block,
                          int n_blocks, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  const RowSide k = side(c, true, k_src), v = side(c, false, v_src);
  const int64_t rows = (int64_t)n_blocks * c.num_kv_heads * 16;
  if (c.head_dim == 128) {
    constexpr int per = kThreads / 16 * kRowsPerLane;
    dim3 grid((unsigned)((rows + per - 1) / per), 2);
    hipLaunchKernelGGL(convert_kernel<128>, grid, dim3(kThreads), 0, s, k, v, first_block, n_blocks,
                       c.num_kv_heads);
  } else {
    constexpr int per = kThreads / 8 * kRowsPerLane;
    dim3 grid((unsigned)((rows + per - 1) / per), 2);
    hipLaunchKernelGGL(convert_kernel<64>, grid, dim3(kThreads), 0, s, k, v, first_block, n_blocks,
                       c.num_kv_heads);
  }
  return hipGetLastError();
}

}  // namespace kvq
