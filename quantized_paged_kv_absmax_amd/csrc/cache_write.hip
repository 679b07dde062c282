// cache_write.hip — fused quantise-and-scatter of K/V rows into the paged cache
// (vLLM issue 4025, methods item 2) and conversion of an existing bf16 paged
// cache (methods item 1).
//
// One row = head_dim bf16 values of one (token, KV head).  A row is handled by
// D/8 consecutive lanes, each loading 16 bytes (8 values) and storing 8 codes
// (8 bytes; 4 bytes for INT4).  INT4 finds the row's min / max with xor
// shuffles inside the lane group, and the group's first lane stores the
// (scale, zero point) pair.  Blocks in y = 0 encode K, y = 1 encode V, so a
// launch streams both tensors; the element format is a per-launch switch that
// is uniform across the grid.
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

// Encode the 8 values this lane holds (x[0..7], elements [8*j, 8*j+8) of the row)
// and store them into the destination row.
template <int D, int LPR>
__device__ __forceinline__ void encode_store(const float (&x)[8], int dtype, float s,
                                             uint8_t* dst_row, float* meta_row, int j) {
  if (dtype == DT_BF16) {
    // unreachable: bf16 rows are copied by the caller
    return;
  }
  if (dtype == DT_INT4) {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
    static_assert(LPR == 8 || LPR == 16, "lanes per row");
    // over the LPR lanes of the row (8 or 16, aligned): within quads, then
    // half-rows (lane i with 7 - i), then rows (i with 15 - i), by DPP moves
    // rather than LDS permutes
    auto dpp = [](float v, auto ctrl) {
      return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, false));
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
    float sc = (mx - mn) / 15.0f;
    if (sc == 0.0f || !(fabsf(sc) <= 3.402823466e38f)) sc = (mn != 0.0f) ? fabsf(mn) : 1.0f;
    const float zp = rintf(-mn / sc);
    const Quot qt(sc);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = rintf(qt(x[i])) + zp;
      q = fminf(fmaxf(q, 0.0f), 15.0f);
      packed |= ((uint32_t)q) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(dst_row + 4 * j) = packed;
    if (j == 0) *reinterpret_cast<float2*>(meta_row) = make_float2(sc, zp);
    return;
  }
  const Quot qt(s);
  float t[2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i / 4][i % 4] = qt(x[i]);
  uint32_t lo = 0, hi = 0;
  if (dtype == DT_INT8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= enc_int8(t[0][i]) << (8 * i);
      hi |= enc_int8(t[1][i]) << (8 * i);
    }
  } else if (dtype == DT_E4M3) {
    lo = enc_fp8x4<DT_E4M3>(t[0]);
    hi = enc_fp8x4<DT_E4M3>(t[1]);
  } else {
    lo = enc_fp8x4<DT_E5M2>(t[0]);
    hi = enc_fp8x4<DT_E5M2>(t[1]);
  }
  *reinterpret_cast<uint2*>(dst_row + 8 * j) = make_uint2(lo, hi);
}

// bf16 bits of a float64 value, rounded once to nearest even.  The value is
// first narrowed to float32 toward zero with inexactness marked in the last bit
// (round to odd): float32 keeps 16 bits beyond bf16's 8 at every magnitude,
// subnormals included, so rounding that to nearest even gives the direct
// rounding of the float64 value (a round-to-odd intermediate with at least two
// extra bits makes the second rounding innocuous).  Past the bf16 range the
// odd float32 maximum rounds on to infinity, as the direct rounding does.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  const float f = __double2float_rz(v);
  uint32_t u = __float_as_uint(f);
  if ((double)f != v && v == v) u |= 1u;
  return f32_to_bf16_bits(__uint_as_float(u));
}

// The unnormalised Walsh-Hadamard transform of a row held by LPR aligned lanes,
// 8 values each (x[i] = element 8 j + i): y = H x with H[i][k] =
// (-1)^popcount(i & k), by the butterfly (stages h = 1, 2, 4 inside the lane,
// then h = 8 .. D/2 between lanes j and j ^ (h / 8); the pair at (i, i + h)
// becomes (a + b, a - b)) in float64, where every sum is exact while the row's
// magnitudes span less than 2^38 (bf16 values carry 8 significant bits; D <=
// 128 terms add 7 more), then rounded once to bf16 (returned as float32).  An
// exact zero comes out as +0.
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
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    const bool upper = j & m;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double other = __shfl_xor(y[i], m, 64);
      y[i] = upper ? other - y[i] : y[i] + other;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = bf16_bits_to_f32(f64_to_bf16_rne(y[i] + 0.0));
}

// this lane's 16 source bytes of a row, and the row's scale
struct RowIn {
  uint4 raw;
  float s;
};

template <int D>
__device__ __forceinline__ RowIn load_row(const RowSide& sd, const uint16_t* src_row, int h, int j) {
  RowIn in;
  in.raw = *reinterpret_cast<const uint4*>(src_row + 8 * j);
  in.s = sd.scale ? sd.scale[sd.scale_per_head ? h : 0] : 1.0f;
  return in;
}

template <int D>
__device__ __forceinline__ void store_row(const RowSide& sd, const RowIn& in, int64_t dst_row_idx, int j) {
  constexpr int LPR = D / 8;
  const uint4 raw = in.raw;
  if (sd.dtype == DT_BF16) {
    *reinterpret_cast<uint4*>(sd.pages + dst_row_idx * (2 * D) + 16 * j) = raw;
    return;
  }
  float x[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
  int dt = sd.dtype;
  if (dt == DT_INT4H) {   // uniform per launch side: every lane of the row takes it
    hadamard_row<LPR>(x, j);
    dt = DT_INT4;
  }
  const int rb = (dt == DT_INT4) ? D / 2 : D;
  encode_store<D, LPR>(x, dt, in.s, sd.pages + dst_row_idx * rb,
                       sd.meta ? sd.meta + dst_row_idx * 2 : nullptr, j);
}

// Each lane takes kRowsPerLane rows (kRowsPerLane x 16 bytes in flight before any
// encode); the rows of one pass are consecutive, the passes of a workgroup too.
constexpr int kRowsPerLane = 4;

// R32: the row count fits 31 bits, so (token, head) come from a 32-bit division
template <int D, bool R32>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(RowSide k, RowSide v, const int64_t* slots,
                                                               int64_t T, int Hkv, int64_t num_slots,
                                                               int32_t* err) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;  // rows per pass
  const RowSide& sd = (blockIdx.y == 0) ? k : v;
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
    in[u] = load_row<D>(sd, sd.src + rr * D, h, j);
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
    store_row<D>(sd, in[u], (blk * Hkv + hh[u]) * 16 + off, j);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void convert_kernel(RowSide k, RowSide v, int first_block, int n_blocks,
                                                           int Hkv) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const RowSide& sd = (blockIdx.y == 0) ? k : v;
  const int j = threadIdx.x % LPR;
  const int64_t rows = (int64_t)n_blocks * Hkv * 16;                 // rows of the block range
  const int64_t r0 = (int64_t)blockIdx.x * RPB * kRowsPerLane + threadIdx.x / LPR;
  RowIn in[kRowsPerLane];
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t r = min(r0 + (int64_t)u * RPB, rows - 1);
    const int64_t dst = (int64_t)first_block * Hkv * 16 + r;        // same slot in source and dest
    in[u] = load_row<D>(sd, sd.src + dst * D, (int)((dst / 16) % Hkv), j);
  }
#pragma unroll
  for (int u = 0; u < kRowsPerLane; ++u) {
    const int64_t r = r0 + (int64_t)u * RPB;
    if (r >= rows) break;                       // uniform over the row's lanes
    store_row<D>(sd, in[u], (int64_t)first_block * Hkv * 16 + r, j);
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
