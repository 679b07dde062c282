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
#include "kvq_rows.h"

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
