// calibrate.hip — absmax scale calibration (the sm86 INT8 summary's offline
// per-layer scaling values; per-tensor or per-attention-head groups as on the
// modelium FP8 page's scale schemes).
//
// Pass 1: each workgroup streams contiguous 16-byte pieces of x ([T][Hkv][D],
// all heads at once, kUnroll pieces per lane in flight) and keeps a running
// max of |x| (fmaxf drops NaN).  For per-KV-head groups the D/8 lanes of one row
// segment share its head: they combine by DPP moves, and one lane folds the
// row's maximum into an LDS slot per head (an LDS atomic max on the bit
// pattern; values are >= +0, where unsigned order equals float order).  At the
// end each head's (or the tensor's) maximum goes to absmax[group] with one
// global atomic max per workgroup and group.  The result is order-independent,
// hence deterministic.
// Pass 2: one small block turns absmax into scale = absmax / qmax (1.0 for 0).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                  // 16-byte pieces per lane in flight
constexpr int kMaxHeadsLds = 4096;          // per-head maxima kept in LDS

__device__ __forceinline__ float abs_max8(uint4 raw, float m) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
  }
  return m;
}

// max over aligned groups of G lanes (G = 8 or 16), by DPP moves
template <int G>
__device__ __forceinline__ float group_max(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  if constexpr (G == 16) v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));   // row_mirror
  return v;
}

// PER_HEAD: one maximum per KV head (Hkv <= kMaxHeadsLds), else one for the tensor
template <int D, bool PER_HEAD>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const uint16_t* x, int64_t n_pieces, int Hkv,
                                                          int64_t pieces_per_block, float* absmax) {
  constexpr int LPR = D / 8;                 // pieces (lanes) per row segment
  __shared__ unsigned int smax[PER_HEAD ? kMaxHeadsLds : kThreads / 64];
  const int tid = threadIdx.x;
  if constexpr (PER_HEAD) {
    for (int h = tid; h < Hkv; h += kThreads) smax[h] = 0u;
    __syncthreads();
  }
  const uint4* src = reinterpret_cast<const uint4*>(x);
  const int64_t p0 = (int64_t)blockIdx.x * pieces_per_block;
  const int64_t p1 = min(n_pieces, p0 + pieces_per_block);
  float m = 0.0f;
  for (int64_t base = p0; base < p1; base += (int64_t)kUnroll * kThreads) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // pieces past p1 re-read piece p1 - 1 of the same row slot: the maximum
      // of its group is unchanged, since a lane's row segment stays the same
      const int64_t i = base + (int64_t)u * kThreads + tid;
      raw[u] = src[i < p1 ? i : p1 - 1];
    }
    if constexpr (!PER_HEAD) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) m = abs_max8(raw[u], m);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        float r = group_max<LPR>(abs_max8(raw[u], 0.0f));
        // lane 0 of the row segment: its head is (row index) mod Hkv; rows are
        // aligned to LPR lanes because every block starts on a row boundary
        if ((tid % LPR) == 0 && i < p1) {
          const int h = (int)((i / LPR) % Hkv);
          atomicMax(&smax[h], __float_as_uint(r));
        }
      }
    }
  }
  if constexpr (!PER_HEAD) {
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
    if ((tid & 63) == 0) smax[tid >> 6] = __float_as_uint(m);
    __syncthreads();
    if (tid == 0) {
      unsigned int b = smax[0];
#pragma unroll
      for (int i = 1; i < kThreads / 64; ++i) b = max(b, smax[i]);
      atomicMax(reinterpret_cast<unsigned int*>(absmax), b);
    }
  } else {
    __syncthreads();
    for (int h = tid; h < Hkv; h += kThreads)
      if (smax[h]) atomicMax(reinterpret_cast<unsigned int*>(absmax + h), smax[h]);
  }
}

// per-KV-head calibration with more heads than the LDS table holds: one
// workgroup per (token chunk, head), each reading its head's rows
template <int D>
__global__ __launch_bounds__(kThreads) void absmax_head_rows_kernel(const uint16_t* x, int64_t T, int Hkv,
                                                                    float* absmax) {
  constexpr int LPR = D / 8;
  constexpr int RPI = kThreads / LPR;
  const int h = blockIdx.y;
  const int j = threadIdx.x % LPR;
  const int64_t t0 = (int64_t)blockIdx.x * 256;
  const int64_t t1 = min(T, t0 + 256);
  float m = 0.0f;
  for (int64_t t = t0 + threadIdx.x / LPR; t < t1; t += RPI)
    m = abs_max8(*reinterpret_cast<const uint4*>(x + (t * Hkv + h) * D + 8 * j), m);
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) b = fmaxf(b, red[i]);
    atomicMax(reinterpret_cast<unsigned int*>(absmax + h), __float_as_uint(b));
  }
}

__global__ void finalize_kernel(const float* absmax, float* scale, int G, float qmax) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  const float a = absmax[g];
  scale[g] = (a == 0.0f) ? 1.0f : a / qmax;
}

}  // namespace

hipError_t launch_calibrate(const uint16_t* x, int64_t T, int Hkv, int D, int per_head, float qmax,
                            float* absmax, float* scale, hipStream_t s) {
  if (T > 0) {
    if (per_head && Hkv > kMaxHeadsLds) {
      dim3 grid((unsigned)((T + 255) / 256), Hkv);
      if (D == 128) hipLaunchKernelGGL(absmax_head_rows_kernel<128>, grid, dim3(kThreads), 0, s, x, T, Hkv, absmax);
      else hipLaunchKernelGGL(absmax_head_rows_kernel<64>, grid, dim3(kThreads), 0, s, x, T, Hkv, absmax);
    } else {
      // about 1024 workgroups (four per compute unit), each a whole number of rows
      const int64_t lpr = D / 8;
      const int64_t n_pieces = T * Hkv * lpr;
      const int64_t step = (int64_t)kUnroll * kThreads;                  // pieces per pass of a workgroup
      int64_t per = (n_pieces + 1023) / 1024;
      per = (per + step - 1) / step * step;                               // whole passes: a multiple of lpr
      const unsigned blocks = (unsigned)((n_pieces + per - 1) / per);
      if (D == 128) {
        if (per_head) hipLaunchKernelGGL((absmax_kernel<128, true>), dim3(blocks), dim3(kThreads), 0, s, x, n_pieces, Hkv, per, absmax);
        else hipLaunchKernelGGL((absmax_kernel<128, false>), dim3(blocks), dim3(kThreads), 0, s, x, n_pieces, Hkv, per, absmax);
      } else {
        if (per_head) hipLaunchKernelGGL((absmax_kernel<64, true>), dim3(blocks), dim3(kThreads), 0, s, x, n_pieces, Hkv, per, absmax);
        else hipLaunchKernelGGL((absmax_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, s, x, n_pieces, Hkv, per, absmax);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = per_head ? Hkv : 1;
  hipLaunchKernelGGL(finalize_kernel, dim3((G + 63) / 64), dim3(64), 0, s, absmax, scale, G, qmax);
  return hipGetLastError();
}

}  // namespace kvq
