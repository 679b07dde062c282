// calibrate.hip — absmax scale calibration (the sm86 INT8 summary's offline
// per-layer scaling values; per-tensor or per-attention-head groups as on the
// modelium FP8 page's scale schemes).
//
// Pass 1: grid (token chunks, KV heads).  Each lane streams 16-byte loads of its
// head's rows, keeps a running max of |x| (fmaxf drops NaN), the block reduces
// with xor shuffles and LDS, and one atomicMax on the float's bit pattern folds
// the block's maximum into absmax[group] (values are >= +0, where unsigned order
// equals float order).  The result is order-independent, hence deterministic.
// Pass 2: one small block turns absmax into scale = absmax / qmax (1.0 for 0).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const uint16_t* x, int64_t T, int Hkv, int per_head,
                                                          float* absmax) {
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPI = kThreads / LPR;     // rows (tokens) per iteration
  const int h = blockIdx.y;
  const int j = threadIdx.x % LPR;
  const int64_t t0 = (int64_t)blockIdx.x * kTokensPerBlock;
  const int64_t t1 = min(T, t0 + kTokensPerBlock);
  float m = 0.0f;
  // kUnroll rows per lane in flight at once; rows past t1 re-read row t1 - 1,
  // which leaves the maximum unchanged
  constexpr int kUnroll = 8;
  for (int64_t t = t0 + threadIdx.x / LPR; t < t1; t += kUnroll * RPI) {
    uint4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t tu = min(t + (int64_t)u * RPI, t1 - 1);
      raw[u] = *reinterpret_cast<const uint4*>(x + (tu * Hkv + h) * D + 8 * j);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xffffu)));
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
      }
    }
  }
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) b = fmaxf(b, red[i]);
    atomicMax(reinterpret_cast<unsigned int*>(absmax + (per_head ? h : 0)), __float_as_uint(b));
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
    dim3 grid((unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock), Hkv);
    if (D == 128)
      hipLaunchKernelGGL(absmax_kernel<128>, grid, dim3(kThreads), 0, s, x, T, Hkv, per_head, absmax);
    else
      hipLaunchKernelGGL(absmax_kernel<64>, grid, dim3(kThreads), 0, s, x, T, Hkv, per_head, absmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = per_head ? Hkv : 1;
  hipLaunchKernelGGL(finalize_kernel, dim3((G + 63) / 64), dim3(64), 0, s, absmax, scale, G, qmax);
  return hipGetLastError();
}

}  // namespace kvq
