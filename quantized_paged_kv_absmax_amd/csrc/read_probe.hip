// read_probe.hip — a measurement aid, not part of the C ABI of libkvq.so: it reads
// the pages a decode call reads (the K and V page, and INT4 metadata, of every
// (page, KV head) of every sequence), in the decode's chunks, and computes
// nothing with them.  bench.py times it beside the decode, so the decode's rate
// can be set against what a read of the same pages reaches in one launch.
// Built into its own library, lib/libkvq_probe.so.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kInFlight = 2;   // pages per wave in flight (K and V each)
constexpr int kMaxChunks = 4;  // 16-byte chunks per lane and page side: pages up to 4 KB

// one 64-lane wave per (chunk, KV head): chunk c covers entries [c C, c C + C) of
// the page list (block ids in the decode's order: sequence by sequence, page by page)
__global__ __launch_bounds__(64) void read_pages_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                        const uint4* __restrict__ km, const uint4* __restrict__ vm,
                                                        const int32_t* __restrict__ list, int64_t n, int hkv,
                                                        int page16, int64_t C, int num_blocks, uint32_t* sink) {
  const int64_t x0 = (int64_t)blockIdx.x * C, x1 = min(x0 + C, n);
  const int h = blockIdx.y, lane = threadIdx.x;
  uint32_t acc = 0;
  for (int64_t x = x0; x < x1; x += kInFlight) {
    uint4 r[kInFlight][2][kMaxChunks];
    uint4 m[kInFlight][2];
#pragma unroll
    for (int p = 0; p < kInFlight; ++p) {
      const int64_t xx = min(x + p, x1 - 1);
      const int bid = min(max(list[xx], 0), num_blocks - 1);
      const size_t page = (size_t)bid * hkv + h;
#pragma unroll
      for (int j = 0; j < kMaxChunks; ++j) {
        r[p][0][j] = r[p][1][j] = make_uint4(0, 0, 0, 0);
        if (64 * j < page16) {                 // uniform: the page has this pass
          const int c = min(lane + 64 * j, page16 - 1);   // (pages under 1 KB: lanes past it reread its last chunk)
          r[p][0][j] = k[page * page16 + c];
          r[p][1][j] = v[page * page16 + c];
        }
      }
      // INT4 metadata: 16 (scale, zero point) pairs of 8 bytes, 128 bytes a page
      // (every lane reads inside the page's 128 bytes; lanes past 8 reread its last chunk)
      m[p][0] = m[p][1] = make_uint4(0, 0, 0, 0);
      if (km) m[p][0] = km[page * 8 + min(lane, 7)];
      if (vm) m[p][1] = vm[page * 8 + min(lane, 7)];
    }
#pragma unroll
    for (int p = 0; p < kInFlight; ++p) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int j = 0; j < kMaxChunks; ++j) acc ^= r[p][s][j].x ^ r[p][s][j].y ^ r[p][s][j].z ^ r[p][s][j].w;
        acc ^= m[p][s].x ^ m[p][s].y ^ m[p][s].z ^ m[p][s].w;
      }
    }
  }
  // a store the compiler cannot prove dead keeps every load
  if (acc == 0x9e3779b9u) sink[blockIdx.x * hkv + h] = acc;
}

}  // namespace

// Reads the pages listed in `block_list` (n_pages block ids, each clamped into
// [0, num_blocks)) for every KV head: K and V pages of page_bytes (16 to 4096, a
// multiple of 16) at [num_blocks][hkv][page_bytes], and, when given, INT4
// metadata of 128 bytes a (block, head).  n_chunks waves per KV head, each a
// contiguous run of the list.  sink: n_chunks * hkv words, written only when a
// wave's checksum hits a fixed value.  Returns the launch's hipError_t.
extern "C" int kvq_probe_read_pages(const void* k_pages, const void* v_pages, const void* k_meta,
                                    const void* v_meta, const int32_t* block_list, int64_t n_pages, int32_t hkv,
                                    int32_t page_bytes, int32_t n_chunks, int32_t num_blocks, uint32_t* sink,
                                    hipStream_t stream) {
  if (!k_pages || !v_pages || !block_list || !sink) return (int)hipErrorInvalidValue;
  if (n_pages <= 0 || hkv <= 0 || n_chunks <= 0 || num_blocks <= 0) return (int)hipErrorInvalidValue;
  if (page_bytes < 16 || page_bytes > 64 * 16 * kMaxChunks || page_bytes % 16) return (int)hipErrorInvalidValue;
  const int64_t C = (n_pages + n_chunks - 1) / n_chunks;
  const int64_t chunks = (n_pages + C - 1) / C;
  hipLaunchKernelGGL(read_pages_kernel, dim3((unsigned)chunks, (unsigned)hkv), dim3(64), 0, stream,
                     static_cast<const uint4*>(k_pages), static_cast<const uint4*>(v_pages),
                     static_cast<const uint4*>(k_meta), static_cast<const uint4*>(v_meta), block_list, n_pages, hkv,
                     page_bytes / 16, C, num_blocks, sink);
  return (int)hipGetLastError();
}
