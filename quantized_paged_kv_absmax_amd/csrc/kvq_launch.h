// kvq_launch.h — internal interface between the C ABI (kvq_api.cpp) and the
// kernel launchers.  Everything here has already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

struct CacheView {
  int k_dtype, v_dtype, k_gran, v_gran;
  int num_blocks, num_kv_heads, head_dim;
  uint8_t* k_pages;
  uint8_t* v_pages;
  const float* k_scale;
  const float* v_scale;
  float* k_meta;
  float* v_meta;
};

hipError_t launch_calibrate(const uint16_t* x, int64_t T, int Hkv, int D, int per_head, float qmax,
                            float* absmax, float* scale, hipStream_t s);

hipError_t launch_cache_write(const CacheView& c, const uint16_t* k_new, const uint16_t* v_new,
                              const int64_t* slots, int64_t T, int32_t* err, hipStream_t s);

// bf16 rows [rows][D] -> bf16 of their Hadamard transform (DT_INT4H's rotation)
hipError_t launch_hadamard(const uint16_t* x, int64_t rows, int D, uint16_t* out, hipStream_t s);

hipError_t launch_convert(const CacheView& c, const uint16_t* k_src, const uint16_t* v_src,
                          int first_block, int n_blocks, hipStream_t s);

struct DecodeArgs {
  const uint16_t* q;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  int batch, max_seq_len, num_q_heads;
  int n_q;           // query tokens per sequence (1: decode)
  float softmax_scale;
  int chunk_pages;   // pages per chunk, 0: chosen on the device from the total
  int n_chunks;      // chunks in the launch
  int min_chunk;     // smallest automatic chunk
  float* ws_m;       // [slots][n_q Hq]      (all four NULL when n_chunks == 1)
  float* ws_l;       // [slots][n_q Hq]
  float* ws_o;       // [slots][n_q Hq][D]
  int32_t* ws_rec;   // [B][2]
  int out_f32;
  void* out;
  int32_t* err;
  // one query token: the step's new token written in the same launch (rows
  // [batch][Hkv][D] bf16, slots [batch]); NULL: none
  const uint16_t* new_k = nullptr;
  const uint16_t* new_v = nullptr;
  const int64_t* new_slot = nullptr;
};

// true if the (K dtype, V dtype, head_dim) combination has a kernel
bool decode_supported(int k_dtype, int v_dtype, int head_dim);

hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t s);

}  // namespace kvq
