// verify.hip — the chunk kernels with several query tokens per sequence (each
// attending causally to the cache up to its own position), for
// kvq_paged_attention_verify; a translation unit of its own so that the two
// sets of instantiations compile in parallel.
#include "decode_kernel.h"

namespace kvq {

hipError_t launch_chunk_verify(const Params& prm, int kt, int vt, int head_dim, dim3 grid, hipStream_t s) {
  return head_dim == 128 ? launch_kv<128, true>(kt, vt, prm, grid, s) : launch_kv<64, true>(kt, vt, prm, grid, s);
}

}  // namespace kvq
