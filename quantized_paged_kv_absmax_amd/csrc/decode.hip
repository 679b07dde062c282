// decode.hip — the paged-attention call: one query token per sequence (the
// chunk kernels instantiated here), or several (verify.hip), then the split-KV
// reduce.  The kernels and their design notes are in decode_kernel.h.
#include "decode_kernel.h"

namespace kvq {

bool decode_supported(int kt, int vt, int D) {
  if (D != 64 && D != 128) return false;
  if (kt == DT_INT4H) kt = DT_INT4;   // rotated keys: the same codes and kernels
  if (kt == DT_INT4 || vt == DT_INT4) return kt == DT_INT4 && vt == DT_INT4;
  const auto ok = [](int t) { return t == DT_BF16 || t == DT_INT8 || t == DT_E4M3 || t == DT_E5M2; };
  return ok(kt) && ok(vt);
}

hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  Params prm;
  prm.k_pages = c.k_pages;
  prm.v_pages = c.v_pages;
  prm.k_scale = c.k_scale;
  prm.v_scale = c.v_scale;
  prm.k_scale_per_head = c.k_gran == 1;
  prm.v_scale_per_head = c.v_gran == 1;
  prm.k_meta = c.k_meta;
  prm.v_meta = c.v_meta;
  prm.q = a.q;
  prm.block_tables = a.block_tables;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.seq_lens = a.seq_lens;
  prm.num_blocks = c.num_blocks;
  prm.Hkv = c.num_kv_heads;
  prm.Hq = a.num_q_heads;
  prm.g = a.num_q_heads / c.num_kv_heads;
  prm.max_seq_len = a.max_seq_len;
  prm.sm_log2 = a.softmax_scale * kLog2e;
  prm.batch = a.batch;
  prm.chunk_pages = a.chunk_pages;
  prm.n_chunks = a.n_chunks;
  prm.min_chunk = a.min_chunk;
  prm.n_q = a.n_q;
  prm.n_tiles = (a.n_q * prm.g + 15) / 16;
  prm.q_slot = (std::min(16, a.n_q * prm.g) * c.head_dim * 2 + 1023) / 1024 * 1024;
  prm.wg_waves = std::min(prm.n_tiles, 4);              // several query tokens: tiles sharing a workgroup
  prm.ws_m = a.ws_m;
  prm.ws_l = a.ws_l;
  prm.ws_o = a.ws_o;
  prm.ws_rec = reinterpret_cast<int2*>(a.ws_rec);
  prm.out_f32 = a.out_f32;
  prm.out = a.out;
  prm.err = a.err;
  prm.new_k = a.n_q == 1 ? a.new_k : nullptr;
  prm.new_v = a.n_q == 1 ? a.new_v : nullptr;
  prm.new_slot = a.n_q == 1 ? a.new_slot : nullptr;

  const int groups = (prm.n_tiles + prm.wg_waves - 1) / prm.wg_waves;   // workgroups per (chunk, KV head)
  dim3 grid(a.n_chunks * groups, c.num_kv_heads);
  hipError_t e;
  const int kt = c.k_dtype;
  if (a.n_q > 1) e = launch_chunk_verify(prm, kt, c.v_dtype, c.head_dim, grid, s);
  else e = (c.head_dim == 128) ? launch_kv<128, false>(kt, c.v_dtype, prm, grid, s)
                               : launch_kv<64, false>(kt, c.v_dtype, prm, grid, s);
  if (e != hipSuccess || a.ws_rec == nullptr) return e;
  // many rows with few pieces each (several query tokens, a large batch): a lane
  // group per row; else a workgroup per row, its groups splitting the pieces
  const int64_t rows = (int64_t)a.num_q_heads * a.n_q;
  const bool by_rows = rows * a.batch >= 8192 && a.n_chunks <= 3 * a.batch;
  if (by_rows) {
    const int per_block = kRedThreads / (c.head_dim / 4);
    dim3 rgrid((unsigned)((rows + per_block - 1) / per_block), a.batch);
    if (c.head_dim == 128)
      hipLaunchKernelGGL(decode_reduce_rows_kernel<128>, rgrid, dim3(kRedThreads), 0, s, prm);
    else
      hipLaunchKernelGGL(decode_reduce_rows_kernel<64>, rgrid, dim3(kRedThreads), 0, s, prm);
  } else {
    dim3 rgrid((unsigned)rows, a.batch);
    if (c.head_dim == 128)
      hipLaunchKernelGGL(decode_reduce_kernel<128>, rgrid, dim3(kRedThreads), 0, s, prm);
    else
      hipLaunchKernelGGL(decode_reduce_kernel<64>, rgrid, dim3(kRedThreads), 0, s, prm);
  }
  return hipGetLastError();
}

}  // namespace kvq
