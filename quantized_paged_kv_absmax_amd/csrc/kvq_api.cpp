// kvq_api.cpp — the C ABI of libkvq (declared in include/kvq.h): host-side
// argument checks, launch geometry and dispatch to the HIP kernels.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and touches no device state (and can be exercised without a GPU).
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_launch.h"

// Decode workspace for kvq_paged_attention_decode_noalloc: one array per GPU,
// zero at load and held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address reaches kernels.
static __device__ __align__(256) uint8_t scratch[KVQ_DECODE_SCRATCH_BYTES];

namespace {

// Decode work split: the pages of all sequences, concatenated in sequence order,
// are cut into chunks; one wave per (chunk, KV head).  Without an explicit
// partition the chunk count aims at kTargetWaves waves (256 compute units with
// 8 resident decode waves each) and the device sizes the chunks from the actual
// page total, never below kMinChunk pages.
constexpr int64_t kTargetWaves = 2048;
constexpr int kMinChunk = 4;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_store_dtype(int32_t d) {
  return d == KVQ_BF16 || d == KVQ_INT8 || d == KVQ_FP8_E4M3 || d == KVQ_FP8_E5M2 || d == KVQ_INT4_ASYM ||
         d == KVQ_INT4_HAD;
}

// Checks shared by every call that takes a cache.
kvq_status check_cache(const kvq_cache* c) {
  if (!c) return KVQ_ERR_NULL;
  if (!valid_store_dtype(c->k_dtype) || !valid_store_dtype(c->v_dtype)) return KVQ_ERR_UNSUPPORTED;
  if (c->v_dtype == KVQ_INT4_HAD) return KVQ_ERR_UNSUPPORTED;   // rotated rows are keys only
  if (c->head_dim != 64 && c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (c->block_size != 16) return KVQ_ERR_UNSUPPORTED;
  if (c->num_kv_heads < 1 || c->num_blocks < 0) return KVQ_ERR_SHAPE;
  if (!c->k_pages || !c->v_pages) return KVQ_ERR_NULL;
  if (!aligned16(c->k_pages) || !aligned16(c->v_pages)) return KVQ_ERR_ALIGN;
  const int32_t dts[2] = {c->k_dtype, c->v_dtype};
  const int32_t grs[2] = {c->k_gran, c->v_gran};
  const float* scales[2] = {c->k_scale, c->v_scale};
  const float* metas[2] = {c->k_meta, c->v_meta};
  for (int i = 0; i < 2; ++i) {
    if (dts[i] == KVQ_INT4_ASYM || dts[i] == KVQ_INT4_HAD) {
      if (grs[i] != KVQ_PER_TOKEN_HEAD) return KVQ_ERR_UNSUPPORTED;
      if (!metas[i]) return KVQ_ERR_NULL;
      if (!aligned16(metas[i])) return KVQ_ERR_ALIGN;
    } else if (dts[i] != KVQ_BF16) {
      if (grs[i] != KVQ_PER_TENSOR && grs[i] != KVQ_PER_KV_HEAD) return KVQ_ERR_UNSUPPORTED;
      (void)scales;  // NULL scale means 1.0
    }
  }
  return KVQ_OK;
}

kvq::CacheView view(const kvq_cache* c) {
  kvq::CacheView v;
  v.k_dtype = c->k_dtype;
  v.v_dtype = c->v_dtype;
  v.k_gran = c->k_gran;
  v.v_gran = c->v_gran;
  v.num_blocks = c->num_blocks;
  v.num_kv_heads = c->num_kv_heads;
  v.head_dim = c->head_dim;
  v.k_pages = static_cast<uint8_t*>(c->k_pages);
  v.v_pages = static_cast<uint8_t*>(c->v_pages);
  v.k_scale = (c->k_dtype == KVQ_BF16 || c->k_dtype == KVQ_INT4_ASYM || c->k_dtype == KVQ_INT4_HAD) ? nullptr
                                                                                                   : c->k_scale;
  v.v_scale = c->v_dtype == KVQ_BF16 || c->v_dtype == KVQ_INT4_ASYM ? nullptr : c->v_scale;
  v.k_meta = c->k_meta;
  v.v_meta = c->v_meta;
  return v;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

struct Split {
  int64_t n_chunks;
  int chunk_pages;   // 0: automatic
};

// n_tiles: waves per (chunk, KV head), one per 16 (query token, head) rows
Split decode_split(int64_t batch, int64_t num_kv_heads, int64_t max_seq_len, int32_t partition,
                   int64_t n_tiles = 1) {
  const int64_t bound = batch * ((max_seq_len + 15) / 16);   // pages, at most
  Split sp;
  if (partition > 0) {
    sp.chunk_pages = partition / 16;
    sp.n_chunks = (bound + sp.chunk_pages - 1) / sp.chunk_pages;
  } else {
    sp.chunk_pages = 0;
    const int64_t target = (kTargetWaves + num_kv_heads * n_tiles - 1) / (num_kv_heads * n_tiles);
    const int64_t most = (bound + kMinChunk - 1) / kMinChunk;
    sp.n_chunks = target < most ? target : most;
  }
  if (sp.n_chunks < 1) sp.n_chunks = 1;
  return sp;
}

// Decode workspace, with S = n_chunks + batch piece slots and R = n_q * Hq rows
// per slot: [m f32 [S][R]] [l f32 [S][R]] [rec int32 [batch][2]] [acc f32 [S][R][D]],
// each region starting on a 16-byte boundary; none when there is one chunk.
struct WsLayout {
  int64_t m, l, rec, o, total;
};

int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

WsLayout workspace_layout(int64_t batch, int64_t num_q_heads, int64_t head_dim, int64_t n_chunks) {
  WsLayout w;
  const int64_t rows = (n_chunks + batch) * num_q_heads;
  w.m = 0;
  w.l = w.m + round16(rows * 4);
  w.rec = w.l + round16(rows * 4);
  w.o = w.rec + round16(batch * 8);
  w.total = w.o + rows * head_dim * 4;
  return w;
}

}  // namespace

extern "C" {

kvq_status kvq_calibrate_scales(const uint16_t* x, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                int32_t granularity, int32_t target_dtype, float* absmax_inout, float* scale_out,
                                void* stream) {
  if (!absmax_inout || !scale_out) return KVQ_ERR_NULL;
  if (num_tokens < 0 || num_kv_heads < 1) return KVQ_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (granularity != KVQ_PER_TENSOR && granularity != KVQ_PER_KV_HEAD) return KVQ_ERR_UNSUPPORTED;
  float qmax;
  switch (target_dtype) {
    case KVQ_INT8: qmax = 127.0f; break;
    case KVQ_FP8_E4M3: qmax = 448.0f; break;
    case KVQ_FP8_E5M2: qmax = 57344.0f; break;
    default: return KVQ_ERR_UNSUPPORTED;
  }
  if (num_tokens > 0) {
    if (!x) return KVQ_ERR_NULL;
    if (!aligned16(x)) return KVQ_ERR_ALIGN;
    if (num_tokens > (int64_t)INT32_MAX * 256) return KVQ_ERR_SHAPE;
  }
  return from_hip(kvq::launch_calibrate(x, num_tokens, num_kv_heads, head_dim, granularity == KVQ_PER_KV_HEAD,
                                        qmax, absmax_inout, scale_out, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_cache_write(const kvq_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t* err_count, void* stream) {
  const kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_tokens < 0) return KVQ_ERR_SHAPE;
  if (num_tokens == 0) return KVQ_OK;
  if (!k_new || !v_new || !slot_mapping) return KVQ_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_ALIGN;
  const int64_t rows = num_tokens * cache->num_kv_heads;
  const int64_t rows_per_block = 256 / (cache->head_dim / 8);
  if ((rows + rows_per_block - 1) / rows_per_block > INT32_MAX) return KVQ_ERR_SHAPE;
  return from_hip(kvq::launch_cache_write(view(cache), k_new, v_new, slot_mapping, num_tokens, err_count,
                                          static_cast<hipStream_t>(stream)));
}

kvq_status kvq_convert_cache(const kvq_cache* dst, const uint16_t* k_src, const uint16_t* v_src,
                             int32_t first_block, int32_t num_blocks, void* stream) {
  const kvq_status st = check_cache(dst);
  if (st != KVQ_OK) return st;
  if (first_block < 0 || num_blocks < 0 || (int64_t)first_block + num_blocks > dst->num_blocks) return KVQ_ERR_SHAPE;
  if (num_blocks == 0) return KVQ_OK;
  if (!k_src || !v_src) return KVQ_ERR_NULL;
  if (!aligned16(k_src) || !aligned16(v_src)) return KVQ_ERR_ALIGN;
  return from_hip(kvq::launch_convert(view(dst), k_src, v_src, first_block, num_blocks,
                                      static_cast<hipStream_t>(stream)));
}

size_t kvq_verify_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t partition) {
  if (batch <= 0 || n_q <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len <= 0) return 0;
  if (partition < 0 || partition % 16 != 0) return 0;
  if (num_q_heads % num_kv_heads != 0 || (int64_t)n_q * num_q_heads > 65535) return 0;
  const int64_t n_tiles = ((int64_t)n_q * (num_q_heads / num_kv_heads) + 15) / 16;
  const Split sp = decode_split(batch, num_kv_heads, max_seq_len, partition, n_tiles);
  if (sp.n_chunks <= 1) return 0;
  return workspace_layout(batch, (int64_t)n_q * num_q_heads, head_dim, sp.n_chunks).total;
}

size_t kvq_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition) {
  return kvq_verify_workspace_size(batch, 1, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition);
}

kvq_status kvq_paged_attention_decode(const kvq_cache* cache, const uint16_t* q, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                      int32_t max_seq_len, int32_t num_q_heads, float softmax_scale,
                                      int32_t partition, void* workspace, size_t workspace_bytes,
                                      int32_t out_dtype, void* out, int32_t* err_count, void* stream) {
  return kvq_paged_attention_verify(cache, q, 1, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                                    num_q_heads, softmax_scale, partition, workspace, workspace_bytes, out_dtype,
                                    out, err_count, stream);
}

}  // extern "C"

namespace {

// the device address of this GPU's `scratch` array, looked up on the first call
// on each device (with that device current) and kept
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kvq_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

// decode / verify; with use_scratch the workspace is this GPU's scratch array
// (workspace and workspace_bytes are then ignored)
kvq_status attention_impl(const kvq_cache* cache, const uint16_t* q, int32_t n_q, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                          int32_t num_q_heads, float softmax_scale, int32_t partition, void* workspace,
                          size_t workspace_bytes, int32_t out_dtype, void* out, int32_t* err_count, void* stream,
                          bool use_scratch, const uint16_t* new_k = nullptr, const uint16_t* new_v = nullptr,
                          const int64_t* new_slot = nullptr, bool check_only = false) {
  const kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!kvq::decode_supported(cache->k_dtype, cache->v_dtype, cache->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32) return KVQ_ERR_UNSUPPORTED;
  if (batch < 0 || max_seq_len < 0 || max_blocks_per_seq < 0) return KVQ_ERR_SHAPE;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0) return KVQ_ERR_SHAPE;
  if (num_q_heads / cache->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
  if (partition < 0 || partition % 16 != 0) return KVQ_ERR_SHAPE;
  if (n_q < 1 || (int64_t)n_q * num_q_heads > 65535) return KVQ_ERR_SHAPE;
  if (batch == 0) return KVQ_OK;
  if (!q || !block_tables || !seq_lens || !out) return KVQ_ERR_NULL;
  if (!aligned16(q)) return KVQ_ERR_ALIGN;
  if (batch > 65535 || cache->num_kv_heads > 65535) return KVQ_ERR_SHAPE;
  if ((int64_t)batch * (((int64_t)max_seq_len + 15) / 16) > INT32_MAX / 2) return KVQ_ERR_SHAPE;
  const int64_t n_tiles = ((int64_t)n_q * (num_q_heads / cache->num_kv_heads) + 15) / 16;
  const Split sp = decode_split(batch, cache->num_kv_heads, max_seq_len, partition, n_tiles);
  if (sp.n_chunks * n_tiles > INT32_MAX / 2) return KVQ_ERR_SHAPE;
  // the query block of one sequence (n_q * Hq rows) is addressed with 32-bit offsets
  if ((int64_t)n_q * num_q_heads * cache->head_dim * 2 > INT32_MAX / 2) return KVQ_ERR_SHAPE;
  kvq::DecodeArgs a;
  a.q = q;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.num_q_heads = num_q_heads;
  a.n_q = n_q;
  a.softmax_scale = softmax_scale;
  a.chunk_pages = sp.chunk_pages;
  a.n_chunks = (int)sp.n_chunks;
  a.min_chunk = kMinChunk;
  a.ws_m = a.ws_l = a.ws_o = nullptr;
  a.ws_rec = nullptr;
  if (sp.n_chunks > 1) {
    const WsLayout lay = workspace_layout(batch, (int64_t)n_q * num_q_heads, cache->head_dim, sp.n_chunks);
    if (use_scratch) {
      if ((size_t)lay.total > (size_t)KVQ_DECODE_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
      const kvq_status ss = scratch_of_current_device(&workspace);
      if (ss != KVQ_OK) return ss;
      workspace_bytes = KVQ_DECODE_SCRATCH_BYTES;
    }
    if (!workspace) return KVQ_ERR_WORKSPACE;
    if (workspace_bytes < (size_t)lay.total) return KVQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
    char* base = static_cast<char*>(workspace);
    a.ws_m = reinterpret_cast<float*>(base + lay.m);
    a.ws_l = reinterpret_cast<float*>(base + lay.l);
    a.ws_rec = reinterpret_cast<int32_t*>(base + lay.rec);
    a.ws_o = reinterpret_cast<float*>(base + lay.o);
  }
  if (check_only) return KVQ_OK;
  a.out_f32 = out_dtype == KVQ_F32;
  a.out = out;
  a.err = err_count;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slot = new_slot;
  return from_hip(kvq::launch_decode(view(cache), a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

kvq_status kvq_paged_attention_verify(const kvq_cache* cache, const uint16_t* q, int32_t n_q,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                      int32_t num_q_heads, float softmax_scale, int32_t partition, void* workspace,
                                      size_t workspace_bytes, int32_t out_dtype, void* out, int32_t* err_count,
                                      void* stream) {
  return attention_impl(cache, q, n_q, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len, num_q_heads,
                        softmax_scale, partition, workspace, workspace_bytes, out_dtype, out, err_count, stream,
                        false);
}

kvq_status kvq_paged_attention_decode_write(const kvq_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                                            const int64_t* slot_mapping, const uint16_t* q,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                            int32_t num_q_heads, float softmax_scale, int32_t partition,
                                            void* workspace, size_t workspace_bytes, int32_t out_dtype, void* out,
                                            int32_t* err_count, void* stream) {
  const kvq_status st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (batch > 0 && (!k_new || !v_new || !slot_mapping)) return KVQ_ERR_NULL;
  if (batch > 0 && (!aligned16(k_new) || !aligned16(v_new))) return KVQ_ERR_ALIGN;
  // every check of the attention first, so that an invalid call enqueues nothing
  const kvq_status sa = attention_impl(cache, q, 1, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len,
                                       num_q_heads, softmax_scale, partition, workspace, workspace_bytes, out_dtype,
                                       out, err_count, stream, false, nullptr, nullptr, nullptr, true);
  if (sa != KVQ_OK || batch == 0) return sa;
  return attention_impl(cache, q, 1, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len, num_q_heads,
                        softmax_scale, partition, workspace, workspace_bytes, out_dtype, out, err_count, stream, false,
                        k_new, v_new, slot_mapping);
}

kvq_status kvq_paged_attention_decode_noalloc(const kvq_cache* cache, const uint16_t* q,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                              int32_t num_q_heads, float softmax_scale, int32_t partition,
                                              int32_t out_dtype, void* out, int32_t* err_count, void* stream) {
  return attention_impl(cache, q, 1, block_tables, max_blocks_per_seq, seq_lens, batch, max_seq_len, num_q_heads,
                        softmax_scale, partition, nullptr, 0, out_dtype, out, err_count, stream, true);
}

kvq_status kvq_hadamard_rotate(const uint16_t* x, int64_t num_rows, int32_t head_dim, uint16_t* out,
                               void* stream) {
  if (head_dim != 64 && head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (num_rows < 0) return KVQ_ERR_SHAPE;
  if (num_rows == 0) return KVQ_OK;
  if (!x || !out) return KVQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return KVQ_ERR_ALIGN;
  const int64_t rows_per_block = 256 / (head_dim / 8);
  if ((num_rows + rows_per_block - 1) / rows_per_block > INT32_MAX) return KVQ_ERR_SHAPE;
  return from_hip(kvq::launch_hadamard(x, num_rows, head_dim, out, static_cast<hipStream_t>(stream)));
}

const char* kvq_status_string(int32_t status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_NULL: return "KVQ_ERR_NULL: a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "KVQ_ERR_SHAPE: a size is out of range or inconsistent";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: dtype, granularity or head_dim not supported";
    case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN: a pointer is not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: decode workspace missing or too small";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: a HIP launch failed";
    default: return "unknown kvq_status";
  }
}

uint64_t kvq_cache_block_bytes(int32_t k_dtype, int32_t v_dtype, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size) {
  if (!valid_store_dtype(k_dtype) || !valid_store_dtype(v_dtype)) return 0;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || (head_dim & 1)) return 0;
  auto row = [&](int32_t d) -> uint64_t {
    if (d == KVQ_BF16) return 2ull * head_dim;
    if (d == KVQ_INT4_ASYM || d == KVQ_INT4_HAD) return (uint64_t)head_dim / 2 + 8;   // codes + fp32 (scale, zero point)
    return (uint64_t)head_dim;
  };
  return (row(k_dtype) + row(v_dtype)) * (uint64_t)num_kv_heads * (uint64_t)block_size;
}

int64_t kvq_blocks_in_budget(uint64_t budget_bytes, int32_t k_dtype, int32_t v_dtype, int32_t num_kv_heads,
                             int32_t head_dim, int32_t num_layers, int32_t block_size) {
  if (num_layers <= 0) return -1;
  const uint64_t per = kvq_cache_block_bytes(k_dtype, v_dtype, num_kv_heads, head_dim, block_size);
  if (per == 0) return -1;
  return (int64_t)(budget_bytes / (per * (uint64_t)num_layers));
}

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

}  // extern "C"
