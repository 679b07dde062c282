/*
 * kvq.h — C ABI of libkvq: a quantized paged KV cache and paged-attention
 * decode over it, for AMD Instinct MI355X (gfx950).
 *
 * What the operations are (pages cited by title and section):
 *   - vLLM issue 4025 "[Feature]: Support for 4-bit KV Cache in paged-attention
 *     op", section "methods": (1) compute the quantisation scale and zero point
 *     and convert an existing fp16/bf16 KV cache; (2) store quantised KV in the
 *     paged-cache write; (3) paged attention that takes optional k_scale,
 *     k_zeropoint, v_scale, v_zeropoint, converts the stored codes back to 16-bit
 *     and computes.
 *   - vLLM PR 4893 "[Misc] Load FP8 kv-cache scaling factors from checkpoints",
 *     description items 1-2: KV dtypes auto (= the model's 16-bit type), fp8
 *     (= e4m3), fp8_e4m3, fp8_e5m2; a scale of 1.0 when none is supplied.
 *   - "vllm-int8-kv-cache-for-ampere-sm86" summary: an INT8 KV cache with
 *     per-layer scaling values calibrated offline; FP8-E4M3 for one part of
 *     the cache (here: K and V dtypes are independent).
 *   - modelium "vLLM FP8 KV-кеш: калибровка и проверка памяти и качества",
 *     scale schemes: per-tensor and per-attention-head scales.
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are HIP device pointers, (host) host pointers.
 *     The caller allocates and owns every buffer, including decode workspace;
 *     the library allocates nothing, keeps no pointer past the call and no state
 *     between calls, and is safe to call from several host threads.  The one
 *     exception is kvq_paged_attention_decode_noalloc, whose workspace is a
 *     device array inside the library (see there).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns without synchronising; buffers must stay
 *     valid until that work has run.
 *   - Argument checks run on the host before any HIP call and return a status;
 *     nothing is enqueued on error.  KVQ_ERR_HIP reports a failed launch.
 *   - Bad data found on the device never faults: out-of-range slots or block
 *     ids are skipped (their contribution is treated as absent) and, when
 *     `err_count` (device int32, nullable) is given, counted into it with an
 *     atomic add.  The caller zeroes *err_count when it wants a fresh count.
 *   - bf16 inputs are passed as uint16_t bit patterns, row-major, contiguous,
 *     16-byte aligned.
 *
 * Paged cache layout (one layer):
 *   pages  [num_blocks][num_kv_heads][block_size][row_bytes], row_bytes =
 *          2*head_dim (BF16), head_dim (INT8 / FP8), head_dim/2 (INT4: two codes
 *          per byte, the even element in the low nibble)
 *   slot   block * block_size + offset
 *   INT4 metadata [num_blocks][num_kv_heads][block_size][2] float32 =
 *          (scale, zero_point) per (token, KV head); x_hat = (q - zp) * scale.
 *   Scales of INT8 / FP8: float32 [1] (per tensor) or [num_kv_heads] (per KV
 *          head); x_hat = code * scale (FP8: decoded value * scale).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL */
  KVQ_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  KVQ_ERR_UNSUPPORTED = 3, /* dtype, granularity or head_dim not supported */
  KVQ_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  KVQ_ERR_WORKSPACE = 5,   /* decode workspace missing or too small */
  KVQ_ERR_HIP = 6          /* a HIP launch failed */
} kvq_status;

/* Element formats.  KVQ_BF16 is the "auto" (unquantised) cache; KVQ_FP8_E4M3 is
 * what "fp8" means.  FP8 is the OCP 8-bit format (e4m3: no infinities, max 448;
 * e5m2: max 57344).  KVQ_F32 is valid only as a decode output type. */
typedef enum kvq_dtype {
  KVQ_BF16 = 0,
  KVQ_INT8 = 1,
  KVQ_FP8_E4M3 = 2,
  KVQ_FP8_E5M2 = 3,
  KVQ_INT4_ASYM = 4,
  KVQ_F32 = 5,
  /* Keys only: KVQ_INT4_ASYM codes of the Hadamard-rotated row (KVarN article,
   * technical context: a Hadamard rotation before asymmetric quantisation).  The
   * rotation is the unnormalised Sylvester-Hadamard transform y = H x of the
   * head_dim values, H[i][k] = (-1)^popcount(i & k), rounded once to bf16 (round
   * to nearest even; an exact zero is +0): exact for rows whose magnitudes span
   * less than 2^38, within one bf16 ulp otherwise.  The key such a slot holds is
   * H y_hat / head_dim (H H = head_dim I).  Decode and verify take the query and
   * softmax_scale exactly as for any other key format: the library rotates the
   * query itself and folds the 1 / head_dim into the logit scale, since
   * (H q) . y_hat = head_dim (q . H y_hat / head_dim).  Values and metadata are
   * laid out as KVQ_INT4_ASYM; V must be KVQ_INT4_ASYM. */
  KVQ_INT4_HAD = 6
} kvq_dtype;

typedef enum kvq_granularity {
  KVQ_PER_TENSOR = 0,     /* one scale for the whole K (or V) cache */
  KVQ_PER_KV_HEAD = 1,    /* one scale per KV head */
  KVQ_PER_TOKEN_HEAD = 2  /* INT4 only: (scale, zero point) per (token, KV head) */
} kvq_granularity;

/* Describes one layer's paged cache.  A host struct read during the call only. */
typedef struct kvq_cache {
  int32_t k_dtype, v_dtype;       /* kvq_dtype, independent (e.g. K e4m3, V int8) */
  int32_t k_gran, v_gran;         /* kvq_granularity (ignored for BF16) */
  int32_t num_blocks;             /* pages in the pool */
  int32_t block_size;             /* tokens per page; must be 16 */
  int32_t num_kv_heads;           /* >= 1 */
  int32_t head_dim;               /* 64 or 128 */
  void* k_pages;                  /* (device) K pages, layout above, 16-B aligned */
  void* v_pages;                  /* (device) V pages */
  const float* k_scale;           /* (device) [1] or [num_kv_heads]; NULL = 1.0; INT8/FP8 only */
  const float* v_scale;           /* (device) idem for V */
  float* k_meta;                  /* (device) INT4 (scale, zero point) metadata, else unused */
  float* v_meta;
} kvq_cache;

/*
 * kvq_calibrate_scales — absmax scale calibration (a running maximum).
 *
 * The sm86 INT8 summary calibrates per-layer scaling values offline; the
 * modelium FP8 page names per-tensor and per-attention-head scales.  For each
 * group (the whole tensor, or all tokens x head_dim of one KV head):
 *     absmax_inout[g] = max(absmax_inout[g], max |x|)     (NaN ignored)
 *     scale_out[g]    = absmax_inout[g] / qmax             (IEEE division)
 *                       or 1.0 when absmax_inout[g] == 0
 * with qmax = 127 (KVQ_INT8), 448 (KVQ_FP8_E4M3), 57344 (KVQ_FP8_E5M2).
 *   x            (device) bf16 [num_tokens][num_kv_heads][head_dim]
 *   granularity  KVQ_PER_TENSOR (G = 1) or KVQ_PER_KV_HEAD (G = num_kv_heads)
 *   absmax_inout (device) float32 [G]; the caller zero-fills it before the first
 *                batch and passes it again to accumulate over batches
 *   scale_out    (device) float32 [G], rewritten on every call
 * num_tokens may be 0 (scale_out is then recomputed from absmax_inout alone).
 */
kvq_status kvq_calibrate_scales(const uint16_t* x, int64_t num_tokens, int32_t num_kv_heads,
                                int32_t head_dim, int32_t granularity, int32_t target_dtype,
                                float* absmax_inout, float* scale_out, void* stream);

/*
 * kvq_cache_write — fused quantise-and-scatter of new K/V rows into the pages.
 *
 * vLLM issue 4025, methods item 2.  Row i of k_new / v_new is encoded and stored
 * at slot_mapping[i]:
 *   INT8:  q = clamp(RNE(x / s), -127, 127)            (NaN -> 0)
 *   FP8:   nearest code of x / s, ties to even, saturating to the largest finite
 *          value (NaN -> a NaN code)
 *   INT4:  per row: s = (max - min) / 15, zp = RNE(-min / s) (s = |min| or 1 for
 *          a constant row), q = clamp(RNE(x / s) + zp, 0, 15); (s, zp) stored
 *          in the metadata.  NaN elements are left out of min and max and get
 *          code 0; a row of only NaNs stores (NaN, NaN) and zero codes
 *   BF16:  copied
 * x / s is an IEEE-correctly-rounded float32 division.
 *   k_new, v_new  (device) bf16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  (device) int64 [num_tokens]; < 0 skips the row; >= num_blocks *
 *                 block_size is skipped and counted in err_count
 *   num_tokens    >= 0
 */
kvq_status kvq_cache_write(const kvq_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int32_t* err_count,
                           void* stream);

/*
 * kvq_convert_cache — convert an existing bf16 paged cache into `dst`'s format.
 *
 * vLLM issue 4025, methods item 1.  Every slot of blocks [first_block,
 * first_block + num_blocks) of the bf16 source pages (same geometry as dst, row
 * bytes 2*head_dim) is encoded as kvq_cache_write would encode it and stored at
 * the same slot of dst.  For INT8 / FP8 dst's scales must be set (calibrate first).
 *   k_src, v_src (device) bf16 [dst->num_blocks][num_kv_heads][block_size][head_dim]
 */
kvq_status kvq_convert_cache(const kvq_cache* dst, const uint16_t* k_src, const uint16_t* v_src,
                             int32_t first_block, int32_t num_blocks, void* stream);

/*
 * kvq_decode_workspace_size — bytes of device workspace kvq_paged_attention_decode
 * needs for these sizes and this partition (0 when the decode runs as a single
 * chunk; also 0 for invalid arguments).  Layout, for reference, with
 * S = n_chunks + batch piece slots (n_chunks as described under `partition`
 * below): float32 max [S][num_q_heads], sum [S][num_q_heads], int32 chunk range
 * [batch][2], float32 accumulators [S][num_q_heads][head_dim], each region
 * 16-byte aligned.
 */
size_t kvq_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t partition);

/*
 * kvq_paged_attention_decode — one query token per sequence against the paged
 * quantised cache.
 *
 * vLLM issue 4025, methods item 3 (attention over the stored codes with their
 * scales / zero points) and vLLM PR 4893's note that decode runs a paged
 * attention kernel.  For sequence b and query head h (KV head h / (Hq/Hkv)):
 *     z_i = softmax_scale * sum_c q[b][h][c] * k_hat_i[c]    for i < seq_lens[b]
 *     out[b][h] = sum_i softmax(z)_i * v_hat_i
 * Token position p of sequence b is read from page block_tables[b][p / 16],
 * offset p % 16.  Accumulation is float32.
 * Work split: the pages of all sequences, concatenated in sequence order, are
 * cut into chunks of equal page count, and each (chunk, KV head) is one unit of
 * work, so every unit streams the same number of bytes whatever the length mix.
 * A sequence inside one chunk is finished there; a sequence cut by chunk
 * boundaries leaves one (max, sum, accumulator) partial per piece in the
 * workspace, and a second kernel merges them (split-KV reduce).
 *   partition = 0: about 2048 / num_kv_heads chunks, their size fixed on the
 *                  device from the page total (at least 4 pages);
 *   partition > 0: chunks of partition / 16 pages, ceil(batch *
 *                  ceil(max_seq_len / 16) / (partition / 16)) of them launched.
 * Results of different partitions agree to float32 accumulation order and the
 * fp16 rounding of the softmax weights (relative 2^-12 per weight).
 *   q             (device) bf16 [batch][num_q_heads][head_dim]; |q| < 65504
 *   block_tables  (device) int32 [batch][max_blocks_per_seq]
 *   seq_lens      (device) int32 [batch]; <= 0 gives a zero output row; values
 *                 above max_seq_len or max_blocks_per_seq*16 are clamped and counted
 *   max_seq_len   host-side upper bound of seq_lens (sizes the launch)
 *   num_q_heads   multiple of num_kv_heads, at most 16 query heads per KV head
 *   partition     0 or a positive multiple of 16
 *   workspace     (device) >= kvq_decode_workspace_size(...) bytes, 16-B aligned;
 *                 may be NULL when that size is 0; no initial contents needed.
 *                 Calls that overlap in time (other streams) need workspaces of
 *                 their own.
 *   out_dtype     KVQ_BF16 (round to nearest even) or KVQ_F32
 *   out           (device) [batch][num_q_heads][head_dim] of out_dtype
 * Supported K/V dtype pairs: any of {INT8, FP8_E4M3, FP8_E5M2, BF16} for K and for
 * V independently, INT4 for both, and KVQ_INT4_HAD keys with INT4 values (q and
 * softmax_scale as for every format: the rotation of q is the library's).
 */
kvq_status kvq_paged_attention_decode(const kvq_cache* cache, const uint16_t* q,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                      int32_t num_q_heads, float softmax_scale, int32_t partition,
                                      void* workspace, size_t workspace_bytes, int32_t out_dtype,
                                      void* out, int32_t* err_count, void* stream);

/*
 * kvq_paged_attention_decode_write — the decode step's two operations in one
 * call: store each sequence's new token (vLLM issue 4025, methods item 2) and
 * attend over the cache that includes it (methods item 3).
 *
 * The same as kvq_cache_write(cache, k_new, v_new, slot_mapping, batch, ...)
 * followed by kvq_paged_attention_decode(...) with these arguments, when every
 * slot_mapping[b] is either negative (nothing written) or the slot of position
 * seq_lens[b] - 1 of sequence b, i.e. block_tables[b][(seq_lens[b] - 1) / 16] *
 * 16 + (seq_lens[b] - 1) % 16: the codes stored, the output and err_count are
 * then bit-identical to the two calls'.  One kernel does both: the wave that
 * reads the page holding position seq_lens[b] - 1 encodes the new rows and
 * stores them before it reads its first page, so the separate write launch and
 * its wait disappear from the step (every format: INT4 rows get their scale and
 * zero point, and rotated keys their rotation, exactly as kvq_cache_write
 * computes them).
 *   k_new, v_new  (device) bf16 [batch][num_kv_heads][head_dim], 16-B aligned: row
 *                 b is sequence b's new token
 *   slot_mapping  (device) int64 [batch]
 *   other arguments, workspace (kvq_decode_workspace_size) and errors as
 *                 kvq_paged_attention_decode; KVQ_ERR_NULL also for a NULL
 *                 k_new, v_new or slot_mapping when batch > 0.
 * A slot that is neither negative nor that position's is not written and is
 * counted once in err_count (kvq_cache_write would have written it); a
 * sequence with seq_lens[b] <= 0 writes nothing.
 */
kvq_status kvq_paged_attention_decode_write(const kvq_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                                            const int64_t* slot_mapping, const uint16_t* q,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                            int32_t num_q_heads, float softmax_scale, int32_t partition,
                                            void* workspace, size_t workspace_bytes, int32_t out_dtype, void* out,
                                            int32_t* err_count, void* stream);

/*
 * kvq_paged_attention_decode_noalloc — kvq_paged_attention_decode without a
 * caller-supplied workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing and calls no allocating routine.
 *
 * The split-KV partials go to a device array inside the library, one per GPU,
 * of KVQ_DECODE_SCRATCH_BYTES, held from the library's first use on that GPU
 * until the process ends.  Its device address is looked up on the first call on
 * each device (the current device, which `stream` must belong to); that call is
 * the only one that touches the HIP runtime beyond the launches.  The array
 * needs no initial contents and keeps the last call's partials.  Calls that
 * overlap in time on one GPU (other streams, other host threads) share it and
 * race: serialise them.
 * Arguments, results and errors as kvq_paged_attention_decode, plus
 * KVQ_ERR_WORKSPACE when kvq_decode_workspace_size(...) of these sizes exceeds
 * KVQ_DECODE_SCRATCH_BYTES, and KVQ_ERR_HIP when the array's address cannot be
 * obtained.
 */
#define KVQ_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

kvq_status kvq_paged_attention_decode_noalloc(const kvq_cache* cache, const uint16_t* q,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                              int32_t num_q_heads, float softmax_scale, int32_t partition,
                                              int32_t out_dtype, void* out, int32_t* err_count, void* stream);

/*
 * kvq_paged_attention_verify — several query tokens per sequence over the
 * cache, causally: speculative-decoding verification or a prefill chunk whose
 * K/V rows are already written.
 *
 * The multi-token form of the paged attention above (vLLM PR 4893's side note
 * on attention backends leaves quantised-KV attention with more than one query
 * to the paged kernel).  The last n_q positions of sequence b are its query
 * tokens: token i (row b * n_q + i of q and out) sits at position
 * p = seq_lens[b] - n_q + i and attends to cache positions 0..p; p < 0 gives a
 * zero row.  Per KV head, the n_q * g (query token, head) rows run as tiles of
 * 16 MFMA columns, a wave per tile; the tiles of a (chunk, KV head), up to four
 * at a time, form one workgroup that reads each page from memory once.  The work
 * split, the workspace and the reduce are those of kvq_paged_attention_decode,
 * which is this call with n_q = 1, except that partition = 0 makes about
 * 2048 / (num_kv_heads * tiles) chunks.
 *   q      (device) bf16 [batch * n_q][num_q_heads][head_dim], token-major
 *   n_q    >= 1, n_q * num_q_heads <= 65535
 *   out    (device) [batch * n_q][num_q_heads][head_dim] of out_dtype
 *   workspace  >= kvq_verify_workspace_size(...) bytes (same rules as decode)
 * Other arguments, errors and dtype pairs as kvq_paged_attention_decode.
 */
kvq_status kvq_paged_attention_verify(const kvq_cache* cache, const uint16_t* q, int32_t n_q,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                      int32_t num_q_heads, float softmax_scale, int32_t partition,
                                      void* workspace, size_t workspace_bytes, int32_t out_dtype,
                                      void* out, int32_t* err_count, void* stream);

/*
 * kvq_verify_workspace_size — device workspace bytes kvq_paged_attention_verify
 * needs (0 when it runs as a single chunk, or for invalid arguments).  The
 * decode layout with n_q * num_q_heads rows per slot in place of num_q_heads.
 */
size_t kvq_verify_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seq_len, int32_t partition);

/*
 * kvq_cache_block_bytes — bytes one block of one layer's cache takes: K and V
 * rows of block_size tokens for num_kv_heads heads, plus the INT4 (scale, zero
 * point) metadata, exactly what a kvq_cache of that geometry holds per block
 * (per-tensor / per-KV-head scales are O(num_kv_heads) per layer and not
 * counted).  Row bytes: 2*head_dim (BF16), head_dim (INT8 / FP8),
 * head_dim/2 + 8 (INT4 codes and metadata).  Host only, no GPU call; 0 for an
 * unsupported dtype or a non-positive size.
 */
uint64_t kvq_cache_block_bytes(int32_t k_dtype, int32_t v_dtype, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size);

/*
 * kvq_blocks_in_budget — whole cache blocks (block_size tokens, num_layers
 * layers, all KV heads) that fit in budget_bytes: the "GPU blocks" count of the
 * L4 benchmark table in vLLM PR 4893, where an 8-bit KV cache holds exactly
 * twice the blocks of a 16-bit one.  floor(budget_bytes / (num_layers *
 * kvq_cache_block_bytes(...))).  Host only; -1 for invalid arguments.
 */
int64_t kvq_blocks_in_budget(uint64_t budget_bytes, int32_t k_dtype, int32_t v_dtype, int32_t num_kv_heads,
                             int32_t head_dim, int32_t num_layers, int32_t block_size);

/*
 * kvq_hadamard_rotate — the KVQ_INT4_HAD rotation of bf16 rows (KVarN article,
 * technical context): the transform the cache write and conversion apply to
 * rotated keys, for callers that rotate other rows the same way (decode and
 * verify rotate their query themselves).
 *   x, out      (device) bf16 [num_rows][head_dim], 16-byte aligned; out may
 *               equal x (each row is read before it is written)
 *   num_rows    >= 0;  head_dim 64 or 128
 * Each output row is bf16(H x) as described at KVQ_INT4_HAD.  Errors:
 * KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED (head_dim),
 * KVQ_ERR_HIP.
 */
kvq_status kvq_hadamard_rotate(const uint16_t* x, int64_t num_rows, int32_t head_dim, uint16_t* out,
                               void* stream);

/* Human-readable name of a status code (static storage). */
const char* kvq_status_string(int32_t status);

/* KVQ_ABI_VERSION of the built library. */
int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
