#pragma once

// decode_kernel.h — paged attention over the quantised cache (vLLM issue 4025,
// methods item 3: read the stored codes, convert them to 16-bit, compute; vLLM
// PR 4893: decode runs a paged-attention kernel), plus the split-KV reduce.
// Included by decode.hip (one query token per sequence) and verify.hip
// (several, causally), each instantiating its own kernels.
//
// Work unit: the pages of all sequences, concatenated, are cut into chunks of
// equal page count; one wave (a 64-thread workgroup) per (chunk, KV head) serves
// all g = Hq/Hkv query heads of that KV head, so each K/V page is read from HBM
// exactly once.  A chunk may hold the tail of one sequence and the head of the
// next (segments); a sequence cut by a chunk boundary leaves partial results
// that the reduce kernel merges.  The wave streams its chunk CH pages per round
// with an online softmax, the DMA of round r+1 into LDS overlapping round r's
// arithmetic.  Each page is loaded through a buffer descriptor that spans exactly
// that page (0 bytes for a page whose block id is out of range), so the loads
// need no branches and an invalid page reads as zeros without touching memory.
//
// Per page (16 tokens) and wave:
//   K, INT8 / INT4 codes: the codes are the int8 operand of
//      v_mfma_i32_16x16x64_i8 against the query written as three int8 digits
//      (INT4 nibbles are unpacked to bytes first).
//   K, FP8 / BF16: the codes become exact fp16 (bf16) operands (e4m3 through
//      v_cvt_scalef32_pk_f16_fp8 with scale 1, e5m2 as the high byte of an fp16)
//      of v_mfma_f32_16x16x32_{f16,bf16} against the query in fp16 (bf16).
//      Either way lane l then holds the logits of head l%16 for tokens
//      4(l/16)+r, r=0..3: the A-operand layout of the PV product.
//   V: lane l loads rows 4(l/16)..4(l/16)+3 at columns [NE*(l%16), NE*(l%16)+NE)
//      (NE = D/16) and transposes that 4 x NE block in registers with byte
//      permutes, so that for every column it holds the 4 tokens the B operand
//      needs.  Codes become exact 16-bit values (int8: fp16 1152 + code; int4:
//      bf16 128 + code; fp8 converted to fp16); v_mfma_f32_16x16x32 over two
//      pages at once accumulates O[head][d], and one more MFMA against a column
//      of ones gives the sum of the same rounded weights (for the softmax
//      denominator and to remove the code offsets).
// Scales: per-tensor / per-head scales multiply the float32 logits (K) and the
// final output (V).  INT4 uses, per token t with (s_t, zp_t):
//   logit_t = s_t * (sum_c q_c code_c - zp_t * sum_c q_c)
//   O       = sum_t (p_t s_t) code_t - sum_t (p_t s_t) zp_t
// with the weights p_t s_t in bf16 hi + lo (BF16 V splits p_t the same way).
// Softmax runs in base 2 (log2 e folded into the logit scale).
// Masking: positions >= seq_len get logit -inf and their V operand is zeroed
// (an unused slot may hold a NaN code; 0 * NaN would leak).
// Split KV: with more than one partition per sequence each wave writes (max, sum,
// unnormalised output) of its partition to the workspace, and a second, small
// kernel merges them (a kernel boundary instead of a device-wide fence: on this
// chip an agent-scope release writes back the L2 of the issuing XCD, which costs
// far more than the launch when thousands of waves do it).
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_rows.h"
#include "kvq_launch.h"

namespace kvq {

struct Params {
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scale;
  const float* v_scale;
  int k_scale_per_head, v_scale_per_head;
  const float* k_meta;
  const float* v_meta;
  const uint16_t* q;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  int batch;
  int num_blocks, Hkv, Hq, g;
  int max_seq_len;
  float sm_log2;     // softmax_scale * log2(e)
  int chunk_pages;   // pages per chunk; 0: ceil(total pages / n_chunks), at least min_chunk
  int n_chunks;      // chunk slots; the automatic split makes this many chunks
  int min_chunk;
  int q_slot;        // LDS bytes of one query buffer (min(16, n_q g) rows of D bf16, rounded up to 1 KB)
  float* ws_m;       // [slot][n_q Hq] exponent reference (base 2) of each piece
  float* ws_l;       // [slot][n_q Hq] softmax sum of each piece
  float* ws_o;       // [slot][n_q Hq][D] unnormalised output of each piece
  int2* ws_rec;      // [B] first and last chunk of each sequence
  int out_f32;
  void* out;
  int32_t* err;
  int n_q;           // query tokens per sequence (1: decode; more: the last n_q positions, causally)
  int n_tiles;       // 16-column MFMA tiles of the n_q * g rows of a (sequence, KV head)
  int wg_waves;      // several query tokens: waves (tiles) of a workgroup, which share its pages
  // the step's new token, written in the same launch (one query token; null:
  // none): bf16 rows [B][Hkv][D] and their slots [B]
  const uint16_t* new_k;
  const uint16_t* new_v;
  const int64_t* new_slot;
};

// chunk kernels with several query tokens per sequence (verify.hip)
hipError_t launch_chunk_verify(const Params& prm, int kt, int vt, int head_dim, dim3 grid, hipStream_t s);

namespace {

constexpr float kLog2e = 1.4426950408889634f;


template <int DT, int D>
struct Geo {
  static constexpr int kRowBytes = (DT == DT_BF16) ? 2 * D : (DT == DT_INT4) ? D / 2 : D;
  static constexpr int kKLaneBytes = kRowBytes / 4;   // K bytes per lane per page
  static constexpr int kKDw = kKLaneBytes / 4;        // ... in dwords
  // A lane's K bytes are kNPC pieces of kPS bytes; piece j of lane group qg sits at
  // row offset j*4*kPS + qg*kPS, so one load instruction reads, from each of the
  // page's 16 rows, 4*kPS contiguous bytes (a whole 64-byte sector).
  static constexpr int kPS = (kKLaneBytes < 16) ? kKLaneBytes : 16;
  static constexpr int kNPC = kKLaneBytes / kPS;
  static constexpr int kNE = D / 16;                  // V columns per lane
  static constexpr int kVRowBytes = kRowBytes / 16;   // V bytes per lane per row
  static constexpr int kVDw = (kVRowBytes + 3) / 4;   // ... in dwords (int4 D=64: 2 bytes -> 1)
};

// row byte offset of dword dw of the K bytes of lane group qg
template <int DT, int D>
__host__ __device__ constexpr int k_byte(int qg, int dw) {
  constexpr int PS = Geo<DT, D>::kPS, DPP = PS / 4;
  return (dw / DPP) * 4 * PS + qg * PS + 4 * (dw % DPP);
}

__device__ __forceinline__ int clamp_len(const Params& p, int b, bool count) {
  int L = p.seq_lens[b];
  const int cap = min(p.max_seq_len, p.max_blocks_per_seq * 16);
  if (L > cap) {
    if (count && p.err) atomicAdd(p.err, 1);
    L = cap;
  }
  return L;
}

// ---------------------------------------------------------------------------
// K codes -> MFMA operand (8 fp16 / bf16 values = 4 dwords) for k-step s
// ---------------------------------------------------------------------------

template <int DT, int D, int N>
__device__ __forceinline__ u32x4 k_operand(const uint32_t (&kw)[N], int s) {
  static_assert(N == Geo<DT, D>::kKDw, "K lane width");
  static_assert(DT == DT_BF16 || DT == DT_E4M3 || DT == DT_E5M2, "INT8 / INT4 K take the integer path");
  u32x4 o;
  if constexpr (DT == DT_BF16) {
    o[0] = kw[4 * s]; o[1] = kw[4 * s + 1]; o[2] = kw[4 * s + 2]; o[3] = kw[4 * s + 3];
  } else if constexpr (DT == DT_E4M3) {
    o[0] = e4m3x2_to_f16x2<false>(kw[2 * s]);
    o[1] = e4m3x2_to_f16x2<true>(kw[2 * s]);
    o[2] = e4m3x2_to_f16x2<false>(kw[2 * s + 1]);
    o[3] = e4m3x2_to_f16x2<true>(kw[2 * s + 1]);
  } else {  // E5M2: the code byte is the fp16 high byte
    o[0] = perm(0u, kw[2 * s], 0x010C000Cu);
    o[1] = perm(0u, kw[2 * s], 0x030C020Cu);
    o[2] = perm(0u, kw[2 * s + 1], 0x010C000Cu);
    o[3] = perm(0u, kw[2 * s + 1], 0x030C020Cu);
  }
  return o;
}

// head-dim index of operand element e of k-step s for lane group qg (must match k_operand)
template <int DT, int D>
__host__ __device__ constexpr int k_dim(int qg, int s, int e) {
  if constexpr (DT == DT_INT4) return 2 * (k_byte<DT, D>(qg, s) + (e & 3)) + (e >> 2);
  else if constexpr (DT == DT_BF16) return (k_byte<DT, D>(qg, 4 * s + (e >> 1)) + 2 * (e & 1)) >> 1;
  else return k_byte<DT, D>(qg, 2 * s + (e >> 2)) + (e & 3);
}

// Integer path (INT8 and INT4 K): the K codes themselves are the operand of
// v_mfma_i32_16x16x64_i8 (16 int8 values per lane and step).  INT4 codes are
// split into even- and odd-element bytes (values 0..15).
template <int DT, int D, int N>
__device__ __forceinline__ u32x4 k_operand_i8(const uint32_t (&kw)[N], int s) {
  static_assert(N == Geo<DT, D>::kKDw, "K lane width");
  if constexpr (DT == DT_INT8) {
    return u32x4{kw[4 * s], kw[4 * s + 1], kw[4 * s + 2], kw[4 * s + 3]};
  } else {
    const uint32_t w0 = kw[2 * s], w1 = kw[2 * s + 1];
    return u32x4{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
  }
}

// head-dim index of element e (0..15) of integer-path step s (must match k_operand_i8)
template <int DT, int D>
__host__ __device__ constexpr int k_dim_i8(int qg, int s, int e) {
  if constexpr (DT == DT_INT8) return k_byte<DT, D>(qg, 4 * s + (e >> 2)) + (e & 3);
  else return 2 * (k_byte<DT, D>(qg, 2 * s + (e >> 3)) + (e & 3)) + ((e >> 2) & 1);
}

// The query elements one lane needs for one k-step are a run of RUN contiguous
// head-dim positions (8 on the fp16 / bf16 path, 16 on the integer path), in an
// order that does not depend on the lane group, starting on a 16-byte boundary:
// the query is read from LDS as whole 16-byte pieces.
template <int DT, int D, bool I8>
__host__ __device__ constexpr int q_dim(int qg, int s, int e) {
  if constexpr (I8) return k_dim_i8<DT, D>(qg, s, e);
  else return k_dim<DT, D>(qg, s, e);
}
template <int DT, int D, bool I8>
constexpr bool q_runs_ok() {
  constexpr int RUN = I8 ? 16 : 8, NSTEP = I8 ? D / 64 : D / 32;
  for (int qg = 0; qg < 4; ++qg)
    for (int s = 0; s < NSTEP; ++s) {
      const int base = q_dim<DT, D, I8>(qg, s, 0);
      if (base % 8 != 0) return false;
      unsigned seen = 0;
      for (int e = 0; e < RUN; ++e) {
        const int pos = q_dim<DT, D, I8>(qg, s, e) - base;
        if (pos < 0 || pos >= RUN || pos != q_dim<DT, D, I8>(0, s, e) - q_dim<DT, D, I8>(0, s, 0)) return false;
        seen |= 1u << pos;
      }
      if (seen != (1u << RUN) - 1u) return false;
    }
  return true;
}

// ---------------------------------------------------------------------------
// V rows -> B operands: for column e (d = NE*(l%16) + e), tokens (4qg..4qg+3) as
// two dwords of packed fp16 / bf16 pairs (t0,t1) and (t2,t3).
// ---------------------------------------------------------------------------

template <int DT, int D, int N, int NE>
__device__ __forceinline__ void v_operands(const uint32_t (&vr)[4][N], u32x2 (&ob)[NE]) {
  static_assert(N == Geo<DT, D>::kVDw && NE == Geo<DT, D>::kNE, "V operand shape");
  if constexpr (DT == DT_BF16) {
    // dword j of a row holds columns 2j, 2j+1
#pragma unroll
    for (int j = 0; j < NE / 2; ++j) {
      ob[2 * j][0] = perm(vr[1][j], vr[0][j], 0x05040100u);
      ob[2 * j][1] = perm(vr[3][j], vr[2][j], 0x05040100u);
      ob[2 * j + 1][0] = perm(vr[1][j], vr[0][j], 0x07060302u);
      ob[2 * j + 1][1] = perm(vr[3][j], vr[2][j], 0x07060302u);
    }
  } else if constexpr (DT == DT_E5M2) {
#pragma unroll
    for (int j = 0; j < NE / 4; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t sel = ((uint32_t)(4 + m) << 24) | (0x0Cu << 16) | ((uint32_t)m << 8) | 0x0Cu;
        ob[4 * j + m][0] = perm(vr[1][j], vr[0][j], sel);
        ob[4 * j + m][1] = perm(vr[3][j], vr[2][j], sel);
      }
    }
  } else if constexpr (DT == DT_INT8 || DT == DT_E4M3) {
#pragma unroll
    for (int j = 0; j < NE / 4; ++j) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        // interleave rows (2pr, 2pr+1): [r0.b0 r1.b0 r0.b1 r1.b1], [r0.b2 r1.b2 r0.b3 r1.b3]
        uint32_t i0 = perm(vr[2 * pr + 1][j], vr[2 * pr][j], 0x05010400u);
        uint32_t i1 = perm(vr[2 * pr + 1][j], vr[2 * pr][j], 0x07030602u);
        if constexpr (DT == DT_INT8) {
          // fp16 value 1152 + code; the 1152 offset is removed after the product
          i0 ^= 0x80808080u;
          i1 ^= 0x80808080u;
          ob[4 * j + 0][pr] = perm(kMagic64, i0, kSelLo);
          ob[4 * j + 1][pr] = perm(kMagic64, i0, kSelHi);
          ob[4 * j + 2][pr] = perm(kMagic64, i1, kSelLo);
          ob[4 * j + 3][pr] = perm(kMagic64, i1, kSelHi);
        } else {
          ob[4 * j + 0][pr] = e4m3x2_to_f16x2<false>(i0);
          ob[4 * j + 1][pr] = e4m3x2_to_f16x2<true>(i0);
          ob[4 * j + 2][pr] = e4m3x2_to_f16x2<false>(i1);
          ob[4 * j + 3][pr] = e4m3x2_to_f16x2<true>(i1);
        }
      }
    }
  } else {  // INT4: byte k of a row holds columns 2k (low nibble), 2k+1 (high nibble);
            // bf16 value 128 + code (exact: 8 significant bits), the offset
            // removed after the product
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const uint32_t a = vr[2 * pr][0], b = vr[2 * pr + 1][0];
#pragma unroll
      for (int hn = 0; hn < 2; ++hn) {
        const uint32_t la = hn ? ((a >> 4) & 0x0F0F0F0Fu) : (a & 0x0F0F0F0Fu);
        const uint32_t lb = hn ? ((b >> 4) & 0x0F0F0F0Fu) : (b & 0x0F0F0F0Fu);
        const uint32_t i0 = perm(lb, la, 0x05010400u);   // bytes 0,1 of both rows
        ob[0 + hn][pr] = perm(kMagic43, i0, kSelLo);     // column 2*0 + hn
        ob[2 + hn][pr] = perm(kMagic43, i0, kSelHi);     // column 2*1 + hn
        if constexpr (NE == 8) {
          const uint32_t i1 = perm(lb, la, 0x07030602u); // bytes 2,3
          ob[4 + hn][pr] = perm(kMagic43, i1, kSelLo);
          ob[6 + hn][pr] = perm(kMagic43, i1, kSelHi);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------

template <bool BF>
__device__ __forceinline__ f32x4 mfma_qk(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma_pv(const u32x2& a, const u32x2& b, const f32x4& c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8(const u32x4& a, const u32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}

// PV over two pages at once: k = 32 tokens
template <bool BF>
__device__ __forceinline__ f32x4 mfma_pv2(const u32x4& a, const u32x4& b, const f32x4& c) {
  return mfma_qk<BF>(a, b, c);
}

// two floats -> a packed 16-bit pair, round to nearest even (bf16: one
// v_cvt_pk_bf16_f32, which turns a NaN into a quiet NaN)
__device__ __forceinline__ uint32_t pack2(float a, float b, bool bf) {
  if (bf) {
    const bf16x2n v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float unpack_lo(uint32_t v, bool bf) {
  if (bf) return bf16_bits_to_f32(v & 0xffffu);
  return (float)__builtin_bit_cast(f16x2, v)[0];
}
__device__ __forceinline__ float unpack_hi(uint32_t v, bool bf) {
  if (bf) return bf16_bits_to_f32(v >> 16);
  return (float)__builtin_bit_cast(f16x2, v)[1];
}

// fp16 pair of the remainders (a - h.lo, b - h.hi), h the fp16 pair of (a, b):
// each remainder is exact in fp32 (h is a rounded to 11 bits), so a mixed fma
// per element, h's half read as fp16 times m1 = -1 plus the element, gives the
// same bits as converting h back and subtracting.  m1 is -1 hidden from the
// optimiser (which would fold it into a subtraction of a reconverted h), and h
// must come in opaque for the same reason; the instructions stay the
// compiler's own, so it keeps their hazards with the MFMAs that read the result.
__device__ __forceinline__ uint32_t f16_remainders(float a, float b, uint32_t h, float m1) {
  const f16x2 hv = __builtin_bit_cast(f16x2, h);
  const f16x2 v = {(_Float16)__builtin_fmaf((float)hv[0], m1, a), (_Float16)__builtin_fmaf((float)hv[1], m1, b)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// per-page buffer resources: a page's K (or V, or INT4 metadata) rows form one
// contiguous range; a descriptor covering exactly that range (0 bytes for an
// invalid page) lets every lane load without a branch: out-of-range loads
// return zeros and touch no memory.
// ---------------------------------------------------------------------------

constexpr int kRsrcFlags = 0x00020000;   // gfx9 buffer descriptor word 3 (raw 32-bit data)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcFlags);
}

// ---------------------------------------------------------------------------
// split-KV reduce: merges the pieces of a sequence that chunk boundaries cut,
//   o = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,  M = max_j m_j.
// Piece j of sequence b (chunk rec.x + j) sits in slot rec.x + j + b.  A lane
// group of D/4 lanes holds one row's 4-column slices.  A separate launch: the
// kernel boundary makes every piece's stores visible without a device-wide
// fence.
//   decode_reduce_kernel: one workgroup per (row, sequence); its groups take
//     every NG-th piece, and LDS combines the groups (for few rows with many
//     pieces each: a long context cut into hundreds of chunks).
//   decode_reduce_rows_kernel: one group per row, NG rows of a sequence per
//     workgroup (for many rows with few pieces each: several query tokens).
// ---------------------------------------------------------------------------

constexpr int kRedThreads = 256;

// running merge of pieces (m_j, l_j, acc_j) for one lane's 4 columns
struct PieceMerge {
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  __device__ __forceinline__ void add(float mj, float lj, const float4& v) {
    const bool ok = (mj != -INFINITY);        // -inf: past P, or a piece with no valid token
    const float Mn = ok ? fmaxf(M, mj) : M;
    const float sc = (Mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float f = ok ? __builtin_amdgcn_exp2f(mj - Mn) : 0.0f;
    acc.x = acc.x * sc + (ok ? f * v.x : 0.0f);
    acc.y = acc.y * sc + (ok ? f * v.y : 0.0f);
    acc.z = acc.z * sc + (ok ? f * v.z : 0.0f);
    acc.w = acc.w * sc + (ok ? f * v.w : 0.0f);
    den = den * sc + (ok ? f * lj : 0.0f);
    M = Mn;
  }
};

// pieces j0, j0 + step, ... (U of them, those past P masked) of one row, all
// loads in flight before any is used
template <int U, int D>
__device__ __forceinline__ void merge_pieces(PieceMerge& pm, const float* m, const float* l, const float* o,
                                             int RS, int P, int j0, int step, int ln) {
  float mj[U], lj[U];
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = j0 + u * step;
    const size_t jj = (size_t)min(j, P - 1);
    mj[u] = (j < P) ? m[jj * RS] : -INFINITY;
    lj[u] = l[jj * RS];
    v[u] = *reinterpret_cast<const float4*>(o + jj * RS * D + 4 * ln);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) pm.add(mj[u], lj[u], v[u]);
}

// the normalised row slice (zeros when no piece holds a valid token)
__device__ __forceinline__ void store_row_slice(const Params& p, size_t oi, float4 a, float dd) {
  const bool any = dd > 0.0f;
  const float r[4] = {any ? a.x / dd : 0.0f, any ? a.y / dd : 0.0f, any ? a.z / dd : 0.0f, any ? a.w / dd : 0.0f};
  if (p.out_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + oi) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    const uint32_t lo = (uint32_t)f32_to_bf16_bits(r[0]) | ((uint32_t)f32_to_bf16_bits(r[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_bits(r[2]) | ((uint32_t)f32_to_bf16_bits(r[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + oi) = make_uint2(lo, hi);
  }
}

template <int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_kernel(Params p) {
  constexpr int LPG = D / 4;                  // lanes per group
  constexpr int NG = kRedThreads / LPG;       // groups
  const int hq = blockIdx.x, b = blockIdx.y;   // hq: row (query token, query head) of sequence b
  // the workspace pointers are read before rec, so that the loads of the pieces
  // follow rec's load by one memory round trip, not by another kernel-argument one
  const float* wm = p.ws_m;
  const float* wl = p.ws_l;
  const float* wo = p.ws_o;
  const int RS = p.Hq * p.n_q;                // rows per sequence and slot
  asm volatile("" ::"s"(wm), "s"(wl), "s"(wo), "s"(RS));
  const int2 rec = p.ws_rec[b];
  if (rec.y <= rec.x) return;                 // one piece: the chunk kernel wrote the row
  const int P = rec.y - rec.x + 1;
  const size_t s0 = (size_t)rec.x + b;
  const float* m = wm + s0 * RS + hq;
  const float* l = wl + s0 * RS + hq;
  const float* o = wo + (s0 * RS + hq) * D;

  const int grp = threadIdx.x / LPG, ln = threadIdx.x % LPG;
  PieceMerge pm;
  if (P <= NG) {
    // at most one piece per group (branch-free, so the three loads go out together)
    merge_pieces<1, D>(pm, m, l, o, RS, P, grp, NG, ln);
  } else {
    // eight pieces per group and pass: a sequence cut into hundreds of pieces
    // is then a few round trips
    for (int j0 = grp; j0 < P; j0 += 8 * NG) merge_pieces<8, D>(pm, m, l, o, RS, P, j0, NG, ln);
  }
  __shared__ float4 s_acc[NG][LPG];
  __shared__ float s_m[NG], s_den[NG];
  s_acc[grp][ln] = pm.acc;
  if (ln == 0) {
    s_m[grp] = pm.M;
    s_den[grp] = pm.den;
  }
  __syncthreads();
  if (threadIdx.x < LPG) {
    float MM = s_m[0];
#pragma unroll
    for (int gi = 1; gi < NG; ++gi) MM = fmaxf(MM, s_m[gi]);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float dd = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float f = (s_m[gi] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[gi] - MM);
      const float4 v = s_acc[gi][threadIdx.x];
      a.x += f * v.x; a.y += f * v.y; a.z += f * v.z; a.w += f * v.w;
      dd += f * s_den[gi];
    }
    store_row_slice(p, ((size_t)b * RS + hq) * D + 4 * threadIdx.x, a, dd);
  }
}

template <int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_rows_kernel(Params p) {
  constexpr int LPG = D / 4;                  // lanes per group
  constexpr int NG = kRedThreads / LPG;       // rows per workgroup
  const float* wm = p.ws_m;
  const float* wl = p.ws_l;
  const float* wo = p.ws_o;
  const int RS = p.Hq * p.n_q;                // rows per sequence and slot
  asm volatile("" ::"s"(wm), "s"(wl), "s"(wo), "s"(RS));
  const int b = blockIdx.y;
  const int2 rec = p.ws_rec[b];
  if (rec.y <= rec.x) return;                 // one piece: the chunk kernel wrote the rows
  const int grp = threadIdx.x / LPG, ln = threadIdx.x % LPG;
  const int hq = blockIdx.x * NG + grp;
  if (hq >= RS) return;
  const int P = rec.y - rec.x + 1;
  const size_t s0 = (size_t)rec.x + b;
  const float* m = wm + s0 * RS + hq;
  const float* l = wl + s0 * RS + hq;
  const float* o = wo + (s0 * RS + hq) * D;
  PieceMerge pm;
  for (int j0 = 0; j0 < P; j0 += 4) merge_pieces<4, D>(pm, m, l, o, RS, P, j0, 1, ln);
  store_row_slice(p, ((size_t)b * RS + hq) * D + 4 * ln, pm.acc, pm.den);
}

// ---------------------------------------------------------------------------
// query rotation for rotated keys: y = H q, H[i][k] = (-1)^popcount(i & k) (the
// rotation of the stored keys).  On the integer path lane group qg holds head-dim
// positions qg * NL + local(s2, e), NL = 16 * D / 64, so the butterfly runs over
// the local positions inside the lane, then over qg between lanes l and l ^ 16,
// l and l ^ 32 (the pair at (i, i + h) becomes (a + b, a - b)), in float32.
// ---------------------------------------------------------------------------

template <int KT, int D>
__host__ __device__ constexpr int q_local(int s2, int e) {
  return q_dim<KT, D, true>(0, s2, e) - q_dim<KT, D, true>(0, 0, 0);
}
template <int KT, int D>
constexpr bool q_lane_block_ok() {
  constexpr int NL = 16 * (D / 64);
  for (int qg = 0; qg < 4; ++qg)
    for (int s2 = 0; s2 < D / 64; ++s2)
      for (int e = 0; e < 16; ++e)
        if (q_dim<KT, D, true>(qg, s2, e) != qg * NL + q_local<KT, D>(s2, e)) return false;
  return true;
}

template <int KT, int D>
__device__ __forceinline__ void rotate_query(float (&qv)[D / 64][16], int qg) {
  constexpr int NSI = D / 64, NL = 16 * NSI;
  static_assert(q_lane_block_ok<KT, D>(), "a lane group holds one contiguous block of head-dim positions");
  float y[NL];
#pragma unroll
  for (int s2 = 0; s2 < NSI; ++s2)
#pragma unroll
    for (int e = 0; e < 16; ++e) y[q_local<KT, D>(s2, e)] = qv[s2][e];
#pragma unroll
  for (int h = 1; h < NL; h <<= 1)
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (!(i & h)) {
        const float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  // v_permlane16_swap of a value with itself leaves the value of the even and
  // of the odd 16-lane row of each pair; v_permlane32_swap that of each half
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[i]), __float_as_uint(y[i]), false, false);
    const float other = __uint_as_float((qg & 1) ? r[0] : r[1]);
    y[i] = (qg & 1) ? other - y[i] : y[i] + other;
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[i]), __float_as_uint(y[i]), false, false);
    const float other = __uint_as_float((qg & 2) ? r[0] : r[1]);
    y[i] = (qg & 2) ? other - y[i] : y[i] + other;
  }
#pragma unroll
  for (int s2 = 0; s2 < NSI; ++s2)
#pragma unroll
    for (int e = 0; e < 16; ++e) qv[s2][e] = y[q_local<KT, D>(s2, e)];
}

// ---------------------------------------------------------------------------
// the chunk kernel: one wave per (chunk, KV head)
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// LDS staging.  A wave streams its partition through an NST-deep ring of LDS
// stages; a stage holds the K and V pages (and INT4 metadata) of one round of CH
// pages.  Pages arrive by buffer_load ... lds DMA: each instruction moves 1 KB
// (64 lanes x 16 B) of one page, whole 128-byte lines, without passing through
// VGPRs, so the ring can hold several rounds in flight.  The 16-byte chunks of a
// row are XOR-swizzled by the row index, which the per-lane source offsets of the
// DMA apply and the ds_read addresses undo; the MFMA-layout reads (16 rows, same
// column) then hit distinct banks.
// ---------------------------------------------------------------------------

template <int DT, int D>
struct LdsPage {
  static constexpr int RB = Geo<DT, D>::kRowBytes;
  static constexpr int CPR = RB / 16;                         // 16-byte chunks per row
  static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;
  static constexpr int PAGE = 16 * RB;
  static constexpr int SLOT = PAGE < 1024 ? 1024 : PAGE;      // LDS bytes reserved per page
  static constexpr int NINSTR = SLOT / 1024;                  // DMA instructions per page
  // LDS byte of row-relative byte `byte` of row `row`
  __device__ static __forceinline__ int at(int row, int byte) {
    return row * RB + (((byte >> 4) ^ (row & SWZ)) << 4) + (byte & 15);
  }
  // page byte lane `lane` of DMA instruction t fetches (its LDS position is 1024t + 16 lane)
  __device__ static __forceinline__ int src(int t, int lane) {
    const int pos = 64 * t + lane;                 // 16-byte chunk index in the slot
    const int row = pos / CPR, cs = pos % CPR;
    return row * RB + ((cs ^ (row & SWZ)) << 4);   // rows >= 16 fall outside the page: read as 0
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

// LDS reads of DMA-filled stages are issued as inline assembly: the compiler cannot
// tell the ring stages apart and would otherwise wait for every DMA in flight
// (vmcnt(0)) before each read.  The explicit vmcnt waits of the ring order the
// reads after their own stage's DMA; lds_fence(regs) waits for the reads
// (lgkmcnt(0)) and ties the registers to that wait so no use can move above it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8_t*)p;
}
__device__ __forceinline__ u32x4 ds_b128(uint32_t a) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ u32x2 ds_b64(uint32_t a) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ uint32_t ds_b32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ uint32_t ds_u16(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// LDS writes in the same (volatile, in-order) stream as the reads above
__device__ __forceinline__ void ds_w32(uint32_t a, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_w64(uint32_t a, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
template <typename T>
__device__ __forceinline__ void lds_tie(T& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_dst, 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt in [3:0] and [15:14]; expcnt and
// lgkmcnt fields left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 32) (larger n: vmcnt(0))
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  if constexpr (N < 32) {
    if (n == N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_rt<N + 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// lazy rescaling: the exponent reference of a head moves only when a logit exceeds
// it by more than this (base 2), so p = 2^(z - m_ref) <= 256 stays finite in fp16
// and the accumulators are rescaled only when a head's maximum jumps.
constexpr float kRescaleSlack = 8.0f;

template <int KT, int VT, int D, int CH>
struct StageGeo {
  using KP = LdsPage<KT, D>;
  using VP = LdsPage<VT, D>;
  static constexpr bool META = (KT == DT_INT4);           // INT4 is K and V together
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = CH * KP::SLOT;
  static constexpr int M_OFF = V_OFF + CH * VP::SLOT;     // per page: K meta [0,256), V meta [256,512)
  static constexpr int STAGE = M_OFF + (META ? CH * 512 : 0);
  static constexpr int LPR = CH * (KP::NINSTR + VP::NINSTR + (META ? 2 : 0));   // DMA loads per round
};

// One round: up to CH consecutive pages of one sequence, all inside one segment
// (the piece of a sequence that lies in this wave's chunk).  Wave-uniform, kept
// small: three of them are live at once in scalar registers.
template <int CH>
struct Desc {
  int b;          // sequence
  int pg;         // first page of the round, counted from the start of the sequence
  int L;          // sequence length in tokens
  int info;       // kNp: pages in the round (0: no round, the chunk is done); flags below
  int bid[CH];    // block id of each page, -1: not loaded (past the segment or out of range)
};
constexpr int kNp = 7;           // info bits 0-2
constexpr int kFirst = 1 << 3;   // first round of its segment
constexpr int kLast = 1 << 4;    // last round of its segment
constexpr int kTail = 1 << 5;    // holds the sequence's last page (tokens past L are masked)
constexpr int kWhole = 1 << 6;   // the segment is the whole sequence
constexpr int kQBuf = 1 << 7;    // query buffer of the segment (segments alternate)

// inclusive prefix sum over the wave by DPP moves: shifts by 1, 2, 4, 8 inside
// each 16-lane row (lanes shifted in from outside the row read 0), then lane 15
// added to rows 1 and 3 and lane 31 to rows 2 and 3 (row broadcasts)
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// MQ: several query tokens per sequence (verify); without it n_q is 1 and the
// (token, head) row arithmetic folds away.  With MQ a workgroup of up to four
// waves, one per 16-column tile, shares each round: every wave DMAs a share of
// the round's pages into the common LDS stage, waits for its share, and a
// barrier makes the whole round visible; a second barrier, once every wave has
// read the round into registers, frees the stage, and the round after next is
// issued into it before the round's arithmetic.  The page bytes are then read
// once for all the tiles of a workgroup.
// The step's new token of one sequence and KV head (the one-call decode step):
// its bf16 K and V rows (src_k, src_v: D values each) encoded as the cache write
// encodes them and stored to their rows of the pages (dst_k, dst_v).  Lanes below
// D / 4 take 4 values each.
template <int KT, int VT, int D>
__device__ __forceinline__ void store_new_rows(const uint16_t* src_k, const uint16_t* src_v, uint8_t* dst_k,
                                               uint8_t* dst_v, float ksc, float vsc, int lane) {
  if (lane >= D / 4) return;
  const u32x2 rk = *reinterpret_cast<const u32x2*>(src_k + 4 * lane);
  const u32x2 rv = *reinterpret_cast<const u32x2*>(src_v + 4 * lane);
  auto put = [&](auto dt_tag, const u32x2& raw, float sc, uint8_t* g) __attribute__((always_inline)) {
    constexpr int DTX = decltype(dt_tag)::value;
    if constexpr (DTX == DT_BF16) {
      *reinterpret_cast<u32x2*>(g + 8 * lane) = raw;
    } else {
      const Quot qt(sc);
      float t[4];
      t[0] = qt(bf16_bits_to_f32(raw[0] & 0xffffu));
      t[1] = qt(bf16_bits_to_f32(raw[0] >> 16));
      t[2] = qt(bf16_bits_to_f32(raw[1] & 0xffffu));
      t[3] = qt(bf16_bits_to_f32(raw[1] >> 16));
      uint32_t w;
      if constexpr (DTX == DT_INT8)
        w = enc_int8(t[0]) | (enc_int8(t[1]) << 8) | (enc_int8(t[2]) << 16) | (enc_int8(t[3]) << 24);
      else
        w = enc_fp8x4<DTX>(t);
      *reinterpret_cast<uint32_t*>(g + 4 * lane) = w;
    }
  };
  put(std::integral_constant<int, KT>{}, rk, ksc, dst_k);
  put(std::integral_constant<int, VT>{}, rv, vsc, dst_v);
}

// The same for INT4 K and V, with the cache write's own row encoder: lanes
// [0, LPR) hold the K row and [LPR, 2 LPR) the V row, 8 values each (LPR = D / 8
// aligned lanes a row, as in the write kernel); a rotated K row (ROT) is rotated
// first.  The row's codes go to dst_k / dst_v, its (scale, zero point) pair to
// meta_k / meta_v.
template <int D, bool ROT>
__device__ __forceinline__ void store_new_rows_int4(const uint16_t* src_k, const uint16_t* src_v, uint8_t* dst_k,
                                                    uint8_t* dst_v, float* meta_k, float* meta_v, int lane) {
  constexpr int LPR = D / 8;
  const int grp = lane / LPR, j = lane % LPR;
  if (grp > 1) return;
  const uint4 raw = *reinterpret_cast<const uint4*>((grp ? src_v : src_k) + 8 * j);
  const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(wd[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(wd[i] >> 16);
  }
  if constexpr (ROT) {
    // every lane of both rows runs the butterfly (its moves stay in the group);
    // the V row keeps its values
    float xr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xr[i] = x[i];
    hadamard_row<LPR>(xr, j);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = grp ? x[i] : xr[i];
  }
  float sc, zp;
  const uint32_t packed = encode_int4<LPR>(x, &sc, &zp);
  *reinterpret_cast<uint32_t*>((grp ? dst_v : dst_k) + 4 * j) = packed;
  if (j == 0) *reinterpret_cast<float2*>(grp ? meta_v : meta_k) = make_float2(sc, zp);
}

template <int KT_DECL, int VT, int D, int CH, bool MQ, bool NEW>
__global__ __launch_bounds__(MQ ? 256 : 64) void decode_chunk_kernel(Params p) {
  // rotated keys (DT_INT4H) are INT4 codes of H k: the same pages and products,
  // with the query rotated alike when a segment's query rows are read
  constexpr bool KROT = (KT_DECL == DT_INT4H);
  constexpr int KT = KROT ? DT_INT4 : KT_DECL;
  static_assert(CH % 2 == 0, "pages are consumed in pairs by the PV product");
  static_assert(CH <= kNp, "pages per round fit the descriptor");
  using KG = Geo<KT, D>;
  using VG = Geo<VT, D>;
  using SG = StageGeo<KT, VT, D, CH>;
  using KP = typename SG::KP;
  using VP = typename SG::VP;
  constexpr int NS = D / 32;       // QK k-steps (fp16 / bf16 path)
  constexpr int NE = VG::kNE;      // PV n-tiles
  constexpr bool KBF = (KT == DT_BF16);
  constexpr bool VBF = (VT == DT_BF16);
  // PV weights in bf16, split hi + lo (two MFMAs, about 16 significant bits):
  // BF16 V, and INT4 V, whose weights p_t s_t carry the token's scale and would
  // leave fp16's range (or its precision) for very large or very small scales
  constexpr bool WBF = (VT == DT_BF16 || VT == DT_INT4);
  // every PV weight goes in as hi + lo (fp16 pairs for INT8 / FP8 V): a single
  // rounded weight carries 2^-11 relative error, which a peaked softmax over
  // large V values does not average away
  constexpr bool WSPLIT = true;
  constexpr bool V_NAN = (VT == DT_E4M3 || VT == DT_E5M2 || VT == DT_BF16);  // codes that can decode to NaN/Inf
  constexpr bool KI8 = (KT == DT_INT8 || KT == DT_INT4);   // integer QK path
  constexpr int NSI = D / 64;                               // its k-steps (16 codes each)
  // V operands carrying a constant offset (fp16 1152 + code, bf16 128 + code): the
  // offset times sum_t p_t is removed after the product, with sum_t p_t taken from
  // one more MFMA against a column of ones (the same rounded p the product saw)
  constexpr bool V_FOLD = (VT == DT_INT8 || VT == DT_INT4);
  constexpr float V_OFFSET = (VT == DT_INT8) ? 1152.0f : 128.0f;
  constexpr int KPAGE = KP::PAGE, VPAGE = VP::PAGE;
  // the step's new token written in this launch (one query token)
  constexpr bool FW = NEW && !MQ;
  static_assert(!NEW || FW, "the new-token write: one query token");
  constexpr int STAGE_B = SG::STAGE;

  // two ring stages, one LDS object each: reads of one stage then carry no
  // dependence on the DMA still filling the other; the query rows of the current
  // and the next segment sit in two dynamic-LDS buffers of p.q_slot bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds0[STAGE_B];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[STAGE_B];
  extern __shared__ __attribute__((aligned(16))) uint8_t qlds_all[];
  auto stage_ptr = [&](auto s_tag) -> uint8_t* {
    if constexpr (decltype(s_tag)::value == 0) return lds0;
    else return lds1;
  };

  // grid (chunks x query tiles, KV heads), the tile fastest: the tiles of one
  // chunk are neighbours in launch order, so they read its pages at about the
  // same time
  const int n_tiles = MQ ? p.n_tiles : 1;
  const int NW = MQ ? p.wg_waves : 1;                      // waves of the workgroup
  // this wave (its tile) in the workgroup, wave-uniform (a scalar register)
  const int wv = MQ ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  const int n_groups = (n_tiles + NW - 1) / NW;            // workgroups per (chunk, KV head)
  const int tau = MQ ? (int)(blockIdx.x % n_groups) * NW + wv : 0;
  const int w = MQ ? (int)(blockIdx.x / n_groups) : (int)blockIdx.x;
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  uint8_t* qlds = qlds_all + 2 * p.q_slot * wv;            // this wave's two query buffers
  const int c = lane & 15, qg = lane >> 4;
  const int g = p.g;
  const int B = p.batch;
  const int n_q = MQ ? p.n_q : 1;
  // rows (query token i, head h) of a (sequence, KV head), row = i g + h; this
  // wave's 16 MFMA columns are rows col0 .. col0 + 15 (decode: the g heads)
  const int rows = n_q * g;
  const int col0 = 16 * tau;
  const int cap = min(p.max_seq_len, p.max_blocks_per_seq * 16);
  const bool counter = (tau == 0 && w == 0 && kvh == 0);   // the one wave that counts clamped lengths

  // warm the caches with the block table (into a ring stage not in use yet; its
  // later DMAs are younger and land after these), so that the scalar loads of
  // block ids after the length scan hit in L2.  Workgroups go to the XCDs in turn
  // (linear id modulo 8), and each XCD has its own L2: the waves of one XCD,
  // those with equal id modulo 8, pull one copy of the table between them, up to
  // 4 KB per wave.  Not with a shared ring: another wave's stage-1 DMA could land
  // before this one.
  if constexpr (!MQ) {
    const size_t bt_bytes = (size_t)B * p.max_blocks_per_seq * 4;
    const size_t wid = (size_t)kvh * gridDim.x + blockIdx.x;
    const size_t per_xcd = ((size_t)gridDim.x * gridDim.y + 7) / 8;
    const size_t kb = min((bt_bytes + per_xcd * 1024 - 1) / (per_xcd * 1024), (size_t)4);   // KB per wave
    const size_t off = (wid / 8) * kb * 1024;
    if (off < bt_bytes) {
      const auto rb = page_rsrc(reinterpret_cast<const uint8_t*>(p.block_tables) + off,
                                (int)min(bt_bytes - off, kb * 1024));
      for (int t = 0; t < (int)kb; ++t) dma16(rb, lds1 + 1024 * t, 1024 * t + 16 * lane);
    }
  }

  // length of sequence b, clamped to [0, cap] (0 past the batch)
  auto load_len = [&](int b, bool count) {
    int L = 0;
    if (b < B) {
      L = p.seq_lens[b];
      if (L > cap) {
        if (count && p.err) atomicAdd(p.err, 1);
        L = cap;
      }
      L = max(L, 0);
    }
    return L;
  };

  // ---- pages of every sequence: their total T fixes the chunk size.  Batches
  //      of up to NR groups of 64 stay in registers (lane j of group r holds
  //      sequence 64 r + j), their lengths loaded all at once; larger batches
  //      are scanned group by group and reloaded where needed ----
  constexpr int NR = 4;
  const bool in_regs = B <= 64 * NR;
  int lr[NR], nr[NR], ir[NR];   // length, pages, inclusive page prefix
  int T = 0;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < NR; ++r) lr[r] = (64 * r < B) ? load_len(64 * r + lane, counter) : 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      nr[r] = (lr[r] + 15) >> 4;
      ir[r] = T;
      if (64 * r < B) {
        ir[r] += wave_incl_sum(nr[r]);
        T = __builtin_amdgcn_readlane(ir[r], 63);
      }
    }
  } else {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int L = load_len(b0 + lane, counter);
      T += __builtin_amdgcn_readlane(wave_incl_sum((L + 15) >> 4), 63);
    }
  }
  int C = p.chunk_pages;
  if (C == 0) C = max(p.min_chunk, (T + p.n_chunks - 1) / p.n_chunks);
  const int n_act = max(1, (T + C - 1) / C);
  if (w >= n_act) return;
  const int x0 = w * C, x1 = min(x0 + C, T);
  const bool last_chunk = (w == n_act - 1);

  // ---- the chunk's first sequence: the first whose pages reach past x0, or an
  //      empty one at or after x0 (empty sequences belong to the chunk holding
  //      their position; those at the very end to the last chunk) ----
  auto starts_here = [&](int np, int inc) { return inc > x0 || (np == 0 && inc >= x0); };
  int bs = 0, ex_bs = 0;
  if (in_regs) {
    // the sequences before the chunk form a prefix of the batch
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (64 * r < B) bs += popc64(__builtin_amdgcn_ballot_w64(64 * r + lane < B && !starts_here(nr[r], ir[r])));
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (r == (bs >> 6)) ex_bs = __builtin_amdgcn_readlane(ir[r] - nr[r], bs & 63);
  } else {
    int carry = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int L = load_len(b0 + lane, false);
      const int np = (L + 15) >> 4;
      const int inc = carry + wave_incl_sum(np);
      const int cnt = popc64(__builtin_amdgcn_ballot_w64(lane < B - b0 && !starts_here(np, inc)));
      if (cnt < min(64, B - b0)) {
        bs = b0 + cnt;
        ex_bs = __builtin_amdgcn_readlane(inc - np, cnt);
        break;
      }
      carry = __builtin_amdgcn_readlane(inc, 63);
    }
  }

  // ---- window: lane j describes sequence bs + j ----
  int wL = 0, wnp = 0, wex = 0, wlo = 0, whi = 0;
  int nwin = 0;
  bool more = false;
  auto make_window = [&](bool from_regs) __attribute__((always_inline)) {
    const int sb = bs + lane;
    const bool wv = sb < B;
    if (from_regs) {
      // sequence bs + j sits in group (bs >> 6) or the next one, at lane sb & 63
      const int g0 = bs >> 6;
      int la = 0, na = 0, xa = 0, lb = 0, nb = 0, xb = 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r == g0) { la = lr[r]; na = nr[r]; xa = ir[r] - nr[r]; }
        if (r == g0 + 1) { lb = lr[r]; nb = nr[r]; xb = ir[r] - nr[r]; }
      }
      const int src = sb & 63;
      const bool second = (sb >> 6) != g0;
      const int ta = __shfl(la, src, 64), tb = __shfl(lb, src, 64);
      const int ua = __shfl(na, src, 64), ub = __shfl(nb, src, 64);
      const int va = __shfl(xa, src, 64), vb = __shfl(xb, src, 64);
      wL = second ? tb : ta;
      wnp = second ? ub : ua;
      wex = second ? vb : va;
    } else {
      wL = load_len(sb, false);
      wnp = (wL + 15) >> 4;
      wex = ex_bs + wave_incl_sum(wnp) - wnp;
    }
    if (!wv) wL = wnp = 0;
    const bool in_chunk = wv && (last_chunk || wex < x1);
    wlo = in_chunk ? max(x0 - wex, 0) : 0;
    whi = in_chunk ? min(x1 - wex, wnp) : 0;
    nwin = popc64(__builtin_amdgcn_ballot_w64(in_chunk));
    more = (nwin == 64) && (bs + 64 < B);
    // records for the reduce: the KV-head-0 wave holding a sequence's last page
    // stores the range of chunks the sequence spans (equal ends: not split)
    if (p.ws_rec && kvh == 0 && tau == 0 && in_chunk) {
      int2 rec;
      if (wnp == 0) rec = make_int2(w, w);
      else rec = make_int2(wex / C, (wex + wnp - 1) / C);
      if (wnp == 0 || wex + wnp <= x1) p.ws_rec[sb] = rec;
    }
    // empty sequences of the chunk: zero rows for this wave's columns
    uint64_t em = __builtin_amdgcn_ballot_w64(in_chunk && wnp == 0);
    while (em) {
      const int j = __builtin_ctzll(em);
      em &= em - 1;
      for (int i = lane; i < 16 * D; i += 64) {
        const int r = col0 + i / D;
        if (r >= rows) break;
        const size_t at = ((((size_t)(bs + j) * n_q + r / g) * p.Hq) + (size_t)kvh * g + r % g) * D + i % D;
        if (p.out_f32) reinterpret_cast<float*>(p.out)[at] = 0.0f;
        else reinterpret_cast<uint16_t*>(p.out)[at] = 0;
      }
    }
  };
  make_window(in_regs);

  // ---- per-wave constants: logit and output scales ----
  // this KV head's K and V scales (1.0 when none is set)
  float ksc = 1.0f, vsc = 1.0f;
  if constexpr (KT == DT_INT8 || KT == DT_E4M3 || KT == DT_E5M2) {
    if (p.k_scale) ksc = p.k_scale[p.k_scale_per_head ? kvh : 0];
  }
  if constexpr (VT == DT_INT8 || VT == DT_E4M3 || VT == DT_E5M2) {
    if (p.v_scale) vsc = p.v_scale[p.v_scale_per_head ? kvh : 0];
  }
  float kfac = p.sm_log2 * ksc;
  const float vfac = vsc;
  int koff[KP::NINSTR], voff[VP::NINSTR];
#pragma unroll
  for (int t = 0; t < KP::NINSTR; ++t) koff[t] = KP::src(t, lane);
#pragma unroll
  for (int t = 0; t < VP::NINSTR; ++t) voff[t] = VP::src(t, lane);
  // page addresses: this KV head's first page plus block id times the block
  // stride (all KV heads of a block), in unsigned 32x32->64 arithmetic
  const uint8_t* kbase = p.k_pages + (size_t)kvh * KPAGE;
  const uint8_t* vbase = p.v_pages + (size_t)kvh * VPAGE;
  const uint32_t kstride = (uint32_t)p.Hkv * KPAGE;
  const uint32_t vstride = (uint32_t)p.Hkv * VPAGE;
  const float* kmbase = p.k_meta + (size_t)kvh * 32;
  const float* vmbase = p.v_meta + (size_t)kvh * 32;
  const uint32_t mstride = (uint32_t)p.Hkv * 128;
  // query rows of a segment: each 16-byte piece t of the wave's query buffer is
  // column (64 t + lane) / (D / 8) and a slice of it, gathered by the DMA from
  // row (token i, head h) of the sequence's query block; pieces of columns past
  // the rows read from beyond the buffer's range, as zeros
  const int q_bytes = n_q * p.Hq * D * 2;        // one sequence's query block
  int q_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int piece = 64 * t + lane;
    const int cc = piece / (D / 8), within = 16 * (piece % (D / 8));
    const int r = col0 + cc;
    const int off = ((r / g) * p.Hq + kvh * g + r % g) * D * 2 + within;
    q_off[t] = (MQ && cc < 16 && r < rows) ? off : q_bytes;
  }

  const int nq = p.q_slot >> 10;              // query-row loads of a segment (1 to 4)
  // DMA units of a round: one instruction each, K, V (and INT4 metadata) of
  // each page in turn; with several waves, unit u is wave (u % NW)'s
  constexpr int UPP = KP::NINSTR + VP::NINSTR + (SG::META ? 2 : 0);   // units per page
  static_assert(CH * UPP <= 32, "DMA units of a round");
  uint32_t my_units = 0;
  for (int u = 0; u < CH * UPP; ++u) my_units |= (u % NW == wv) ? (1u << u) : 0u;

  // ---- cursor over the rounds of the chunk (wave-uniform) ----
  int cj = -1, cpg = 0, clo = 0, chi = 0, cqb = kQBuf;
  int bad = 0;                                 // pages with an out-of-range block id
  auto next = [&]() __attribute__((always_inline)) {
    Desc<CH> d;
    d.b = d.pg = d.L = d.info = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) d.bid[i] = -1;
    while (cpg >= chi) {                       // on to the next non-empty segment
      ++cj;
      if (cj >= nwin) {
        if (!more) return d;
        ex_bs = __builtin_amdgcn_readlane(wex, 63) + __builtin_amdgcn_readlane(wnp, 63);
        bs += 64;
        make_window(false);
        cj = 0;
        if (nwin == 0) return d;
      }
      clo = __builtin_amdgcn_readlane(wlo, cj);
      chi = __builtin_amdgcn_readlane(whi, cj);
      cpg = clo;
      if (chi > clo) cqb ^= kQBuf;
    }
    const int pages = __builtin_amdgcn_readlane(wnp, cj);
    const int np = min(CH, chi - cpg);
    d.b = bs + cj;
    d.pg = cpg;
    d.L = __builtin_amdgcn_readlane(wL, cj);
    d.info = np | cqb | (cpg == clo ? kFirst : 0) | (cpg + CH >= chi ? kLast : 0) |
             ((MQ ? (cpg + np) * 16 + n_q - 1 > d.L : cpg + np == pages) ? kTail : 0) |
             (clo == 0 && chi == pages ? kWhole : 0);
    // block ids are scalar loads (the table is read-only here), counted by
    // lgkmcnt and never by the vmcnt the ring waits on; they are issued two
    // rounds before the round's DMA
    const_i32_t* row = (const_i32_t*)(p.block_tables + (size_t)d.b * p.max_blocks_per_seq);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int bb = row[cpg + min(i, np - 1)];
      const bool inb = (uint32_t)bb < (uint32_t)p.num_blocks;
      if (i < np) {
        d.bid[i] = inb ? bb : -1;
        if (!inb) bad++;
      }
    }
    cpg += CH;
    return d;
  };

  // DMA of one round into a stage: first the query rows when the round opens a
  // segment, then K, V (and INT4 metadata) of its pages.  The ring waits count
  // only the page loads: loads issued before them are older, so a wait that
  // leaves the newest LPR loads in flight has finished them too.
  auto issue = [&](const Desc<CH>& d, auto s_tag) __attribute__((always_inline)) {
    uint8_t* sb = stage_ptr(s_tag);
    // the per-unit tests below are scalar bit tests made here, each time: hoisted
    // out of the loop as lane masks they would crowd the scalar registers
    const uint32_t mu = MQ ? (uint32_t)__builtin_amdgcn_readfirstlane((int)my_units) : ~0u;
    const int nqo = MQ ? __builtin_amdgcn_readfirstlane(nq) : nq;
    if (d.info & kFirst) {
      uint8_t* qd = qlds + ((d.info & kQBuf) ? p.q_slot : 0);
      if constexpr (MQ) {
        const auto rq = page_rsrc(p.q + (size_t)d.b * n_q * p.Hq * D, q_bytes);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (t < nqo) dma16(rq, qd + 1024 * t, q_off[t]);
      } else {
        // one token: its g rows are one contiguous run
        const auto rq = page_rsrc(p.q + ((size_t)d.b * p.Hq + (size_t)kvh * g) * D, g * D * 2);
        for (int t = 0; t < p.q_slot; t += 1024) dma16(rq, qd + t, t + 16 * lane);
      }
    }
    // load unit u of the round (one DMA instruction) is this wave's when bit u
    // of my_units is set (every unit when the wave is alone)
    auto mine = [&](int u) { return !MQ || ((mu >> u) & 1u); };
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool ok = d.bid[i] >= 0;
      const uint32_t bid = ok ? (uint32_t)d.bid[i] : 0u;
      const uint64_t koffb = (uint64_t)bid * kstride;
      const uint64_t voffb = (VPAGE == KPAGE) ? koffb : (uint64_t)bid * vstride;
      const auto rk = page_rsrc(kbase + koffb, ok ? KPAGE : 0);
#pragma unroll
      for (int t = 0; t < KP::NINSTR; ++t)
        if (mine(i * UPP + t)) dma16(rk, sb + SG::K_OFF + i * KP::SLOT + 1024 * t, koff[t]);
      const auto rv = page_rsrc(vbase + voffb, ok ? VPAGE : 0);
#pragma unroll
      for (int t = 0; t < VP::NINSTR; ++t)
        if (mine(i * UPP + KP::NINSTR + t)) dma16(rv, sb + SG::V_OFF + i * VP::SLOT + 1024 * t, voff[t]);
      if constexpr (SG::META) {
        const uint64_t moff = (uint64_t)bid * mstride;
        const auto rkm = page_rsrc(reinterpret_cast<const uint8_t*>(kmbase) + moff, ok ? 128 : 0);
        if (mine(i * UPP + KP::NINSTR + VP::NINSTR)) dma4(rkm, sb + SG::M_OFF + i * 512, 4 * lane);
        const auto rvm = page_rsrc(reinterpret_cast<const uint8_t*>(vmbase) + moff, ok ? 128 : 0);
        if (mine(i * UPP + KP::NINSTR + VP::NINSTR + 1)) dma4(rvm, sb + SG::M_OFF + i * 512 + 256, 4 * lane);
      }
    }
  };

  float m1 = -1.0f;                 // -1, opaque to the optimiser (f16_remainders)
  asm("" : "+v"(m1));

  // ---- segment state ----
  // query operand: head c (zero if c >= g), in the k order of the K operand.
  // Integer path: q = sq * (q2 + q1 / 128 + q0 / 16384), three int8 digits and a
  // per-head scale sq = max|q| / 127; each digit's remainder lies in [-64, 64], so
  // no digit clips, and the representation error is below 2^-15 sq per element
  u32x4 qop[KI8 ? 1 : NS];
  u32x4 qd[KI8 ? 3 : 1][KI8 ? NSI : 1];
  float qsum_i = 0.0f;   // INT4: sum over d of (16384 q2 + 128 q1 + q0) for head c
  float kq = 0.0f;       // integer path: logit = kq * (16384 a2 + 128 a1 + a0)
  float kq4 = 0.0f;      // INT4: the same times the token's scale
  float m_ref = -INFINITY;   // exponent reference of head c (uniform over qg)
  float corr_run = 0.0f;     // INT4 V: per-lane partial of sum (p s) zp
  float l_run = 0.0f;        // INT4 V: per-lane partial softmax sum (its operand is p s)
  f32x4 oacc[NE];
  // sum over tokens of the P operand per head (all columns alike), from one MFMA
  // against a column of ones: the softmax denominator, from the same rounded
  // weights as the numerator (INT4 V: sum_t p_t s_t, the V offset multiplier),
  // and (V_FOLD) the multiplier of the V offset
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
  // logit factor of this lane's head, 0 for lanes past the group (their logits
  // become -inf through lane_bias, so their weights are 0)
  const bool hv_lane = col0 + c < rows;
  const float lane_bias = hv_lane ? 0.0f : -INFINITY;
  float kf_lane = hv_lane ? kfac : 0.0f;
  // causal limit of this lane's column: token i attends to positions below
  // L - n_q + i + 1 (decode: L)
  const int lim_off = MQ ? 1 - n_q + (hv_lane ? (col0 + c) / g : 0) : 0;

  auto begin_segment = [&](const Desc<CH>& d) __attribute__((always_inline)) {
    m_ref = -INFINITY;
    corr_run = 0.0f;
    l_run = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool hv = col0 + c < rows;
    const uint32_t qb = lds_addr(qlds + ((d.info & kQBuf) ? p.q_slot : 0)) + (uint32_t)((hv ? c : 0) * D * 2);
    static_assert(q_runs_ok<KT, D, KI8>(), "query runs");
    if constexpr (KI8) {
      // step s2: 16 bf16 values, two 16-byte reads
      u32x4 raw[NSI][2];
#pragma unroll
      for (int s2 = 0; s2 < NSI; ++s2) {
        const uint32_t a = qb + 2 * q_dim<KT, D, true>(qg, s2, 0);
        raw[s2][0] = ds_b128(a);
        raw[s2][1] = ds_b128(a + 16);
      }
      lds_fence();
#pragma unroll
      for (int s2 = 0; s2 < NSI; ++s2) {
        lds_tie(raw[s2][0]);
        lds_tie(raw[s2][1]);
      }
      // lanes of a padding head (c >= g) read head 0's row; their digits come out
      // zero through inv = 0 below
      auto qval = [&](int s2, int e) {
        const int pos = q_dim<KT, D, true>(0, s2, e) - q_dim<KT, D, true>(0, s2, 0);
        const uint32_t wd = raw[s2][pos >> 3][(pos >> 1) & 3];
        return __uint_as_float((pos & 1) ? (wd & 0xffff0000u) : (wd << 16));
      };
      float qv[NSI][16];
#pragma unroll
      for (int s2 = 0; s2 < NSI; ++s2)
#pragma unroll
        for (int e = 0; e < 16; ++e) qv[s2][e] = qval(s2, e);
      if constexpr (KROT) rotate_query<KT, D>(qv, qg);
      float amax = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < NSI; ++s2)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(qv[s2][e]));
      amax = xor32_max(xor16_max(amax));
      const float sq = (amax > 0.0f) ? amax / 127.0f : 1.0f;
      const float inv = hv ? 1.0f / sq : 0.0f;
      // digits by the 1.5 * 2^23 trick: for |x| < 2^22, x + M rounds x to the
      // nearest integer (ties to even, as rintf) and holds it, in two's
      // complement, in its low mantissa bits; (x + M) - M is that integer
      constexpr float kM = 12582912.0f;
      float dsum[3] = {0.f, 0.f, 0.f};      // INT4: digit sums (exact small integers)
#pragma unroll
      for (int s2 = 0; s2 < NSI; ++s2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t tb[3][4];                // bits of x + M: the digit in the low byte
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // |x| <= 127 up to rounding, so the first digit lies in [-127, 127]
            float x = qv[s2][4 * i + k] * inv;
#pragma unroll
            for (int dg = 0; dg < 3; ++dg) {
              const float t = x + kM;
              const float digit = t - kM;
              tb[dg][k] = __float_as_uint(t);
              if (dg < 2) x = (x - digit) * 128.0f;
              if constexpr (KT == DT_INT4) dsum[dg] += digit;
            }
          }
          // low bytes of the four words: [k0 k1 k2 k3]
#pragma unroll
          for (int dg = 0; dg < 3; ++dg) {
            const uint32_t lo = perm(tb[dg][1], tb[dg][0], 0x0c0c0400u);
            const uint32_t hi = perm(tb[dg][3], tb[dg][2], 0x0c0c0400u);
            qd[dg][s2][i] = perm(hi, lo, 0x05040100u);
          }
        }
      }
      if constexpr (KT == DT_INT4) {
#pragma unroll
        for (int dg = 0; dg < 3; ++dg) {
          dsum[dg] = xor32_sum(xor16_sum(dsum[dg]));
        }
        qsum_i = (dsum[0] * 128.0f + dsum[1]) * 128.0f + dsum[2];
      }
      kq = hv ? kfac * sq * (1.0f / 16384.0f) : 0.0f;
      // rotated keys: (H q) . (H k) = D (q . k), so the logit takes 1 / D more
      kq4 = hv ? p.sm_log2 * sq * (1.0f / 16384.0f) * (KROT ? 1.0f / D : 1.0f) : 0.0f;
    } else {
      // step s: 8 bf16 values, one 16-byte read
      u32x4 raw[NS];
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) raw[s2] = ds_b128(qb + 2 * q_dim<KT, D, false>(qg, s2, 0));
      lds_fence();
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        lds_tie(raw[s2]);
        uint32_t qb8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = q_dim<KT, D, false>(0, s2, e) - q_dim<KT, D, false>(0, s2, 0);
          const uint32_t wd = raw[s2][pos >> 1];
          qb8[e] = hv ? ((pos & 1) ? (wd >> 16) : (wd & 0xffffu)) : 0u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (KBF) {
            qop[s2][i] = qb8[2 * i] | (qb8[2 * i + 1] << 16);
          } else {
            f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(bf16_bits_to_f32(qb8[2 * i]),
                                                                            bf16_bits_to_f32(qb8[2 * i + 1])));
            qop[s2][i] = __builtin_bit_cast(uint32_t, h2);
          }
        }
      }
    }
  };

  // ---- one round from an LDS stage: QK, softmax, PV ----
  // TAIL: the round holds the sequence's last page, the only one with tokens past
  // its end; other rounds skip every per-token test.
  auto round = [&](auto tail_tag, const Desc<CH>& cur, auto s_tag, auto&& after_reads) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const uint8_t* sb = stage_ptr(s_tag);

    // every LDS read of the round (K, V and INT4 metadata of its pages) is issued
    // at once, behind one wait
    u32x4 kv16[CH][KG::kNPC];
    u32x2 kv8[CH][KG::kNPC];
    u32x4 km[CH][2];
    u32x4 vraw16[CH][4];
    u32x2 vraw8[CH][4];
    uint32_t vraw4[CH][4];
    u32x4 vm[CH][2];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t kb = lds_addr(sb + SG::K_OFF + i * KP::SLOT);
#pragma unroll
      for (int j = 0; j < KG::kNPC; ++j) {
        const uint32_t at = kb + KP::at(c, j * 4 * KG::kPS + qg * KG::kPS);
        if constexpr (KG::kPS == 16) kv16[i][j] = ds_b128(at);
        else kv8[i][j] = ds_b64(at);
      }
      if constexpr (KT == DT_INT4) {
        const uint32_t mb = lds_addr(sb + SG::M_OFF + i * 512 + 32 * qg);
        km[i][0] = ds_b128(mb);
        km[i][1] = ds_b128(mb + 16);
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t vb = lds_addr(sb + SG::V_OFF + i * VP::SLOT);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t at = vb + VP::at(4 * qg + r, c * VG::kVRowBytes);
        if constexpr (VG::kVRowBytes == 16) vraw16[i][r] = ds_b128(at);
        else if constexpr (VG::kVRowBytes == 8) vraw8[i][r] = ds_b64(at);
        else if constexpr (VG::kVRowBytes == 4) vraw4[i][r] = ds_b32(at);
        else vraw4[i][r] = ds_u16(at);
      }
      if constexpr (VT == DT_INT4) {
        const uint32_t mb = lds_addr(sb + SG::M_OFF + i * 512 + 256 + 32 * qg);
        vm[i][0] = ds_b128(mb);
        vm[i][1] = ds_b128(mb + 16);
      }
    }
    lds_fence();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
#pragma unroll
      for (int j = 0; j < KG::kNPC; ++j) {
        if constexpr (KG::kPS == 16) lds_tie(kv16[i][j]);
        else lds_tie(kv8[i][j]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (VG::kVRowBytes == 16) lds_tie(vraw16[i][r]);
        else if constexpr (VG::kVRowBytes == 8) lds_tie(vraw8[i][r]);
        else lds_tie(vraw4[i][r]);
      }
      if constexpr (KT == DT_INT4) { lds_tie(km[i][0]); lds_tie(km[i][1]); }
      if constexpr (VT == DT_INT4) { lds_tie(vm[i][0]); lds_tie(vm[i][1]); }
    }
    after_reads();   // the stage's data is in registers: the stage may be refilled

    // QK: logits of head c for tokens 4qg+r of each page
    float sl[CH][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      uint32_t kw[KG::kKDw];
#pragma unroll
      for (int j = 0; j < KG::kNPC; ++j) {
        if constexpr (KG::kPS == 16) {
          kw[4 * j] = kv16[i][j][0]; kw[4 * j + 1] = kv16[i][j][1]; kw[4 * j + 2] = kv16[i][j][2]; kw[4 * j + 3] = kv16[i][j][3];
        } else {
          kw[2 * j] = kv8[i][j][0]; kw[2 * j + 1] = kv8[i][j][1];
        }
      }
      float4 km0, km1;
      if constexpr (KT == DT_INT4) {
        km0 = __builtin_bit_cast(float4, km[i][0]);
        km1 = __builtin_bit_cast(float4, km[i][1]);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KI8) {
        i32x4 a2 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, a0 = {0, 0, 0, 0};
#pragma unroll
        for (int s2 = 0; s2 < NSI; ++s2) {
          const u32x4 ko = k_operand_i8<KT, D>(kw, s2);
          a2 = mfma_i8(ko, qd[0][s2], a2);
          a1 = mfma_i8(ko, qd[1][s2], a1);
          a0 = mfma_i8(ko, qd[2][s2], a0);
        }
        // (128 a2 + a1) is exact in int32; the last digit joins in float32
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = (float)((a2[r] << 7) + a1[r]) * 128.0f + (float)a0[r];
      } else {
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) acc = mfma_qk<KBF>(k_operand<KT, D>(kw, s2), qop[s2], acc);
      }
      // logit = factor * acc + bias: a page not loaded has factor 0 and bias
      // -inf, as have lanes past the group, so its weights come out 0
      const int tbase = (cur.pg + i) * 16 + 4 * qg;
      const bool okp = cur.bid[i] >= 0;
      const float zb = okp ? lane_bias : -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float z;
        if constexpr (KT == DT_INT4) {
          const float ks = (r < 2) ? ((r == 0) ? km0.x : km0.z) : ((r == 2) ? km1.x : km1.z);
          const float kz = (r < 2) ? ((r == 0) ? km0.y : km0.w) : ((r == 2) ? km1.y : km1.w);
          z = okp ? fmaf(ks * kq4, acc[r] - kz * qsum_i, lane_bias) : -INFINITY;
        } else if constexpr (KT == DT_INT8) {
          z = fmaf(acc[r], okp ? kq : 0.0f, zb);
        } else {
          z = fmaf(acc[r], okp ? kf_lane : 0.0f, zb);
        }
        if constexpr (TAIL) z = (tbase + r < cur.L + lim_off) ? z : -INFINITY;
        sl[i][r] = z;
        cmax = fmaxf(cmax, z);
      }
    }

    // lazy online-softmax update (the first round of a segment only sets the
    // reference: its accumulators are still zero)
    cmax = xor32_max(xor16_max(cmax));
    if (cur.info & kFirst) {
      m_ref = cmax;
    } else {
      const bool jump = cmax > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(jump)) {
        const float alpha = jump ? __builtin_amdgcn_exp2f(m_ref - cmax) : 1.0f;   // m_ref = -inf -> 0
        m_ref = jump ? cmax : m_ref;
        corr_run *= alpha;
        l_run *= alpha;
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = shfl_f(alpha, 4 * qg + r);   // alpha of head 4qg+r
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[e][r] *= ar[r];
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[r] *= ar[r];
      }
    }
    const float msub = (m_ref == -INFINITY) ? 0.0f : m_ref;

    // PV, two pages per MFMA (32 tokens): the V operands of the page pair, then
    // the weights and the products
#pragma unroll
    for (int i = 0; i < CH; i += 2) {
      u32x2 vop[2][NE];
      float vs[2][4], vz[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pi = i + h2;
        // V rows 4qg..4qg+3 of the page, this lane's columns (and INT4 metadata)
        uint32_t vw[4][VG::kVDw];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (VG::kVRowBytes == 16) {
            vw[r][0] = vraw16[pi][r][0]; vw[r][1] = vraw16[pi][r][1]; vw[r][2] = vraw16[pi][r][2]; vw[r][3] = vraw16[pi][r][3];
          } else if constexpr (VG::kVRowBytes == 8) {
            vw[r][0] = vraw8[pi][r][0]; vw[r][1] = vraw8[pi][r][1];
          } else {
            vw[r][0] = vraw4[pi][r];
          }
        }
        if constexpr (VT == DT_INT4) {
          const float4 vm0 = __builtin_bit_cast(float4, vm[pi][0]);
          const float4 vm1 = __builtin_bit_cast(float4, vm[pi][1]);
          vs[h2][0] = vm0.x; vs[h2][1] = vm0.z; vs[h2][2] = vm1.x; vs[h2][3] = vm1.z;
          vz[h2][0] = vm0.y; vz[h2][1] = vm0.w; vz[h2][2] = vm1.y; vz[h2][3] = vm1.w;
        }
        v_operands<VT, D>(vw, vop[h2]);
        if constexpr (TAIL && V_NAN) {
          // tokens past the end of the sequence: their slots may hold NaN codes
          const int tb = (cur.pg + pi) * 16 + 4 * qg;
          const uint32_t m01 = ((tb + 0 < cur.L) ? 0x0000ffffu : 0u) | ((tb + 1 < cur.L) ? 0xffff0000u : 0u);
          const uint32_t m23 = ((tb + 2 < cur.L) ? 0x0000ffffu : 0u) | ((tb + 3 < cur.L) ? 0xffff0000u : 0u);
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            vop[h2][e][0] &= m01;
            vop[h2][e][1] &= m23;
          }
        }
      }
      u32x4 aop;
      u32x4 aop_lo;   // weights w = w_hi + w_lo (w_hi alone carries 8 or 11 bits)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pi = i + h2;
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(sl[pi][r] - msub);     // -inf -> 0
          if constexpr (VT == DT_INT4) l_run += pr[r];
        }
        uint32_t a0, a1;
        if constexpr (VT == DT_INT4) {
          // only the sequence's last page holds unwritten slots, whose metadata
          // may be NaN: there a zero weight must not meet it
          float ps[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ps[r] = (!TAIL || pr[r] != 0.0f) ? pr[r] * vs[h2][r] : 0.0f;
          a0 = pack2(ps[0], ps[1], true);
          a1 = pack2(ps[2], ps[3], true);
          aop_lo[2 * h2] = pack2(ps[0] - unpack_lo(a0, true), ps[1] - unpack_hi(a0, true), true);
          aop_lo[2 * h2 + 1] = pack2(ps[2] - unpack_lo(a1, true), ps[3] - unpack_hi(a1, true), true);
          // the zero-point term from the unrounded weights (hi + lo equals them to
          // about 2^-17; this keeps the error off the term zp, which is unbounded)
#pragma unroll
          for (int r = 0; r < 4; ++r) corr_run += (!TAIL || ps[r] != 0.0f) ? ps[r] * vz[h2][r] : 0.0f;
        } else {
          a0 = pack2(pr[0], pr[1], VBF);
          a1 = pack2(pr[2], pr[3], VBF);
        }
        aop[2 * h2] = a0;
        aop[2 * h2 + 1] = a1;
        if constexpr (VT != DT_INT4 && WBF) {
          aop_lo[2 * h2] = pack2(pr[0] - unpack_lo(a0, true), pr[1] - unpack_hi(a0, true), true);
          aop_lo[2 * h2 + 1] = pack2(pr[2] - unpack_lo(a1, true), pr[3] - unpack_hi(a1, true), true);
        } else if constexpr (VT != DT_INT4 && WSPLIT) {
          asm("" : "+v"(a0), "+v"(a1));
          aop_lo[2 * h2] = f16_remainders(pr[0], pr[1], a0, m1);
          aop_lo[2 * h2 + 1] = f16_remainders(pr[2], pr[3], a1, m1);
        }
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const u32x4 bop = {vop[0][e][0], vop[0][e][1], vop[1][e][0], vop[1][e][1]};
        oacc[e] = mfma_pv2<WBF>(aop, bop, oacc[e]);
        if constexpr (WBF || WSPLIT) oacc[e] = mfma_pv2<WBF>(aop_lo, bop, oacc[e]);
      }
      {
        constexpr uint32_t one2 = WBF ? 0x3F803F80u : 0x3C003C00u;   // bf16 / fp16 1.0 pairs
        const u32x4 ones = {one2, one2, one2, one2};
        sacc = mfma_pv2<WBF>(aop, ones, sacc);
        if constexpr (WBF || WSPLIT) sacc = mfma_pv2<WBF>(aop_lo, ones, sacc);
      }
    }
  };

  // ---- end of a segment: the sequence's output, or the piece's partial ----
  auto end_segment = [&](const Desc<CH>& d) __attribute__((always_inline)) {
    float c_all = 0.0f, l_all = 0.0f;
    if constexpr (VT == DT_INT4) {
      c_all = xor32_sum(xor16_sum(corr_run));
      l_all = xor32_sum(xor16_sum(l_run));
    }
    // lane (qg, c) holds O[head 4qg+r][d = NE*c + e] and that head's operand sum;
    // fetch its reference (and INT4 sums) from the lanes of head 4qg+r
    float lh[4], ch[4], mh[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lh[r] = (VT == DT_INT4) ? shfl_f(l_all, 4 * qg + r) : sacc[r];
      ch[r] = (VT == DT_INT4) ? shfl_f(c_all, 4 * qg + r) : 0.0f;
      mh[r] = shfl_f(m_ref, 4 * qg + r);
    }
    const int slot = w + d.b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = col0 + 4 * qg + r;       // row (token rr / g, head rr % g)
      if (rr >= rows) continue;
      const int tok = (n_q == 1) ? 0 : rr / g;
      const size_t hq = (size_t)tok * p.Hq + (size_t)kvh * g + (rr - tok * g);   // row of the token's block
      float o[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        float v = oacc[e][r] - ch[r];
        if constexpr (V_FOLD) v -= V_OFFSET * sacc[r];
        o[e] = v * vfac;
      }
      if (d.info & kWhole) {
        const size_t row = (size_t)d.b * n_q * p.Hq + hq;
        // one reciprocal per row (within an ulp of dividing each element)
        const float rl = (lh[r] > 0.0f) ? 1.0f / lh[r] : 0.0f;
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] *= rl;
        if (p.out_f32) {
          float* dst = reinterpret_cast<float*>(p.out) + row * D + NE * c;
#pragma unroll
          for (int e = 0; e < NE; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
        } else {
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + row * D + NE * c;
          uint32_t pk[NE / 2];
#pragma unroll
          for (int e = 0; e < NE; e += 2) pk[e / 2] = pack2(o[e], o[e + 1], true);
          if constexpr (NE == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          else *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
        }
      } else {
        const size_t prow = (size_t)slot * n_q * p.Hq + hq;
        float* dst = p.ws_o + prow * D + NE * c;
#pragma unroll
        for (int e = 0; e < NE; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
        if (c == 0) {
          p.ws_m[prow] = mh[r];
          p.ws_l[prow] = lh[r];
        }
      }
    }
  };

  // The two waves sharing a SIMD are served oldest first; left alone, the older
  // one finishes its chunk long before the younger, and the CU then runs the
  // rest of the kernel with half its waves.  Each wave lowers its own priority
  // as its share of the chunk gets done, so the one that is behind is served
  // first and the waves of a CU finish together.
  // (the quarter of the chunk done, 4 done / total, by comparisons, not a division)
  int done4 = 0;
  const int total_rounds = max(1, (x1 - x0 + CH - 1) / CH);
  auto pace = [&]() {
    if (done4 < total_rounds) __builtin_amdgcn_s_setprio(3);
    else if (done4 < 2 * total_rounds) __builtin_amdgcn_s_setprio(2);
    else if (done4 < 3 * total_rounds) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    done4 += 4;
  };
  auto compute = [&](const Desc<CH>& d, auto s_tag, auto&& after_reads) __attribute__((always_inline)) {
    if constexpr (!MQ) pace();   // the workgroup's barriers already keep its waves together
    if (d.info & kFirst) begin_segment(d);
    if (d.info & kTail) round(std::true_type{}, d, s_tag, after_reads);
    else round(std::false_type{}, d, s_tag, after_reads);
    if (d.info & kLast) end_segment(d);
  };

  // ---- the ring: round r sits in stage r % 2; while it is computed, round r+1
  //      is in flight and the block ids of round r+2 are being loaded ----
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // wait for everything but the round just issued (d): its page loads, plus its
  // query-row loads when it opens a segment; a fixed LPR would make the wave
  // wait for part of d itself, one full memory latency at every segment start
  // a workgroup's wave issues every NW-th load unit of a round
  const int my_lpr = (SG::LPR - wv + NW - 1) / NW;
  auto wait_issued = [&](const Desc<CH>& d) {
    if (!(d.info & kNp)) wait_vmcnt<0>();
    else if (MQ) wait_vmcnt_rt(my_lpr + ((d.info & kFirst) ? nq : 0));
    else if (!(d.info & kFirst)) wait_vmcnt<SG::LPR>();
    else if (nq <= 1) wait_vmcnt<SG::LPR + 1>();
    else if (nq == 2) wait_vmcnt<SG::LPR + 2>();
    else if (nq == 3) wait_vmcnt<SG::LPR + 3>();
    else wait_vmcnt<SG::LPR + 4>();
  };
  // Several query tokens: the waves of the workgroup share each round, so a
  // barrier after every wave's wait for its share makes the round visible to
  // all, and a barrier after every wave has read it frees its stage.
  // kEarly: both stages are filled at the start, and the round after next is
  // issued into a stage as soon as the barrier marks it read, ahead of the
  // round's arithmetic, so it has nearly two rounds of arithmetic to arrive in.
  // With a bf16 V operand the registers this keeps live push the kernel past
  // 256 VGPRs (one wave per SIMD), so there, as with one query token, the
  // round after next is issued once the round is done.
  constexpr bool kEarly = MQ && VT != DT_BF16;

  // ---- the step's new tokens (the one-call decode step) ----
  // Each sequence whose last page lies in this chunk takes its new token at
  // position L - 1: row (L - 1) % 16 of page (L - 1) / 16.  Its slot must be that
  // position's; then its K and V rows are encoded as the cache write encodes
  // them and stored to the page before any page of the chunk is read (the page
  // is read later by this wave alone, and a wave's memory operations to one
  // address take effect in order; the wait below completes the stores too).  A
  // negative slot writes nothing; any other slot is counted (once, by the
  // KV-head-0 wave) and not written.
  if constexpr (FW) {
    auto write_new = [&](int b, int L) __attribute__((always_inline)) {
      const int64_t S = p.new_slot[b];
      if (S < 0) return;
      const int pos = L - 1;
      const int bb = p.block_tables[(size_t)b * p.max_blocks_per_seq + (pos >> 4)];
      if ((uint32_t)bb >= (uint32_t)p.num_blocks || S != (int64_t)bb * 16 + (pos & 15)) {
        if (p.err && kvh == 0 && lane == 0) atomicAdd(p.err, 1);
        return;
      }
      const size_t row = ((size_t)b * p.Hkv + kvh) * D;
      uint8_t* dk = const_cast<uint8_t*>(kbase) + (size_t)bb * kstride + (size_t)(pos & 15) * KP::RB;
      uint8_t* dv = const_cast<uint8_t*>(vbase) + (size_t)bb * vstride + (size_t)(pos & 15) * VP::RB;
      if constexpr (KT == DT_INT4) {
        // (scale, zero point) of row r of the (block, KV head) page: [block][Hkv][16][2]
        const size_t mi = (((size_t)bb * p.Hkv + kvh) * 16 + (pos & 15)) * 2;
        store_new_rows_int4<D, KROT>(p.new_k + row, p.new_v + row, dk, dv, const_cast<float*>(p.k_meta) + mi,
                                     const_cast<float*>(p.v_meta) + mi, lane);
      } else {
        store_new_rows<KT, VT, D>(p.new_k + row, p.new_v + row, dk, dv, ksc, vsc, lane);
      }
    };
    // the sequence's last page (inclusive page prefix inc, minus one) is in the chunk
    auto ends_here = [&](int np, int inc) { return np > 0 && inc - 1 >= x0 && inc - 1 < x1; };
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (64 * r >= B) continue;
        uint64_t m = __builtin_amdgcn_ballot_w64(64 * r + lane < B && ends_here(nr[r], ir[r]));
        while (m) {
          const int j = __builtin_ctzll(m);
          m &= m - 1;
          write_new(64 * r + j, __builtin_amdgcn_readlane(lr[r], j));
        }
      }
    } else {
      int carry = 0;
      for (int b0 = 0; b0 < B && carry < x1; b0 += 64) {
        const int L = load_len(b0 + lane, false);
        const int np = (L + 15) >> 4;
        const int inc = carry + wave_incl_sum(np);
        uint64_t m = __builtin_amdgcn_ballot_w64(lane < B - b0 && ends_here(np, inc));
        while (m) {
          const int j = __builtin_ctzll(m);
          m &= m - 1;
          write_new(b0 + j, __builtin_amdgcn_readlane(L, j));
        }
        carry = __builtin_amdgcn_readlane(inc, 63);
      }
    }
    wait_vmcnt<0>();
  }

  Desc<CH> da = next();
  if constexpr (!kEarly) {
    if (da.info & kNp) {
      // the first round's DMA goes out before the second round's block ids are read
      issue(da, S0{});
      Desc<CH> dn = next();
      Desc<CH> db;
      auto none = []() __attribute__((always_inline)) {};
      while (true) {
        if (dn.info & kNp) issue(dn, S1{});
        db = dn;
        dn = next();
        wait_issued(db);
        if constexpr (MQ) __builtin_amdgcn_s_barrier();
        compute(da, S0{}, none);
        if constexpr (MQ) __builtin_amdgcn_s_barrier();
        if (!(db.info & kNp)) break;

        if (dn.info & kNp) issue(dn, S0{});
        da = dn;
        dn = next();
        wait_issued(da);
        if constexpr (MQ) __builtin_amdgcn_s_barrier();
        compute(db, S1{}, none);
        if constexpr (MQ) __builtin_amdgcn_s_barrier();
        if (!(da.info & kNp)) break;
      }
    }
  } else if (da.info & kNp) {
    Desc<CH> db = next();
    issue(da, S0{});
    if (db.info & kNp) issue(db, S1{});
    Desc<CH> dn = next();
    while (true) {
      wait_issued(db);
      __builtin_amdgcn_s_barrier();
      compute(da, S0{}, [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_barrier();
        if (dn.info & kNp) issue(dn, S0{});
      });
      if (!(db.info & kNp)) break;
      da = dn;
      dn = next();

      wait_issued(da);
      __builtin_amdgcn_s_barrier();
      compute(db, S1{}, [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_barrier();
        if (dn.info & kNp) issue(dn, S1{});
      });
      if (!(da.info & kNp)) break;
      db = dn;
      dn = next();
    }
  }
  if (bad && p.err && lane == 0) atomicAdd(p.err, bad);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// pages per round (the ring has two stages: one round in flight while one is consumed)
template <int KT, int VT>
constexpr int pages_per_round() {
  return 2;
}

template <int KT, int VT, int D, bool MQ>
hipError_t launch_typed(const Params& prm, dim3 grid, hipStream_t s) {
  const int nw = MQ ? prm.wg_waves : 1;
  constexpr int CH = pages_per_round<KT, VT>();
  // the variant that also writes the step's new token (one query token)
  if constexpr (!MQ) {
    if (prm.new_k) {
      hipLaunchKernelGGL((decode_chunk_kernel<KT, VT, D, CH, MQ, true>), grid, dim3(64 * nw), 2 * prm.q_slot * nw, s,
                         prm);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_chunk_kernel<KT, VT, D, CH, MQ, false>), grid, dim3(64 * nw), 2 * prm.q_slot * nw, s,
                     prm);
  return hipGetLastError();
}

template <int KT, int D, bool MQ>
hipError_t launch_v(int vt, const Params& prm, dim3 grid, hipStream_t s) {
  switch (vt) {
    case DT_BF16: return launch_typed<KT, DT_BF16, D, MQ>(prm, grid, s);
    case DT_INT8: return launch_typed<KT, DT_INT8, D, MQ>(prm, grid, s);
    case DT_E4M3: return launch_typed<KT, DT_E4M3, D, MQ>(prm, grid, s);
    case DT_E5M2: return launch_typed<KT, DT_E5M2, D, MQ>(prm, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool MQ>
hipError_t launch_kv(int kt, int vt, const Params& prm, dim3 grid, hipStream_t s) {
  if (kt == DT_INT4 || kt == DT_INT4H) {
    if (vt != DT_INT4) return hipErrorInvalidValue;
    return kt == DT_INT4 ? launch_typed<DT_INT4, DT_INT4, D, MQ>(prm, grid, s)
                         : launch_typed<DT_INT4H, DT_INT4, D, MQ>(prm, grid, s);
  }
  switch (kt) {
    case DT_BF16: return launch_v<DT_BF16, D, MQ>(vt, prm, grid, s);
    case DT_INT8: return launch_v<DT_INT8, D, MQ>(vt, prm, grid, s);
    case DT_E4M3: return launch_v<DT_E4M3, D, MQ>(vt, prm, grid, s);
    case DT_E5M2: return launch_v<DT_E5M2, D, MQ>(vt, prm, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace kvq
