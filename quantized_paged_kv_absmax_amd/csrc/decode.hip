// decode.hip — paged-attention decode over the quantised cache (vLLM issue 4025,
// methods item 3: read the stored codes, convert them to 16-bit, compute; vLLM
// PR 4893: decode runs a paged-attention kernel), plus the split-KV reduce.
//
// Work unit: one workgroup per (partition, KV head, sequence) serves all g = Hq/Hkv
// query heads of that KV head, so each K/V page is read from HBM exactly once.
// NW waves split the partition's pages; each wave takes CH consecutive pages per
// round and keeps its own online-softmax state, and the waves are merged through
// LDS at the end.
//
// Per page (16 tokens) and wave:
//   K: lane l loads token l%16, a quarter (l/16) of the row: D/4 elements.  The
//      codes are turned into exact fp16 (bf16 for a bf16 cache) MFMA operands:
//        int8  byte ^ 0x80 placed in an fp16 with exponent 2^10, minus 1152
//        int4  nibble in the same way, minus 1024
//        e4m3  v_cvt_scalef32_pk_f16_fp8 (scale 1)
//        e5m2  the byte is the high byte of an fp16
//      S^T[token][head] = K . Q^T with v_mfma_f32_16x16x32_{f16,bf16}, D/32 of them.
//      Lane l then holds the logits of head l%16 for tokens 4(l/16)+r, r=0..3,
//      which is exactly the A-operand layout of the 16x16x16 PV product.
//   V: lane l loads rows 4(l/16)..4(l/16)+3 at columns [NE*(l%16), NE*(l%16)+NE)
//      (NE = D/16) and transposes that 4 x NE block in registers with byte
//      permutes, so that for every column it holds the 4 tokens the B operand of
//      v_mfma_f32_16x16x16 needs.  NE MFMAs per page accumulate O[head][d].
// Scales: per-tensor / per-head scales multiply the float32 logits (K) and the
// final output (V).  INT4 uses, per token t with (s_t, zp_t):
//   logit_t = s_t * (sum_c q_c code_c - zp_t * sum_c q_c)
//   O       = sum_t (p_t s_t) code_t - sum_t (p_t s_t) zp_t
// Softmax runs in base 2 (log2 e folded into the logit scale).
// Masking: positions >= seq_len get logit -inf and their V operand is zeroed
// (an unused slot may hold a NaN code; 0 * NaN would leak).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNW = 4;  // waves per workgroup

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
  int num_blocks, Hkv, Hq, g;
  int max_seq_len;
  float sm_log2;  // softmax_scale * log2(e)
  int partition;
  int num_partitions;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int out_f32;
  void* out;
  int32_t* err;
};

template <int DT, int D>
struct Geo {
  static constexpr int kRowBytes = (DT == DT_BF16) ? 2 * D : (DT == DT_INT4) ? D / 2 : D;
  static constexpr int kKLaneBytes = kRowBytes / 4;   // K bytes per lane per page
  static constexpr int kKDw = kKLaneBytes / 4;        // ... in dwords
  static constexpr int kNE = D / 16;                  // V columns per lane
  static constexpr int kVRowBytes = kRowBytes / 16;   // V bytes per lane per row
  static constexpr int kVDw = (kVRowBytes + 3) / 4;   // ... in dwords (int4 D=64: 2 bytes -> 1)
};

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
// loads
// ---------------------------------------------------------------------------

template <int NDW>
__device__ __forceinline__ void load_dw(uint32_t (&r)[NDW], const uint8_t* ptr) {
  if constexpr (NDW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NDW / 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(ptr + 16 * i);
      r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
    }
  } else if constexpr (NDW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(ptr);
    r[0] = v.x; r[1] = v.y;
  } else {
    static_assert(NDW == 1, "unsupported load width");
    r[0] = *reinterpret_cast<const uint32_t*>(ptr);
  }
}

// V bytes of one row for this lane: VRB bytes (2, 4, 8 or 16)
template <int DT, int D, int N>
__device__ __forceinline__ void load_v_row(uint32_t (&r)[N], const uint8_t* ptr) {
  constexpr int VRB = Geo<DT, D>::kVRowBytes;
  static_assert(N == Geo<DT, D>::kVDw, "V row width");
  if constexpr (VRB == 2) {
    r[0] = *reinterpret_cast<const uint16_t*>(ptr);
  } else {
    load_dw<N>(r, ptr);
  }
}

// ---------------------------------------------------------------------------
// K codes -> MFMA operand (8 fp16 / bf16 values = 4 dwords) for k-step s
// ---------------------------------------------------------------------------

template <int DT, int D, int N>
__device__ __forceinline__ u32x4 k_operand(const uint32_t (&kw)[N], int s) {
  static_assert(N == Geo<DT, D>::kKDw, "K lane width");
  u32x4 o;
  if constexpr (DT == DT_BF16) {
    o[0] = kw[4 * s]; o[1] = kw[4 * s + 1]; o[2] = kw[4 * s + 2]; o[3] = kw[4 * s + 3];
  } else if constexpr (DT == DT_INT8) {
    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t a = kw[2 * s] ^ 0x80808080u, b = kw[2 * s + 1] ^ 0x80808080u;
    o[0] = pk_add_f16(perm(kMagic64, a, kSelLo), bias);
    o[1] = pk_add_f16(perm(kMagic64, a, kSelHi), bias);
    o[2] = pk_add_f16(perm(kMagic64, b, kSelLo), bias);
    o[3] = pk_add_f16(perm(kMagic64, b, kSelHi), bias);
  } else if constexpr (DT == DT_E4M3) {
    o[0] = e4m3x2_to_f16x2<false>(kw[2 * s]);
    o[1] = e4m3x2_to_f16x2<true>(kw[2 * s]);
    o[2] = e4m3x2_to_f16x2<false>(kw[2 * s + 1]);
    o[3] = e4m3x2_to_f16x2<true>(kw[2 * s + 1]);
  } else if constexpr (DT == DT_E5M2) {
    o[0] = perm(0u, kw[2 * s], 0x010C000Cu);
    o[1] = perm(0u, kw[2 * s], 0x030C020Cu);
    o[2] = perm(0u, kw[2 * s + 1], 0x010C000Cu);
    o[3] = perm(0u, kw[2 * s + 1], 0x030C020Cu);
  } else {  // INT4: element order (even d of bytes 0..3, then odd d of bytes 0..3)
    const f16x2 bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const uint32_t w = kw[s];
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    o[0] = pk_add_f16(perm(kMagic64, lo, kSelLo), bias);
    o[1] = pk_add_f16(perm(kMagic64, lo, kSelHi), bias);
    o[2] = pk_add_f16(perm(kMagic64, hi, kSelLo), bias);
    o[3] = pk_add_f16(perm(kMagic64, hi, kSelHi), bias);
  }
  return o;
}

// head-dim index of operand element e of k-step s for lane group qg (must match k_operand)
template <int DT, int D>
__device__ __forceinline__ int k_dim(int qg, int s, int e) {
  const int base = (D / 4) * qg + 8 * s;
  if constexpr (DT == DT_INT4) return base + ((e < 4) ? 2 * e : 2 * (e - 4) + 1);
  return base + e;
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
          const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
          i0 ^= 0x80808080u;
          i1 ^= 0x80808080u;
          ob[4 * j + 0][pr] = pk_add_f16(perm(kMagic64, i0, kSelLo), bias);
          ob[4 * j + 1][pr] = pk_add_f16(perm(kMagic64, i0, kSelHi), bias);
          ob[4 * j + 2][pr] = pk_add_f16(perm(kMagic64, i1, kSelLo), bias);
          ob[4 * j + 3][pr] = pk_add_f16(perm(kMagic64, i1, kSelHi), bias);
        } else {
          ob[4 * j + 0][pr] = e4m3x2_to_f16x2<false>(i0);
          ob[4 * j + 1][pr] = e4m3x2_to_f16x2<true>(i0);
          ob[4 * j + 2][pr] = e4m3x2_to_f16x2<false>(i1);
          ob[4 * j + 3][pr] = e4m3x2_to_f16x2<true>(i1);
        }
      }
    }
  } else {  // INT4: byte k of a row holds columns 2k (low nibble), 2k+1 (high nibble)
    const f16x2 bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const uint32_t a = vr[2 * pr][0], b = vr[2 * pr + 1][0];
#pragma unroll
      for (int hn = 0; hn < 2; ++hn) {
        const uint32_t la = hn ? ((a >> 4) & 0x0F0F0F0Fu) : (a & 0x0F0F0F0Fu);
        const uint32_t lb = hn ? ((b >> 4) & 0x0F0F0F0Fu) : (b & 0x0F0F0F0Fu);
        const uint32_t i0 = perm(lb, la, 0x05010400u);   // bytes 0,1 of both rows
        ob[0 + hn][pr] = pk_add_f16(perm(kMagic64, i0, kSelLo), bias);   // column 2*0 + hn
        ob[2 + hn][pr] = pk_add_f16(perm(kMagic64, i0, kSelHi), bias);   // column 2*1 + hn
        if constexpr (NE == 8) {
          const uint32_t i1 = perm(lb, la, 0x07030602u); // bytes 2,3
          ob[4 + hn][pr] = pk_add_f16(perm(kMagic64, i1, kSelLo), bias);
          ob[6 + hn][pr] = pk_add_f16(perm(kMagic64, i1, kSelHi), bias);
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

__device__ __forceinline__ uint32_t pack2(float a, float b, bool bf) {
  if (bf) return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
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

// ---------------------------------------------------------------------------
// the partition kernel
// ---------------------------------------------------------------------------

template <int KT, int VT, int D, int CH>
__global__ __launch_bounds__(kNW * 64) void decode_partition_kernel(Params p) {
  using KG = Geo<KT, D>;
  using VG = Geo<VT, D>;
  constexpr int NS = D / 32;       // QK k-steps
  constexpr int NE = VG::kNE;      // PV n-tiles
  constexpr bool KBF = (KT == DT_BF16);
  constexpr bool VBF = (VT == DT_BF16);

  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, qg = lane >> 4;
  const int g = p.g;

  const int L = clamp_len(p, b, part == 0 && kvh == 0 && threadIdx.x == 0);
  const int tok0 = part * p.partition;
  const bool single = (p.num_partitions == 1);

  if (L <= 0 || tok0 >= L) {
    if (single && L <= 0) {
      // zero output rows for this KV head's query heads
      for (int i = threadIdx.x; i < g * D; i += kNW * 64) {
        const size_t o = ((size_t)b * p.Hq + (size_t)kvh * g + i / D) * D + (i % D);
        if (p.out_f32) reinterpret_cast<float*>(p.out)[o] = 0.0f;
        else reinterpret_cast<uint16_t*>(p.out)[o] = 0;
      }
    }
    return;
  }
  const int tok_end = min(L, tok0 + p.partition);
  const int n_pages = (tok_end - tok0 + 15) >> 4;
  const int pg0 = tok0 >> 4;

  // ---- query operand: head c (zero if c >= g), k-dim order of the K operand ----
  u32x4 qop[NS];
  float qsum = 0.0f;
  {
    const bool hv = c < g;
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + (size_t)kvh * g + (hv ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int base = (D / 4) * qg + 8 * s;
      const uint4 raw = hv ? *reinterpret_cast<const uint4*>(qrow + base) : make_uint4(0, 0, 0, 0);
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
      float qf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[2 * i] = bf16_bits_to_f32(rw[i] & 0xffffu);
        qf[2 * i + 1] = bf16_bits_to_f32(rw[i] >> 16);
      }
      float qe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qe[e] = qf[k_dim<KT, D>(qg, s, e) - base];
      if constexpr (KBF) {
        qop[s] = u32x4{rw[0], rw[1], rw[2], rw[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(qe[2 * i], qe[2 * i + 1]));
          qop[s][i] = __builtin_bit_cast(uint32_t, h2);
          if constexpr (KT == DT_INT4) qsum += (float)h2[0] + (float)h2[1];
        }
      }
    }
    if constexpr (KT == DT_INT4) {
      qsum += shfl_xor_f(qsum, 16);
      qsum += shfl_xor_f(qsum, 32);
    }
  }

  // logit scale (base 2) for per-tensor / per-head K scales; INT4 scales per token
  float kfac = p.sm_log2;
  if constexpr (KT == DT_INT8 || KT == DT_E4M3 || KT == DT_E5M2) {
    if (p.k_scale) kfac *= p.k_scale[p.k_scale_per_head ? kvh : 0];
  }

  // ---- wave state ----
  float m_run = -INFINITY;   // running max, head c (uniform over qg)
  float l_run = 0.0f;        // per-lane partial softmax sum
  float corr_run = 0.0f;     // INT4 V: per-lane partial of sum (p s) zp
  f32x4 oacc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = p.block_tables + (size_t)b * p.max_blocks_per_seq;
  const size_t head_stride = 16;  // rows per (block, head)

  for (int r0 = 0; r0 < n_pages; r0 += kNW * CH) {
    const int wp0 = r0 + w * CH;
    if (wp0 >= n_pages) continue;           // no pages for this wave this round
    const int np = min(CH, n_pages - wp0);

    int blk[CH];
    bool pok[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      int bb = 0;
      bool ok = false;
      if (i < np) {
        bb = bt[pg0 + wp0 + i];
        ok = (bb >= 0) && (bb < p.num_blocks);
        if (!ok) {
          if (p.err && lane == 0) atomicAdd(p.err, 1);
          bb = 0;
        }
      }
      blk[i] = bb;
      pok[i] = ok;
    }

    // ---- issue all loads of the round ----
    uint32_t kw[CH][KG::kKDw];
    uint32_t vw[CH][4][VG::kVDw];
    float4 kmeta[CH][2], vmeta[CH][2];   // INT4: (s, zp) of tokens 4qg..4qg+3
    // a page with a bad block id issues no load; its data stay zero and its
    // tokens are masked below
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < np) {
        if (pok[i]) {
          const size_t rowbase = ((size_t)blk[i] * p.Hkv + kvh) * head_stride;
          load_dw<KG::kKDw>(kw[i], p.k_pages + (rowbase + c) * KG::kRowBytes + qg * KG::kKLaneBytes);
          if constexpr (KT == DT_INT4) {
            const float4* mp = reinterpret_cast<const float4*>(p.k_meta + (rowbase + 4 * qg) * 2);
            kmeta[i][0] = mp[0];
            kmeta[i][1] = mp[1];
          }
        } else {
#pragma unroll
          for (int k = 0; k < KG::kKDw; ++k) kw[i][k] = 0u;
          kmeta[i][0] = kmeta[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < np) {
        if (pok[i]) {
          const size_t rowbase = ((size_t)blk[i] * p.Hkv + kvh) * head_stride;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            load_v_row<VT, D>(vw[i][r], p.v_pages + (rowbase + 4 * qg + r) * VG::kRowBytes + c * VG::kVRowBytes);
          if constexpr (VT == DT_INT4) {
            const float4* mp = reinterpret_cast<const float4*>(p.v_meta + (rowbase + 4 * qg) * 2);
            vmeta[i][0] = mp[0];
            vmeta[i][1] = mp[1];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < VG::kVDw; ++k) vw[i][r][k] = 0u;
          vmeta[i][0] = vmeta[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }

    // ---- QK: logits of head c for tokens 4qg+r of each page ----
    float sl[CH][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < np) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) acc = mfma_qk<KBF>(k_operand<KT, D>(kw[i], s), qop[s], acc);
        const int tbase = tok0 + (wp0 + i) * 16 + 4 * qg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z;
          if constexpr (KT == DT_INT4) {
            const float ks = (r < 2) ? ((r == 0) ? kmeta[i][0].x : kmeta[i][0].z)
                                     : ((r == 2) ? kmeta[i][1].x : kmeta[i][1].z);
            const float kz = (r < 2) ? ((r == 0) ? kmeta[i][0].y : kmeta[i][0].w)
                                     : ((r == 2) ? kmeta[i][1].y : kmeta[i][1].w);
            z = (ks * p.sm_log2) * (acc[r] - kz * qsum);
          } else {
            z = acc[r] * kfac;
          }
          const bool valid = pok[i] && (tbase + r < tok_end);
          z = valid ? z : -INFINITY;
          sl[i][r] = z;
          cmax = fmaxf(cmax, z);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) sl[i][r] = -INFINITY;
      }
    }
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 16));
    cmax = fmaxf(cmax, shfl_xor_f(cmax, 32));

    // ---- online softmax update ----
    const float m_new = fmaxf(m_run, cmax);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const float msub = any ? m_new : 0.0f;
    m_run = m_new;
    l_run *= alpha;
    corr_run *= alpha;
    {
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = shfl_f(alpha, 4 * qg + r);   // alpha of head 4qg+r
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[e][r] *= ar[r];
    }

    // ---- PV ----
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < np) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(sl[i][r] - msub);     // -inf -> 0
          l_run += pr[r];
        }
        u32x2 aop;
        if constexpr (VT == DT_INT4) {
          const float vs[4] = {vmeta[i][0].x, vmeta[i][0].z, vmeta[i][1].x, vmeta[i][1].z};
          const float vz[4] = {vmeta[i][0].y, vmeta[i][0].w, vmeta[i][1].y, vmeta[i][1].w};
          float ps[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ps[r] = (pr[r] != 0.0f) ? pr[r] * vs[r] : 0.0f;
          aop[0] = pack2(ps[0], ps[1], false);
          aop[1] = pack2(ps[2], ps[3], false);
          // correction uses the rounded operand values the MFMA sees
          const float r0 = unpack_lo(aop[0], false), r1 = unpack_hi(aop[0], false);
          const float r2 = unpack_lo(aop[1], false), r3 = unpack_hi(aop[1], false);
          corr_run += (r0 != 0.f ? r0 * vz[0] : 0.f) + (r1 != 0.f ? r1 * vz[1] : 0.f) +
                      (r2 != 0.f ? r2 * vz[2] : 0.f) + (r3 != 0.f ? r3 * vz[3] : 0.f);
        } else {
          aop[0] = pack2(pr[0], pr[1], VBF);
          aop[1] = pack2(pr[2], pr[3], VBF);
        }
        if (c >= g) aop = u32x2{0u, 0u};

        u32x2 vop[NE];
        v_operands<VT, D>(vw[i], vop);
        // zero V operands of tokens that are not valid (tail of the last page, bad block)
        const int tbase = tok0 + (wp0 + i) * 16 + 4 * qg;
        const bool full = pok[i] && (tok0 + (wp0 + i) * 16 + 16 <= tok_end);
        if (!full) {
          uint32_t m01 = 0, m23 = 0;
          if (pok[i]) {
            m01 = ((tbase + 0 < tok_end) ? 0x0000ffffu : 0u) | ((tbase + 1 < tok_end) ? 0xffff0000u : 0u);
            m23 = ((tbase + 2 < tok_end) ? 0x0000ffffu : 0u) | ((tbase + 3 < tok_end) ? 0xffff0000u : 0u);
          }
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            vop[e][0] &= m01;
            vop[e][1] &= m23;
          }
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) oacc[e] = mfma_pv<VBF>(aop, vop[e], oacc[e]);
      }
    }
  }

  // ---- finish the wave: full sums over the lane groups ----
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if constexpr (VT == DT_INT4) {
    corr_run += shfl_xor_f(corr_run, 16);
    corr_run += shfl_xor_f(corr_run, 32);
  }

  // ---- merge the waves through LDS ----
  __shared__ float s_m[kNW][16], s_l[kNW][16], s_c[kNW][16];
  __shared__ float s_o[kNW][16][D];
  if (qg == 0) {
    s_m[w][c] = m_run;
    s_l[w][c] = l_run;
    s_c[w][c] = corr_run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * qg + r;
    if (h < g) {
      float M = s_m[0][h];
#pragma unroll
      for (int ww = 1; ww < kNW; ++ww) M = fmaxf(M, s_m[ww][h]);
      const float mw = s_m[w][h];
      const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
      for (int e = 0; e < NE; ++e) s_o[w][h][NE * c + e] = f * oacc[e][r];
    }
  }
  __syncthreads();

  float vfac = 1.0f;
  if constexpr (VT == DT_INT8 || VT == DT_E4M3 || VT == DT_E5M2) {
    if (p.v_scale) vfac = p.v_scale[p.v_scale_per_head ? kvh : 0];
  }
  for (int i = threadIdx.x; i < g * D; i += kNW * 64) {
    const int h = i / D, d = i % D;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kNW; ++ww) M = fmaxf(M, s_m[ww][h]);
    float num = 0.f, den = 0.f, cor = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float mw = s_m[ww][h];
      const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      num += s_o[ww][h][d];
      den += f * s_l[ww][h];
      if constexpr (VT == DT_INT4) cor += f * s_c[ww][h];
    }
    num = (num - cor) * vfac;
    const int hq = kvh * g + h;
    if (single) {
      const float o = num / den;
      const size_t oi = ((size_t)b * p.Hq + hq) * D + d;
      if (p.out_f32) reinterpret_cast<float*>(p.out)[oi] = o;
      else reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16_bits(o);
    } else {
      const size_t row = (size_t)b * p.Hq + hq;
      p.ws_o[(row * p.num_partitions + part) * D + d] = num;
      if (d == 0) {
        p.ws_m[row * p.num_partitions + part] = M;
        p.ws_l[row * p.num_partitions + part] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split-KV reduce: o = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j
// ---------------------------------------------------------------------------

constexpr int kRedThreads = 256;

template <int D>
__global__ __launch_bounds__(kRedThreads) void decode_reduce_kernel(Params p) {
  constexpr int LPG = D / 4;                  // lanes per group, 4 columns each
  constexpr int NG = kRedThreads / LPG;       // groups
  const int hq = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(p, b, false);
  const size_t orow = ((size_t)b * p.Hq + hq) * D;
  if (L <= 0) {
    for (int d = threadIdx.x; d < D; d += kRedThreads) {
      if (p.out_f32) reinterpret_cast<float*>(p.out)[orow + d] = 0.0f;
      else reinterpret_cast<uint16_t*>(p.out)[orow + d] = 0;
    }
    return;
  }
  const int P = (L + p.partition - 1) / p.partition;
  const size_t row = (size_t)b * p.Hq + hq;
  const float* m = p.ws_m + row * p.num_partitions;
  const float* l = p.ws_l + row * p.num_partitions;
  const float* o = p.ws_o + row * p.num_partitions * D;

  __shared__ float s_red[kRedThreads / 64];
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < P; j += kRedThreads) mx = fmaxf(mx, m[j]);
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) mx = fmaxf(mx, __shfl_xor(mx, k, 64));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int i = 1; i < kRedThreads / 64; ++i) M = fmaxf(M, s_red[i]);

  const int grp = threadIdx.x / LPG, ln = threadIdx.x % LPG;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int j = grp; j < P; j += NG) {
    const float f = __builtin_amdgcn_exp2f(m[j] - M);
    const float4 v = *reinterpret_cast<const float4*>(o + (size_t)j * D + 4 * ln);
    acc.x += f * v.x; acc.y += f * v.y; acc.z += f * v.z; acc.w += f * v.w;
    den += f * l[j];
  }
  __shared__ float4 s_acc[NG][LPG];
  __shared__ float s_den[NG];
  s_acc[grp][ln] = acc;
  if (ln == 0) s_den[grp] = den;
  __syncthreads();
  if (threadIdx.x < LPG) {
    float4 a = s_acc[0][threadIdx.x];
    float dd = s_den[0];
#pragma unroll
    for (int gi = 1; gi < NG; ++gi) {
      const float4 v = s_acc[gi][threadIdx.x];
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      dd += s_den[gi];
    }
    const float r[4] = {a.x / dd, a.y / dd, a.z / dd, a.w / dd};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t oi = orow + 4 * threadIdx.x + k;
      if (p.out_f32) reinterpret_cast<float*>(p.out)[oi] = r[k];
      else reinterpret_cast<uint16_t*>(p.out)[oi] = f32_to_bf16_bits(r[k]);
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

template <int KT, int VT>
constexpr int pages_per_round() {
  return (KT == DT_BF16 || VT == DT_BF16 || KT == DT_INT4 || VT == DT_INT4) ? 4 : 8;
}

template <int KT, int VT, int D>
hipError_t launch_typed(const Params& prm, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_partition_kernel<KT, VT, D, pages_per_round<KT, VT>()>), grid, dim3(kNW * 64), 0, s,
                     prm);
  return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_v(int vt, const Params& prm, dim3 grid, hipStream_t s) {
  switch (vt) {
    case DT_BF16: return launch_typed<KT, DT_BF16, D>(prm, grid, s);
    case DT_INT8: return launch_typed<KT, DT_INT8, D>(prm, grid, s);
    case DT_E4M3: return launch_typed<KT, DT_E4M3, D>(prm, grid, s);
    case DT_E5M2: return launch_typed<KT, DT_E5M2, D>(prm, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_kv(int kt, int vt, const Params& prm, dim3 grid, hipStream_t s) {
  if (kt == DT_INT4) {
    if (vt != DT_INT4) return hipErrorInvalidValue;
    return launch_typed<DT_INT4, DT_INT4, D>(prm, grid, s);
  }
  switch (kt) {
    case DT_BF16: return launch_v<DT_BF16, D>(vt, prm, grid, s);
    case DT_INT8: return launch_v<DT_INT8, D>(vt, prm, grid, s);
    case DT_E4M3: return launch_v<DT_E4M3, D>(vt, prm, grid, s);
    case DT_E5M2: return launch_v<DT_E5M2, D>(vt, prm, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int kt, int vt, int D) {
  if (D != 64 && D != 128) return false;
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
  prm.partition = a.partition;
  prm.num_partitions = a.num_partitions;
  prm.ws_m = a.ws_m;
  prm.ws_l = a.ws_l;
  prm.ws_o = a.ws_o;
  prm.out_f32 = a.out_f32;
  prm.out = a.out;
  prm.err = a.err;

  dim3 grid(a.num_partitions, c.num_kv_heads, a.batch);
  hipError_t e = (c.head_dim == 128) ? launch_kv<128>(c.k_dtype, c.v_dtype, prm, grid, s)
                                     : launch_kv<64>(c.k_dtype, c.v_dtype, prm, grid, s);
  if (e != hipSuccess || a.num_partitions == 1) return e;
  dim3 rgrid(a.num_q_heads, a.batch);
  if (c.head_dim == 128)
    hipLaunchKernelGGL(decode_reduce_kernel<128>, rgrid, dim3(kRedThreads), 0, s, prm);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<64>, rgrid, dim3(kRedThreads), 0, s, prm);
  return hipGetLastError();
}

}  // namespace kvq
