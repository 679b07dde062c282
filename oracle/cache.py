"""Oracle paged cache: calibration, write, conversion, gather — TEST INFRASTRUCTURE ONLY.

Layout (the pages speak of "GPU blocks" of KV cache, vLLM PR 4893 L4 table, and
of a paged-cache write, vLLM issue 4025 methods item 2; the layout itself is
this library's reading):
  pages  uint8 [num_blocks][Hkv][block_size][row_bytes]  one array for K, one for V
         row_bytes = 2*D (bf16, little endian), D (int8, e4m3, e5m2), D/2 (int4)
  meta   float32 [num_blocks][Hkv][block_size][2] = (scale, zero_point), int4 only
  slot   = block * block_size + offset; token position p of sequence b lives in
         block_tables[b][p // block_size] at offset p % block_size.

Pins (tests/test_oracle_cache.py): calibration is exact and order-free (token
permutation, chunked running max == one shot, per-tensor == max of per-head);
write/convert agree with row-wise codec calls placed by hand; the paged gather
equals the contiguous token order on a permuted pool.
"""

import numpy as np

from . import codecs

F32 = np.float32
# int4h: INT4 asymmetric of the Hadamard-rotated row (K only; codecs.hadamard_rotate_bf16)
CODE_DTYPES = ("bf16", "int8", "e4m3", "e5m2", "int4", "int4h")
QMAX = {"int8": 127.0, "e4m3": 448.0, "e5m2": 57344.0}


def row_bytes(dtype, D):
    return {"bf16": 2 * D, "int8": D, "e4m3": D, "e5m2": D, "int4": D // 2, "int4h": D // 2}[dtype]


# ---------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------


def calibrate(x_bits, granularity, qmax, absmax_in=None):
    """absmax calibration of a bf16 tensor x [T][Hkv][D].

    The sm86 INT8 summary calibrates per-layer scaling values offline; the
    modelium FP8 page (scale schemes) names per-tensor and per-attention-head
    scales.  Reading:
      absmax = max |x| over the group (whole tensor, or all tokens x D of one KV
               head), NaN ignored; running: absmax = fmax(absmax_in, absmax)
      scale  = fl32(absmax / qmax)  (qmax = 127 int8, 448 e4m3, 57344 e5m2)
      absmax == 0 -> scale 1.0 (the vLLM PR 4893 default scale).
    Returns (absmax float32 [G], scale float32 [G]); G = 1 or Hkv.
    """
    x = np.abs(codecs.bf16_to_f32(x_bits))
    if x.ndim != 3:
        raise ValueError("x must be [T][Hkv][D]")
    T, H, D = x.shape
    if granularity == "per_tensor":
        groups = x.reshape(1, -1) if T else np.zeros((1, 0), F32)
    elif granularity == "per_kv_head":
        groups = x.transpose(1, 0, 2).reshape(H, -1)
    else:
        raise ValueError(granularity)
    if groups.shape[1]:
        a = np.fmax.reduce(groups, axis=1)          # fmax: NaN operands ignored
        a = np.where(np.isnan(a), F32(0), a)        # a group of only NaNs
    else:
        a = np.zeros(groups.shape[0], F32)
    a = a.astype(F32)
    if absmax_in is not None:
        a = np.fmax(np.asarray(absmax_in, F32), a).astype(F32)
    s = np.divide(a, F32(qmax), dtype=F32)
    s = np.where(a == 0, F32(1.0), s).astype(F32)
    return a, s


# ---------------------------------------------------------------------------
# rows -> stored bytes
# ---------------------------------------------------------------------------


def _head_scale(scale, H):
    """Per-head scale vector [H] from None (-> 1.0), [1] or [H]."""
    if scale is None:
        return np.ones(H, F32)
    s = np.asarray(scale, F32).reshape(-1)
    if s.size == 1:
        return np.full(H, s[0], F32)
    if s.size != H:
        raise ValueError("scale must have 1 or Hkv entries")
    return s


def encode_rows(x_bits, dtype, scale=None):
    """Encode bf16 rows x [N][Hkv][D] to stored bytes [N][Hkv][row_bytes].

    Returns (bytes uint8, meta float32 [N][Hkv][2] or None).
    """
    x_bits = np.asarray(x_bits, np.uint16)
    N, H, D = x_bits.shape
    if dtype == "bf16":
        return x_bits.view(np.uint8).reshape(N, H, 2 * D).copy(), None
    if dtype == "int4h":
        x_bits, dtype = codecs.hadamard_rotate_bf16(x_bits), "int4"
    x = codecs.bf16_to_f32(x_bits)
    if dtype == "int4":
        codes, s, zp = codecs.int4_encode_rows(x)
        meta = np.stack([s, zp], axis=-1).astype(F32)
        return codecs.int4_pack(codes), meta
    s = _head_scale(scale, H)[None, :, None]
    if dtype == "int8":
        return codecs.int8_encode(x, s).view(np.uint8), None
    if dtype in ("e4m3", "e5m2"):
        return codecs.fp8_encode(x, s, dtype), None
    raise ValueError(dtype)


def decode_rows(b, dtype, D, scale=None, meta=None):
    """Stored bytes [..., Hkv, row_bytes] -> float32 x_hat [..., Hkv, D]."""
    b = np.asarray(b, np.uint8)
    H = b.shape[-2]
    if dtype == "bf16":
        return codecs.bf16_to_f32(b.view(np.uint16))
    if dtype in ("int4", "int4h"):   # int4h: the rotated row
        codes = codecs.int4_unpack(b)
        return codecs.int4_decode(codes, meta[..., 0], meta[..., 1])
    s = _head_scale(scale, H)[:, None]
    if dtype == "int8":
        return codecs.int8_decode(b.view(np.int8), s)
    return codecs.fp8_decode(b, s, dtype)


# ---------------------------------------------------------------------------
# the paged cache
# ---------------------------------------------------------------------------


class PagedCache:
    """One layer's paged K and V cache in the oracle's representation."""

    def __init__(self, num_blocks, num_kv_heads, head_dim, k_dtype, v_dtype,
                 k_scale=None, v_scale=None, block_size=16, fill=0xFF):
        self.nb, self.H, self.D, self.bs = num_blocks, num_kv_heads, head_dim, block_size
        self.k_dtype, self.v_dtype = k_dtype, v_dtype
        self.k_scale = None if k_scale is None else np.asarray(k_scale, F32).reshape(-1)
        self.v_scale = None if v_scale is None else np.asarray(v_scale, F32).reshape(-1)
        shape = (num_blocks, num_kv_heads, block_size)
        self.k_pages = np.full(shape + (row_bytes(k_dtype, head_dim),), fill, np.uint8)
        self.v_pages = np.full(shape + (row_bytes(v_dtype, head_dim),), fill, np.uint8)
        self.k_meta = np.full(shape + (2,), np.nan, F32) if k_dtype in ("int4", "int4h") else None
        self.v_meta = np.full(shape + (2,), np.nan, F32) if v_dtype in ("int4", "int4h") else None

    # -- write -------------------------------------------------------------
    def write(self, k_bits, v_bits, slot_mapping):
        """Encode token rows and store them at their slots.

        vLLM issue 4025, methods item 2 (store 4-bit KV in the paged-cache
        write), read for every element format: row i of k_bits / v_bits
        [T][Hkv][D] is encoded and stored at slot_mapping[i] = block *
        block_size + offset.  A negative slot is skipped; a slot beyond the pool
        is skipped and counted.  Returns the count of out-of-range slots.
        """
        slots = np.asarray(slot_mapping, np.int64)
        ok = (slots >= 0) & (slots < self.nb * self.bs)
        bad = int(np.sum(slots >= self.nb * self.bs))
        idx = np.nonzero(ok)[0]
        if idx.size == 0:
            return bad
        blk, off = slots[idx] // self.bs, slots[idx] % self.bs
        for which, bits in (("k", k_bits), ("v", v_bits)):
            dtype = getattr(self, which + "_dtype")
            b, meta = encode_rows(np.asarray(bits, np.uint16)[idx], dtype, getattr(self, which + "_scale"))
            getattr(self, which + "_pages")[blk, :, off, :] = b
            if meta is not None:
                getattr(self, which + "_meta")[blk, :, off, :] = meta
        return bad

    # -- convert -----------------------------------------------------------
    def convert_from_bf16(self, k_src_bits, v_src_bits, first_block, n_blocks):
        """vLLM issue 4025, methods item 1: convert an existing bf16 paged cache.

        k_src_bits / v_src_bits are bf16 pages [num_blocks][Hkv][bs][D] with the
        same geometry; every slot of blocks [first_block, first_block+n_blocks)
        is encoded into this cache (with the row's own scale / zero point for
        int4, the cache's scales otherwise).
        """
        sl = slice(first_block, first_block + n_blocks)
        for which, src in (("k", k_src_bits), ("v", v_src_bits)):
            dtype = getattr(self, which + "_dtype")
            rows = np.asarray(src, np.uint16)[sl]              # [n][H][bs][D]
            r = rows.transpose(0, 2, 1, 3).reshape(-1, self.H, self.D)
            b, meta = encode_rows(r, dtype, getattr(self, which + "_scale"))
            n = rows.shape[0]
            getattr(self, which + "_pages")[sl] = b.reshape(n, self.bs, self.H, -1).transpose(0, 2, 1, 3)
            if meta is not None:
                getattr(self, which + "_meta")[sl] = meta.reshape(n, self.bs, self.H, 2).transpose(0, 2, 1, 3)

    # -- gather ------------------------------------------------------------
    def gather(self, block_table_row, L, which, heads=None):
        """Dequantised rows of one sequence's first L positions: float32 [L][Hkv'][D].

        Position p lives in block_table_row[p // bs] at offset p % bs.  Unused
        slots are never read.
        """
        p = np.arange(L)
        blk = np.asarray(block_table_row, np.int64)[p // self.bs]
        off = p % self.bs
        hs = np.arange(self.H) if heads is None else np.asarray(heads)
        pages = getattr(self, which + "_pages")
        b = pages[blk[:, None], hs[None, :], off[:, None], :]        # [L][h][rb]
        dtype = getattr(self, which + "_dtype")
        meta = getattr(self, which + "_meta")
        m = None if meta is None else meta[blk[:, None], hs[None, :], off[:, None], :]
        sc = getattr(self, which + "_scale")
        if sc is not None and sc.size > 1:
            sc = sc[hs]
        return decode_rows(b, dtype, self.D, sc, m)

    def kv_bytes_per_token_head(self):
        return codecs.kv_bytes_per_token_head(self.k_dtype, self.v_dtype, self.D)
