"""Python binding of libkvq with the C names; torch tensors supply device memory
and the current HIP stream.  Every step of the work runs in the HIP kernels.

    cache = PagedKVCache(num_blocks, num_kv_heads, head_dim, "int8", "int8",
                         k_gran="per_tensor", v_gran="per_tensor", device="cuda")
    kvq_calibrate_scales(k_bf16, "per_tensor", "int8", cache.k_absmax, cache.k_scale)
    kvq_cache_write(cache, k_new, v_new, slot_mapping)
    out = kvq_paged_attention_decode(cache, q, block_tables, seq_lens, max_seq_len, scale)
"""

import ctypes

import torch

from . import _lib
from ._lib import DTYPES, GRANULARITIES, check

_TORCH_BYTES = torch.uint8


def _dt(x):
    return DTYPES[x] if isinstance(x, str) else int(x)


def _gr(x):
    return GRANULARITIES[x] if isinstance(x, str) else int(x)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def row_bytes(dtype, head_dim):
    d = _dt(dtype)
    return {_lib.BF16: 2 * head_dim, _lib.INT8: head_dim, _lib.FP8_E4M3: head_dim, _lib.FP8_E5M2: head_dim,
            _lib.INT4_ASYM: head_dim // 2}[d]


class PagedKVCache:
    """One layer's paged K/V cache in device memory, plus its scales / metadata.

    pages: uint8 [num_blocks][num_kv_heads][block_size][row_bytes]; INT8/FP8 scales
    float32 [1] (per_tensor) or [num_kv_heads] (per_kv_head), initialised to 1.0
    (the default scale when none is calibrated); INT4 metadata float32
    [num_blocks][num_kv_heads][block_size][2].
    """

    def __init__(self, num_blocks, num_kv_heads, head_dim, k_dtype, v_dtype, k_gran="per_tensor",
                 v_gran="per_tensor", device="cuda", block_size=16, fill=0xFF):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size = num_blocks, num_kv_heads, head_dim, block_size
        self.k_dtype, self.v_dtype = _dt(k_dtype), _dt(v_dtype)
        self.k_gran = _lib.PER_TOKEN_HEAD if self.k_dtype == _lib.INT4_ASYM else _gr(k_gran)
        self.v_gran = _lib.PER_TOKEN_HEAD if self.v_dtype == _lib.INT4_ASYM else _gr(v_gran)
        shp = (num_blocks, num_kv_heads, block_size)
        self.k_pages = torch.full(shp + (row_bytes(self.k_dtype, head_dim),), fill, dtype=torch.uint8, device=device)
        self.v_pages = torch.full(shp + (row_bytes(self.v_dtype, head_dim),), fill, dtype=torch.uint8, device=device)
        g = lambda gr: num_kv_heads if gr == _lib.PER_KV_HEAD else 1
        self.k_scale = torch.ones(g(self.k_gran), dtype=torch.float32, device=device)
        self.v_scale = torch.ones(g(self.v_gran), dtype=torch.float32, device=device)
        self.k_absmax = torch.zeros_like(self.k_scale)
        self.v_absmax = torch.zeros_like(self.v_scale)
        meta = lambda dt: (torch.full(shp + (2,), float("nan"), dtype=torch.float32, device=device)
                           if dt == _lib.INT4_ASYM else None)
        self.k_meta, self.v_meta = meta(self.k_dtype), meta(self.v_dtype)

    def struct(self, k_pages=None, v_pages=None):
        """The C kvq_cache describing this cache (optionally over other page buffers
        of the same shape, e.g. a rotating copy)."""
        kp = self.k_pages if k_pages is None else k_pages
        vp = self.v_pages if v_pages is None else v_pages
        s = _lib.KvqCacheStruct()
        s.k_dtype, s.v_dtype, s.k_gran, s.v_gran = self.k_dtype, self.v_dtype, self.k_gran, self.v_gran
        s.num_blocks, s.block_size = self.num_blocks, self.block_size
        s.num_kv_heads, s.head_dim = self.num_kv_heads, self.head_dim
        s.k_pages, s.v_pages = kp.data_ptr(), vp.data_ptr()
        s.k_scale = self.k_scale.data_ptr()
        s.v_scale = self.v_scale.data_ptr()
        s.k_meta = None if self.k_meta is None else self.k_meta.data_ptr()
        s.v_meta = None if self.v_meta is None else self.v_meta.data_ptr()
        return s


def kvq_calibrate_scales(x, granularity, target_dtype, absmax_inout, scale_out, stream=None):
    """absmax calibration of bf16 x [T][Hkv][D] into absmax_inout / scale_out (float32)."""
    _need(x, torch.bfloat16, "x")
    T, H, D = x.shape
    st = _lib.load().kvq_calibrate_scales(_ptr(x), T, H, D, _gr(granularity), _dt(target_dtype),
                                          _ptr(absmax_inout), _ptr(scale_out), _stream(stream))
    check(st, "kvq_calibrate_scales")


def kvq_cache_write(cache, k_new, v_new, slot_mapping, err_count=None, stream=None, struct=None):
    """Encode bf16 rows k_new / v_new [T][Hkv][D] into the pages at slot_mapping (int64 [T])."""
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(slot_mapping, torch.int64, "slot_mapping")
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_cache_write(ctypes.byref(s), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                     k_new.shape[0], _ptr(err_count), _stream(stream))
    check(st, "kvq_cache_write")


def kvq_convert_cache(cache, k_src, v_src, first_block=0, num_blocks=None, stream=None):
    """Convert bf16 pages [num_blocks][Hkv][16][D] into the cache's format."""
    _need(k_src, torch.bfloat16, "k_src")
    _need(v_src, torch.bfloat16, "v_src")
    n = cache.num_blocks - first_block if num_blocks is None else num_blocks
    s = cache.struct()
    st = _lib.load().kvq_convert_cache(ctypes.byref(s), _ptr(k_src), _ptr(v_src), first_block, n, _stream(stream))
    check(st, "kvq_convert_cache")


def kvq_verify_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition=0):
    return int(_lib.load().kvq_verify_workspace_size(batch, n_q, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                     partition))


def kvq_paged_attention_verify(cache, q, n_q, block_tables, seq_lens, max_seq_len, softmax_scale, partition=0,
                               workspace=None, out_dtype="bf16", out=None, err_count=None, stream=None,
                               struct=None):
    """n_q query tokens per sequence, causally: q bf16 [B * n_q][Hq][D] -> out [B * n_q][Hq][D].

    Row b * n_q + i is sequence b's token at position seq_lens[b] - n_q + i; it
    attends to cache positions up to its own.  Arguments otherwise as
    kvq_paged_attention_decode.
    """
    _need(q, torch.bfloat16, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_lens, torch.int32, "seq_lens")
    T, Hq, D = q.shape
    B = seq_lens.shape[0]
    if T != B * n_q:
        raise ValueError(f"q has {T} rows, expected batch * n_q = {B * n_q}")
    odt = _dt(out_dtype)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32 if odt == _lib.F32 else torch.bfloat16, device=q.device)
    need = kvq_verify_workspace_size(B, n_q, Hq, cache.num_kv_heads, D, max_seq_len, partition)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_paged_attention_verify(
        ctypes.byref(s), _ptr(q), int(n_q), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B,
        int(max_seq_len), Hq, float(softmax_scale), int(partition), _ptr(workspace), ws_bytes, odt, _ptr(out),
        _ptr(err_count), _stream(stream))
    check(st, "kvq_paged_attention_verify")
    return out


def kvq_cache_block_bytes(k_dtype, v_dtype, num_kv_heads, head_dim, block_size=16):
    """Bytes of one block of one layer's cache (K + V rows, INT4 metadata); 0 if unsupported."""
    return int(_lib.load().kvq_cache_block_bytes(_dt(k_dtype), _dt(v_dtype), num_kv_heads, head_dim, block_size))


def kvq_blocks_in_budget(budget_bytes, k_dtype, v_dtype, num_kv_heads, head_dim, num_layers, block_size=16):
    """Whole blocks of num_layers layers that fit in budget_bytes; -1 for invalid arguments."""
    return int(_lib.load().kvq_blocks_in_budget(int(budget_bytes), _dt(k_dtype), _dt(v_dtype), num_kv_heads,
                                                head_dim, num_layers, block_size))


def kvq_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition=0):
    return int(_lib.load().kvq_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                     partition))


def kvq_paged_attention_decode(cache, q, block_tables, seq_lens, max_seq_len, softmax_scale, partition=0,
                               workspace=None, out_dtype="bf16", out=None, err_count=None, stream=None,
                               struct=None):
    """Decode one query per sequence: q bf16 [B][Hq][D] -> out [B][Hq][D] (bf16 or f32).

    block_tables int32 [B][max_blocks]; seq_lens int32 [B]; max_seq_len: host int.
    A workspace is allocated here with torch when the call needs one and none is given.
    """
    _need(q, torch.bfloat16, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_lens, torch.int32, "seq_lens")
    B, Hq, D = q.shape
    odt = _dt(out_dtype)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32 if odt == _lib.F32 else torch.bfloat16, device=q.device)
    need = kvq_decode_workspace_size(B, Hq, cache.num_kv_heads, D, max_seq_len, partition)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_paged_attention_decode(
        ctypes.byref(s), _ptr(q), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len),
        Hq, float(softmax_scale), int(partition), _ptr(workspace), ws_bytes, odt, _ptr(out), _ptr(err_count),
        _stream(stream))
    check(st, "kvq_paged_attention_decode")
    return out
