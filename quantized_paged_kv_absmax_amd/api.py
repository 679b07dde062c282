"""Python binding of libkvq with the C names; torch tensors supply device memory
and the current HIP stream.  Every step of the work runs in the HIP kernels.

    cache = PagedKVCache(num_blocks, num_kv_heads, head_dim, "int8", "int8",
                         k_gran="per_tensor", v_gran="per_tensor", device="cuda")
    kvq_calibrate_scales(k_bf16, "per_tensor", "int8", cache.k_absmax, cache.k_scale)
    kvq_cache_write(cache, k_new, v_new, slot_mapping)
    out = kvq_paged_attention_decode(cache, q, block_tables, seq_lens, max_seq_len, scale)
"""

import contextlib
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


def _on(stream):
    """Context for the binding's own allocations (output, workspace): made on the
    stream the call enqueues on, so that torch's caching allocator orders their
    reuse after that work and not after the current stream's."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _need(t, dtype, name, shape=None, device=None, min_numel=None):
    """The C ABI takes bare device pointers and cannot see sizes: every tensor is
    checked here (type, GPU residence, layout, shape) before its pointer is passed,
    so a mismatch raises instead of reaching a kernel as an out-of-bounds access."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _opt(t, dtype, name, device, min_numel=1):
    if t is not None:
        _need(t, dtype, name, device=device, min_numel=min_numel)


def _out_torch_dtype(odt):
    if odt == _lib.F32:
        return torch.float32
    if odt == _lib.BF16:
        return torch.bfloat16
    raise ValueError(f"out_dtype must be bf16 or f32, got {odt}")


def row_bytes(dtype, head_dim):
    d = _dt(dtype)
    return {_lib.BF16: 2 * head_dim, _lib.INT8: head_dim, _lib.FP8_E4M3: head_dim, _lib.FP8_E5M2: head_dim,
            _lib.INT4_ASYM: head_dim // 2, _lib.INT4_HAD: head_dim // 2}[d]


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
        int4 = (_lib.INT4_ASYM, _lib.INT4_HAD)
        self.k_gran = _lib.PER_TOKEN_HEAD if self.k_dtype in int4 else _gr(k_gran)
        self.v_gran = _lib.PER_TOKEN_HEAD if self.v_dtype in int4 else _gr(v_gran)
        shp = (num_blocks, num_kv_heads, block_size)
        self.k_pages = torch.full(shp + (row_bytes(self.k_dtype, head_dim),), fill, dtype=torch.uint8, device=device)
        self.v_pages = torch.full(shp + (row_bytes(self.v_dtype, head_dim),), fill, dtype=torch.uint8, device=device)
        g = lambda gr: num_kv_heads if gr == _lib.PER_KV_HEAD else 1
        self.k_scale = torch.ones(g(self.k_gran), dtype=torch.float32, device=device)
        self.v_scale = torch.ones(g(self.v_gran), dtype=torch.float32, device=device)
        self.k_absmax = torch.zeros_like(self.k_scale)
        self.v_absmax = torch.zeros_like(self.v_scale)
        meta = lambda dt: (torch.full(shp + (2,), float("nan"), dtype=torch.float32, device=device)
                           if dt in int4 else None)
        self.k_meta, self.v_meta = meta(self.k_dtype), meta(self.v_dtype)

    def struct(self, k_pages=None, v_pages=None):
        """The C kvq_cache describing this cache (optionally over other page buffers
        of the same shape, e.g. a rotating copy)."""
        kp = self.k_pages if k_pages is None else k_pages
        vp = self.v_pages if v_pages is None else v_pages
        _need(kp, torch.uint8, "k_pages", shape=self.k_pages.shape, device=self.k_pages.device)
        _need(vp, torch.uint8, "v_pages", shape=self.v_pages.shape, device=self.k_pages.device)
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
    if x.dim() != 3:
        raise ValueError(f"x must be [T][Hkv][D], got shape {tuple(x.shape)}")
    T, H, D = x.shape
    groups = H if _gr(granularity) == _lib.PER_KV_HEAD else 1
    _need(absmax_inout, torch.float32, "absmax_inout", device=x.device, min_numel=groups)
    _need(scale_out, torch.float32, "scale_out", device=x.device, min_numel=groups)
    st = _lib.load().kvq_calibrate_scales(_ptr(x), T, H, D, _gr(granularity), _dt(target_dtype),
                                          _ptr(absmax_inout), _ptr(scale_out), _stream(stream))
    check(st, "kvq_calibrate_scales")


def kvq_cache_write(cache, k_new, v_new, slot_mapping, err_count=None, stream=None, struct=None):
    """Encode bf16 rows k_new / v_new [T][Hkv][D] into the pages at slot_mapping (int64 [T])."""
    dev = cache.k_pages.device
    _need(k_new, torch.bfloat16, "k_new", device=dev)
    T = k_new.shape[0] if k_new.dim() == 3 else -1
    _need(k_new, torch.bfloat16, "k_new", shape=(T, cache.num_kv_heads, cache.head_dim))
    _need(v_new, torch.bfloat16, "v_new", shape=(T, cache.num_kv_heads, cache.head_dim), device=dev)
    _need(slot_mapping, torch.int64, "slot_mapping", shape=(T,), device=dev)
    _opt(err_count, torch.int32, "err_count", dev)
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_cache_write(ctypes.byref(s), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                     k_new.shape[0], _ptr(err_count), _stream(stream))
    check(st, "kvq_cache_write")


def kvq_convert_cache(cache, k_src, v_src, first_block=0, num_blocks=None, stream=None):
    """Convert bf16 pages [num_blocks][Hkv][16][D] into the cache's format."""
    dev = cache.k_pages.device
    shp = (cache.num_blocks, cache.num_kv_heads, cache.block_size, cache.head_dim)
    _need(k_src, torch.bfloat16, "k_src", shape=shp, device=dev)
    _need(v_src, torch.bfloat16, "v_src", shape=shp, device=dev)
    n = cache.num_blocks - first_block if num_blocks is None else num_blocks
    s = cache.struct()
    st = _lib.load().kvq_convert_cache(ctypes.byref(s), _ptr(k_src), _ptr(v_src), first_block, n, _stream(stream))
    check(st, "kvq_convert_cache")


def kvq_hadamard_rotate(x, out=None, stream=None):
    """bf16 rows x [..., D] -> bf16 rows of H x, the rotation of rotated-key (int4h) caches."""
    _need(x, torch.bfloat16, "x")
    D = x.shape[-1]
    if out is None:
        with _on(stream):
            out = torch.empty_like(x)
    _need(out, torch.bfloat16, "out", shape=x.shape, device=x.device)
    st = _lib.load().kvq_hadamard_rotate(_ptr(x), x.numel() // max(D, 1), D, _ptr(out), _stream(stream))
    check(st, "kvq_hadamard_rotate")
    return out


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
    dev = cache.k_pages.device
    _need(seq_lens, torch.int32, "seq_lens", device=dev)
    if seq_lens.dim() != 1:
        raise ValueError(f"seq_lens must be [B], got shape {tuple(seq_lens.shape)}")
    B = seq_lens.shape[0]
    _need(block_tables, torch.int32, "block_tables", device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_blocks], got shape {tuple(block_tables.shape)}")
    if q.dim() != 3:
        raise ValueError(f"q must be [B * n_q][Hq][D], got shape {tuple(q.shape)}")
    Hq = q.shape[1]
    _need(q, torch.bfloat16, "q", shape=(B * n_q, Hq, cache.head_dim), device=dev)
    T, D = B * n_q, cache.head_dim
    odt = _dt(out_dtype)
    need = kvq_verify_workspace_size(B, n_q, Hq, cache.num_kv_heads, D, max_seq_len, partition)
    with _on(stream):
        if out is None:
            out = torch.empty((T, Hq, D), dtype=_out_torch_dtype(odt), device=dev)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(out, _out_torch_dtype(odt), "out", shape=(T, Hq, D), device=dev)
    _opt(err_count, torch.int32, "err_count", dev)
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace", device=dev)
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


def _decode_args(cache, q, block_tables, seq_lens, max_seq_len, partition, workspace, out_dtype, out, err_count,
                 stream):
    """Checks of one-token decode arguments; the output (and the workspace, when
    the call needs one and none is given) allocated on the call's stream."""
    dev = cache.k_pages.device
    _need(seq_lens, torch.int32, "seq_lens", device=dev)
    if seq_lens.dim() != 1:
        raise ValueError(f"seq_lens must be [B], got shape {tuple(seq_lens.shape)}")
    B = seq_lens.shape[0]
    _need(block_tables, torch.int32, "block_tables", device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_blocks], got shape {tuple(block_tables.shape)}")
    if q.dim() != 3:
        raise ValueError(f"q must be [B][Hq][D], got shape {tuple(q.shape)}")
    Hq, D = q.shape[1], cache.head_dim
    _need(q, torch.bfloat16, "q", shape=(B, Hq, D), device=dev)
    odt = _dt(out_dtype)
    need = kvq_decode_workspace_size(B, Hq, cache.num_kv_heads, D, max_seq_len, partition)
    with _on(stream):
        if out is None:
            out = torch.empty((B, Hq, D), dtype=_out_torch_dtype(odt), device=dev)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(out, _out_torch_dtype(odt), "out", shape=(B, Hq, D), device=dev)
    _opt(err_count, torch.int32, "err_count", dev)
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace", device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return B, Hq, odt, out, workspace, ws_bytes


def kvq_paged_attention_decode(cache, q, block_tables, seq_lens, max_seq_len, softmax_scale, partition=0,
                               workspace=None, out_dtype="bf16", out=None, err_count=None, stream=None,
                               struct=None):
    """Decode one query per sequence: q bf16 [B][Hq][D] -> out [B][Hq][D] (bf16 or f32).

    block_tables int32 [B][max_blocks]; seq_lens int32 [B]; max_seq_len: host int.
    A workspace is allocated here with torch when the call needs one and none is given.
    """
    B, Hq, odt, out, workspace, ws_bytes = _decode_args(cache, q, block_tables, seq_lens, max_seq_len, partition,
                                                        workspace, out_dtype, out, err_count, stream)
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_paged_attention_decode(
        ctypes.byref(s), _ptr(q), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len),
        Hq, float(softmax_scale), int(partition), _ptr(workspace), ws_bytes, odt, _ptr(out), _ptr(err_count),
        _stream(stream))
    check(st, "kvq_paged_attention_decode")
    return out


def kvq_paged_attention_decode_write(cache, k_new, v_new, slot_mapping, q, block_tables, seq_lens, max_seq_len,
                                     softmax_scale, partition=0, workspace=None, out_dtype="bf16", out=None,
                                     err_count=None, stream=None, struct=None):
    """The decode step in one call: write each sequence's new token (k_new / v_new
    bf16 [B][Hkv][D] at slot_mapping int64 [B]) and decode q over the cache that
    holds it; the same as kvq_cache_write then kvq_paged_attention_decode when each
    slot is negative or that of position seq_lens[b] - 1."""
    B, Hq, odt, out, workspace, ws_bytes = _decode_args(cache, q, block_tables, seq_lens, max_seq_len, partition,
                                                        workspace, out_dtype, out, err_count, stream)
    dev = cache.k_pages.device
    _need(k_new, torch.bfloat16, "k_new", shape=(B, cache.num_kv_heads, cache.head_dim), device=dev)
    _need(v_new, torch.bfloat16, "v_new", shape=(B, cache.num_kv_heads, cache.head_dim), device=dev)
    _need(slot_mapping, torch.int64, "slot_mapping", shape=(B,), device=dev)
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_paged_attention_decode_write(
        ctypes.byref(s), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q), _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len), Hq, float(softmax_scale), int(partition),
        _ptr(workspace), ws_bytes, odt, _ptr(out), _ptr(err_count), _stream(stream))
    check(st, "kvq_paged_attention_decode_write")
    return out


def kvq_paged_attention_decode_noalloc(cache, q, block_tables, seq_lens, max_seq_len, softmax_scale, partition=0,
                                       out_dtype="bf16", out=None, err_count=None, stream=None, struct=None):
    """kvq_paged_attention_decode with the library's own per-GPU scratch array as
    workspace (no device allocation by the library).  Calls that overlap on one
    GPU share that array: serialise them.  ``out`` is allocated here only when
    not given."""
    dev = cache.k_pages.device
    _need(seq_lens, torch.int32, "seq_lens", device=dev)
    if seq_lens.dim() != 1:
        raise ValueError(f"seq_lens must be [B], got shape {tuple(seq_lens.shape)}")
    B = seq_lens.shape[0]
    _need(block_tables, torch.int32, "block_tables", device=dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_blocks], got shape {tuple(block_tables.shape)}")
    if q.dim() != 3:
        raise ValueError(f"q must be [B][Hq][D], got shape {tuple(q.shape)}")
    Hq, D = q.shape[1], cache.head_dim
    _need(q, torch.bfloat16, "q", shape=(B, Hq, D), device=dev)
    odt = _dt(out_dtype)
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, D), dtype=_out_torch_dtype(odt), device=dev)
    _need(out, _out_torch_dtype(odt), "out", shape=(B, Hq, D), device=dev)
    _opt(err_count, torch.int32, "err_count", dev)
    s = cache.struct() if struct is None else struct
    st = _lib.load().kvq_paged_attention_decode_noalloc(
        ctypes.byref(s), _ptr(q), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), B, int(max_seq_len),
        Hq, float(softmax_scale), int(partition), odt, _ptr(out), _ptr(err_count), _stream(stream))
    check(st, "kvq_paged_attention_decode_noalloc")
    return out
