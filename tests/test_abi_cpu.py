"""The C ABI without a GPU: the library loads, exports what include/kvq.h declares,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from quantized_paged_kv_absmax_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libkvq.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvq_abi_version() == 1


def test_status_strings():
    lib = _lib.load()
    for s in range(7):
        assert lib.kvq_status_string(s).startswith(b"KVQ_")
    assert lib.kvq_status_string(99) == b"unknown kvq_status"


FAKE = 0x10000  # an aligned address that is never dereferenced on the host


def _cache(**kw):
    c = _lib.KvqCacheStruct()
    c.k_dtype = c.v_dtype = _lib.INT8
    c.k_gran = c.v_gran = _lib.PER_TENSOR
    c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim = 8, 16, 2, 128
    c.k_pages = c.v_pages = FAKE
    c.k_scale = c.v_scale = None
    c.k_meta = c.v_meta = None
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _decode(c, B=2, Hq=4, max_seq_len=100, partition=0, ws=None, ws_bytes=0, out_dtype=_lib.BF16, q=FAKE,
            out=FAKE):
    lib = _lib.load()
    return lib.kvq_paged_attention_decode(ctypes.byref(c) if c is not None else None, q, FAKE, 8, FAKE, B,
                                          max_seq_len, Hq, 0.088, partition, ws, ws_bytes, out_dtype, out, None,
                                          None)


def test_decode_argument_errors():
    assert _decode(None) == _lib.ERR_NULL
    assert _decode(_cache(head_dim=96)) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(block_size=32)) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(k_pages=None)) == _lib.ERR_NULL
    assert _decode(_cache(v_pages=FAKE + 4)) == _lib.ERR_ALIGN
    assert _decode(_cache(k_dtype=_lib.INT4_ASYM, k_gran=_lib.PER_TOKEN_HEAD, k_meta=FAKE)) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(k_dtype=_lib.INT4_ASYM, k_gran=_lib.PER_TOKEN_HEAD)) == _lib.ERR_NULL
    assert _decode(_cache(k_gran=_lib.PER_TOKEN_HEAD)) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(k_dtype=9)) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(), Hq=5) == _lib.ERR_SHAPE
    assert _decode(_cache(), Hq=34) == _lib.ERR_UNSUPPORTED        # 17 query heads per KV head
    assert _decode(_cache(), partition=24) == _lib.ERR_SHAPE
    assert _decode(_cache(), out_dtype=_lib.INT8) == _lib.ERR_UNSUPPORTED
    assert _decode(_cache(), q=FAKE + 2) == _lib.ERR_ALIGN
    assert _decode(_cache(), out=None) == _lib.ERR_NULL
    # a split decode needs a workspace of the advertised size
    assert _decode(_cache(), max_seq_len=2000) == _lib.ERR_WORKSPACE
    need = _lib.load().kvq_decode_workspace_size(2, 4, 2, 128, 2000, 0)
    assert _decode(_cache(), max_seq_len=2000, ws=FAKE, ws_bytes=need - 1) == _lib.ERR_WORKSPACE
    assert _decode(_cache(), max_seq_len=2000, ws=FAKE + 8, ws_bytes=need) == _lib.ERR_ALIGN
    # batch 0 is a no-op that succeeds without touching the device
    assert _decode(_cache(), B=0) == _lib.OK


def test_decode_write_argument_errors():
    """The decode step in one call checks the new rows and slots, then every
    argument of the decode, before anything is enqueued (for INT4 caches, whose
    write is a launch of its own, too)."""
    lib = _lib.load()

    def dw(c, kn=FAKE, vn=FAKE, sl=FAKE, B=2, Hq=4, max_seq_len=100, partition=0, q=FAKE, out=FAKE):
        return lib.kvq_paged_attention_decode_write(ctypes.byref(c) if c is not None else None, kn, vn, sl, q, FAKE,
                                                    8, FAKE, B, max_seq_len, Hq, 0.088, partition, None, 0,
                                                    _lib.BF16, out, None, None)

    i4 = dict(k_dtype=_lib.INT4_ASYM, v_dtype=_lib.INT4_ASYM, k_gran=_lib.PER_TOKEN_HEAD,
              v_gran=_lib.PER_TOKEN_HEAD, k_meta=FAKE, v_meta=FAKE)
    for kw in ({}, i4):
        assert dw(None) == _lib.ERR_NULL
        assert dw(_cache(**kw), kn=None) == _lib.ERR_NULL
        assert dw(_cache(**kw), vn=None) == _lib.ERR_NULL
        assert dw(_cache(**kw), sl=None) == _lib.ERR_NULL
        assert dw(_cache(**kw), kn=FAKE + 8) == _lib.ERR_ALIGN
        assert dw(_cache(**kw), Hq=5) == _lib.ERR_SHAPE
        assert dw(_cache(**kw), partition=24) == _lib.ERR_SHAPE
        assert dw(_cache(**kw), q=FAKE + 2) == _lib.ERR_ALIGN
        assert dw(_cache(**kw), out=None) == _lib.ERR_NULL
        assert dw(_cache(**kw), max_seq_len=2000) == _lib.ERR_WORKSPACE
        assert dw(_cache(**kw), B=0, kn=None, vn=None, sl=None) == _lib.OK


def test_verify_argument_errors():
    lib = _lib.load()

    def verify(n_q, Hq=4, B=2):
        c = _cache()
        return lib.kvq_paged_attention_verify(ctypes.byref(c), FAKE, n_q, FAKE, 8, FAKE, B, 100, Hq, 0.088, 0, None,
                                              0, _lib.BF16, FAKE, None, None)

    assert verify(0) == _lib.ERR_SHAPE
    assert verify(-3) == _lib.ERR_SHAPE
    assert verify(20000, Hq=4) == _lib.ERR_SHAPE          # n_q * Hq above 65535
    assert verify(4, Hq=5) == _lib.ERR_SHAPE
    assert verify(4, B=0) == _lib.OK


def test_workspace_size():
    lib = _lib.load()
    r16 = lambda x: (x + 15) // 16 * 16

    def layout(B, Hq, D, n_chunks):
        rows = (n_chunks + B) * Hq
        return 2 * r16(rows * 4) + r16(B * 8) + rows * D * 4

    # automatic split: min(ceil(2048 / Hkv), ceil(pages bound / 4)) chunks
    assert lib.kvq_decode_workspace_size(1, 32, 8, 128, 64, 0) == 0               # 4 pages: one chunk
    assert lib.kvq_decode_workspace_size(1, 32, 8, 128, 80, 0) == layout(1, 32, 128, 2)
    assert lib.kvq_decode_workspace_size(64, 32, 8, 128, 4096, 0) == layout(64, 32, 128, 256)
    assert lib.kvq_decode_workspace_size(64, 33, 3, 128, 4096, 0) == layout(64, 33, 128, 683)
    # explicit partition: ceil(B * ceil(max_seq_len / 16) / (partition / 16)) chunks
    assert lib.kvq_decode_workspace_size(4, 32, 8, 128, 512, 512) == layout(4, 32, 128, 4)
    assert lib.kvq_decode_workspace_size(4, 32, 8, 128, 1100, 256) == layout(4, 32, 128, 18)
    assert lib.kvq_decode_workspace_size(1, 32, 8, 128, 512, 512) == 0
    # invalid arguments: 0
    assert lib.kvq_decode_workspace_size(4, 32, 8, 128, 512, 24) == 0
    assert lib.kvq_decode_workspace_size(4, 32, 0, 128, 512, 0) == 0
    assert lib.kvq_decode_workspace_size(0, 32, 8, 128, 512, 0) == 0
    assert lib.kvq_decode_workspace_size(64, 32, 3, 128, 4096, 0) == 0      # Hq not a multiple of Hkv
    # several query tokens: n_q * Hq rows per slot, chunks for about 2048 waves of
    # n_tiles = ceil(n_q * g / 16) tiles each
    assert lib.kvq_verify_workspace_size(64, 1, 32, 8, 128, 4096, 0) == layout(64, 32, 128, 256)
    assert lib.kvq_verify_workspace_size(64, 16, 32, 8, 128, 4096, 0) == layout(64, 16 * 32, 128, 64)
    assert lib.kvq_verify_workspace_size(4, 3, 32, 8, 128, 1100, 256) == layout(4, 3 * 32, 128, 18)
    assert lib.kvq_verify_workspace_size(4, 0, 32, 8, 128, 1100, 256) == 0


def test_write_convert_calibrate_argument_errors():
    lib = _lib.load()
    c = _cache()
    assert lib.kvq_cache_write(None, FAKE, FAKE, FAKE, 4, None, None) == _lib.ERR_NULL
    assert lib.kvq_cache_write(ctypes.byref(c), None, FAKE, FAKE, 4, None, None) == _lib.ERR_NULL
    assert lib.kvq_cache_write(ctypes.byref(c), FAKE + 2, FAKE, FAKE, 4, None, None) == _lib.ERR_ALIGN
    assert lib.kvq_cache_write(ctypes.byref(c), FAKE, FAKE, FAKE, -1, None, None) == _lib.ERR_SHAPE
    assert lib.kvq_cache_write(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None, None) == _lib.OK
    assert lib.kvq_convert_cache(ctypes.byref(c), FAKE, FAKE, 4, 5, None) == _lib.ERR_SHAPE
    assert lib.kvq_convert_cache(ctypes.byref(c), FAKE, FAKE, -1, 1, None) == _lib.ERR_SHAPE
    assert lib.kvq_convert_cache(ctypes.byref(c), None, FAKE, 0, 1, None) == _lib.ERR_NULL
    assert lib.kvq_convert_cache(ctypes.byref(c), FAKE, FAKE, 0, 0, None) == _lib.OK
    assert lib.kvq_calibrate_scales(FAKE, 10, 2, 128, _lib.PER_TENSOR, _lib.INT8, None, FAKE, None) == _lib.ERR_NULL
    assert lib.kvq_calibrate_scales(FAKE, 10, 2, 128, _lib.PER_TOKEN_HEAD, _lib.INT8, FAKE, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert lib.kvq_calibrate_scales(FAKE, 10, 2, 128, _lib.PER_TENSOR, _lib.INT4_ASYM, FAKE, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert lib.kvq_calibrate_scales(FAKE, 10, 2, 100, _lib.PER_TENSOR, _lib.INT8, FAKE, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert lib.kvq_calibrate_scales(None, 10, 2, 128, _lib.PER_TENSOR, _lib.INT8, FAKE, FAKE, None) == _lib.ERR_NULL
    assert lib.kvq_calibrate_scales(FAKE + 4, 10, 2, 128, _lib.PER_TENSOR, _lib.INT8, FAKE, FAKE, None) == _lib.ERR_ALIGN


def test_capacity_accounting():
    # vLLM PR 4893's L4 table: at one memory budget the block count scales with
    # 1 / (KV bytes per element); the library's count equals the oracle's for every
    # dtype pair, and a PagedKVCache holds exactly that many bytes per block
    import json

    import quantized_paged_kv_absmax_amd as kvq
    from oracle import codecs as oc

    dts = ["bf16", "int8", "e4m3", "e5m2", "int4"]
    for D in (64, 128):
        for kd in dts:
            for vd in dts:
                if (kd == "int4") != (vd == "int4"):
                    continue
                per = kvq.kvq_cache_block_bytes(kd, vd, 8, D)
                assert per == oc.kv_bytes_per_token_head(kd, vd, D) * 8 * 16, (kd, vd, D)
                for budget in (0, per - 1, per, 10 * per + 7, 240 << 30):
                    assert kvq.kvq_blocks_in_budget(budget, kd, vd, 8, D, 32) == \
                        oc.blocks_in_budget(budget, kd, vd, D, 8, 32), (kd, vd, D, budget)
                c = kvq.PagedKVCache(3, 8, D, kd, vd, device="cpu")
                held = c.k_pages.numel() + c.v_pages.numel()
                held += sum(4 * m.numel() for m in (c.k_meta, c.v_meta) if m is not None)
                assert held == 3 * per, (kd, vd, D)
    # Llama-3-8B's cache (32 layers, 8 KV heads, head_dim 128) in 240 GiB of HBM
    budget = 240 << 30
    n = {d: kvq.kvq_blocks_in_budget(budget, d, d, 8, 128, 32) for d in ("bf16", "e5m2", "e4m3", "int8", "int4")}
    assert n["e5m2"] == n["e4m3"] == n["int8"] == 2 * n["bf16"]
    assert abs(n["int4"] / n["bf16"] - 256 / 72) < 1e-3
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "l4_gpu_blocks.json")))["rows"]
    assert g[1]["gpu_blocks"] / g[0]["gpu_blocks"] == n["e5m2"] / n["bf16"] == 2.0
    # invalid arguments
    assert kvq.kvq_cache_block_bytes(9, 1, 8, 128) == 0
    assert kvq.kvq_cache_block_bytes("int8", "int8", 0, 128) == 0
    assert kvq.kvq_blocks_in_budget(budget, "int8", "int8", 8, 128, 0) == -1


def test_binding_rejects_host_tensors():
    """Host tensors never reach the C ABI as device pointers: the binding raises
    before loading the library's compute entry points."""
    import torch
    import quantized_paged_kv_absmax_amd as kvq
    c = kvq.PagedKVCache(2, 2, 128, "int8", "int8", device="cpu")
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 2), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.kvq_paged_attention_decode(c, q, bt, sl, 16, 0.088)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.kvq_paged_attention_verify(c, q, 1, bt, sl, 16, 0.088)
    x = torch.zeros((3, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.kvq_cache_write(c, x, x, torch.arange(3))
    with pytest.raises(ValueError, match="GPU tensor"):
        kvq.kvq_calibrate_scales(x, "per_tensor", "int8", c.k_absmax, c.k_scale)
    with pytest.raises(TypeError):
        kvq.kvq_cache_write(c, x.float(), x, torch.arange(3))


def test_rotated_key_format_argument_errors():
    """KVQ_INT4_HAD is a key format (INT4 layout, metadata required) and
    kvq_hadamard_rotate checks its arguments before any launch."""
    lib = _lib.load()
    tok = dict(k_dtype=_lib.INT4_HAD, v_dtype=_lib.INT4_ASYM, k_gran=_lib.PER_TOKEN_HEAD,
               v_gran=_lib.PER_TOKEN_HEAD, k_meta=FAKE, v_meta=FAKE)
    c = _cache(**tok)
    assert lib.kvq_cache_write(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None, None) == _lib.OK
    bad_v = _cache(**dict(tok, v_dtype=_lib.INT4_HAD))
    assert lib.kvq_cache_write(ctypes.byref(bad_v), FAKE, FAKE, FAKE, 0, None, None) == _lib.ERR_UNSUPPORTED
    no_meta = _cache(**dict(tok, k_meta=None))
    assert lib.kvq_cache_write(ctypes.byref(no_meta), FAKE, FAKE, FAKE, 0, None, None) == _lib.ERR_NULL
    per_tensor = _cache(**dict(tok, k_gran=_lib.PER_TENSOR))
    assert lib.kvq_cache_write(ctypes.byref(per_tensor), FAKE, FAKE, FAKE, 0, None, None) == _lib.ERR_UNSUPPORTED
    assert lib.kvq_cache_block_bytes(_lib.INT4_HAD, _lib.INT4_ASYM, 8, 128, 16) == \
        lib.kvq_cache_block_bytes(_lib.INT4_ASYM, _lib.INT4_ASYM, 8, 128, 16)
    assert lib.kvq_hadamard_rotate(FAKE, 4, 96, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert lib.kvq_hadamard_rotate(FAKE, -1, 128, FAKE, None) == _lib.ERR_SHAPE
    assert lib.kvq_hadamard_rotate(FAKE, 0, 128, FAKE, None) == _lib.OK
    assert lib.kvq_hadamard_rotate(None, 4, 128, FAKE, None) == _lib.ERR_NULL
    assert lib.kvq_hadamard_rotate(FAKE, 4, 64, None, None) == _lib.ERR_NULL
    assert lib.kvq_hadamard_rotate(FAKE + 2, 4, 64, FAKE, None) == _lib.ERR_ALIGN


def test_noalloc_decode_argument_checks():
    """kvq_paged_attention_decode_noalloc rejects bad arguments, and splits whose
    workspace exceeds its static array, on the host before any HIP call."""
    lib = _lib.load()
    c = _cache()
    args = lambda **kw: dict(dict(q=FAKE, bt=FAKE, sl=FAKE, B=2, L=100, Hq=4, part=0, odt=_lib.BF16, out=FAKE), **kw)

    def call(cache=c, **kw):
        a = args(**kw)
        return lib.kvq_paged_attention_decode_noalloc(ctypes.byref(cache) if cache is not None else None, a["q"],
                                                      a["bt"], 8, a["sl"], a["B"], a["L"], a["Hq"], 0.088,
                                                      a["part"], a["odt"], a["out"], None, None)
    assert call(cache=None) == _lib.ERR_NULL
    assert call(q=None) == _lib.ERR_NULL
    assert call(out=None) == _lib.ERR_NULL
    assert call(Hq=3) == _lib.ERR_SHAPE
    assert call(part=8) == _lib.ERR_SHAPE
    assert call(odt=_lib.INT8) == _lib.ERR_UNSUPPORTED
    assert call(B=0) == _lib.OK
    big = _cache(num_kv_heads=8)
    assert lib.kvq_decode_workspace_size(64, 64, 8, 128, 131072, 16) > _lib.DECODE_SCRATCH_BYTES
    assert call(cache=big, B=64, L=131072, Hq=64, part=16) == _lib.ERR_WORKSPACE
