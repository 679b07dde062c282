"""kvq_paged_attention_decode_noalloc (the decode entry point that allocates
nothing, its workspace the library's per-GPU scratch array) against
kvq_paged_attention_decode with a caller workspace, through the C ABI: two calls
in a row, the second with a smaller batch and shorter lengths, at the automatic
split and at a forced small partition.  The same kernels run over the same
workspace layout, so the outputs agree bit for bit; both stay within the
tolerance of the oracle."""

import ctypes

import numpy as np
import pytest
import torch

from quantized_paged_kv_absmax_amd import _lib
from tests.kvq_harness import (build_library_cache, build_oracle_cache, gate_errors, log, oracle_decode,
                               softmax_scale)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu


def _call(lib, fn, r, inp, partition, out, ws=None):
    w = inp.w
    s = r.cache.struct()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    head = (ctypes.byref(s), ctypes.c_void_p(r.q.data_ptr()), ctypes.c_void_p(r.bt.data_ptr()), r.bt.shape[1],
            ctypes.c_void_p(r.sl.data_ptr()), w.B, inp.max_seq_len, w.Hq, softmax_scale(w.D), partition)
    if fn == "noalloc":
        return lib.kvq_paged_attention_decode_noalloc(*head, _lib.F32, ctypes.c_void_p(out.data_ptr()), None, stream)
    return lib.kvq_paged_attention_decode(*head, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _lib.F32,
                                          ctypes.c_void_p(out.data_ptr()), None, stream)


@pytest.mark.parametrize("partition", [0, 64])
def test_noalloc_equals_workspace_decode(partition):
    lib = _lib.load()
    w = WORKLOADS["llama8b_int8"]
    for B, hi in ((16, 2500), (5, 700)):           # the second call: a smaller input
        inp = make_decode_inputs(w, B=B, lens=("uniform", 20, hi))
        log(f"noalloc partition={partition} B={B} lens={inp.seq_lens.tolist()}")
        r = build_library_cache(inp.w, inp)
        need = lib.kvq_decode_workspace_size(B, w.Hq, w.Hkv, w.D, inp.max_seq_len, partition)
        assert 0 < need <= _lib.DECODE_SCRATCH_BYTES
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        a = torch.full((B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
        b = torch.full_like(a, float("nan"))
        assert _call(lib, "noalloc", r, inp, partition, a) == _lib.OK
        assert _call(lib, "workspace", r, inp, partition, b, ws) == _lib.OK
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        o = build_oracle_cache(inp.w, inp)
        mx, nbad = gate_errors(a, oracle_decode(o, inp), "f32")
        log(f"  max|err| vs oracle {mx:.3e}")
        assert nbad == 0


def test_noalloc_rejects_sizes_beyond_its_array():
    """A split whose workspace exceeds KVQ_DECODE_SCRATCH_BYTES is refused on the
    host with KVQ_ERR_WORKSPACE, before any launch."""
    lib = _lib.load()
    B, Hq, Hkv, D, L, part = 64, 64, 8, 128, 131072, 16
    assert lib.kvq_decode_workspace_size(B, Hq, Hkv, D, L, part) > _lib.DECODE_SCRATCH_BYTES
    c = _lib.KvqCacheStruct()
    c.k_dtype = c.v_dtype = _lib.INT8
    c.k_gran = c.v_gran = _lib.PER_TENSOR
    c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim = 8, 16, Hkv, D
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    c.k_pages = c.v_pages = buf.data_ptr()
    st = lib.kvq_paged_attention_decode_noalloc(ctypes.byref(c), buf.data_ptr(), buf.data_ptr(), L // 16,
                                                buf.data_ptr(), B, L, Hq, 0.088, part, _lib.BF16, buf.data_ptr(),
                                                None, None)
    assert st == _lib.ERR_WORKSPACE
