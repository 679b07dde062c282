"""GPU parity over every supported pair of 8- and 16-bit formats: K and V each
bf16, int8, e4m3 or e5m2 (16 pairs), at head sizes 64 and 128.  Each pair and
head size is a kernel instantiation of its own (page sizes, DMA units, QK path,
V conversion), so each is run, through the C ABI, against the oracle:
  * the written codes, bit-exact;
  * decode (one query token) within the float32 output gate, unsplit and with
    16-token splits, sequences of 0, 1 and 16 tokens among them;
  * verify (5 query tokens, 4 heads per KV head: two 16-column tiles sharing a
    workgroup) within the same gate, one sequence shorter than the query block;
  * the decode step in one call (kvq_paged_attention_decode_write) equal, bit for
    bit, to the write followed by the decode, and within the gate of the oracle's
    decode over the cache that holds the new tokens."""

import numpy as np
import pytest
import torch

import quantized_paged_kv_absmax_amd as kvq
from tests.kvq_harness import (assert_codes_equal, build_library_cache, build_oracle_cache, dev_bf16, gate_errors,
                               library_decode, log, oracle_decode, softmax_scale)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu

FORMATS = ["bf16", "int8", "e4m3", "e5m2"]
PAIRS = [(k, v) for k in FORMATS for v in FORMATS]


def _workload(kd, vd, D, lens, n_q=1, new_tokens=0, seed=47):
    return WORKLOADS["tiny_int8"].with_(
        Hq=8, Hkv=2, D=D, k_dtype=kd, v_dtype=vd, B=len(lens), lens=("fixed", tuple(lens)), n_q=n_q,
        new_tokens=new_tokens, seed=seed, k_gran="per_tensor", v_gran="per_tensor",
        k_scale_mode="one" if kd == "bf16" else "absmax", v_scale_mode="one" if vd == "bf16" else "absmax",
        calib="all")


def _check(w, partitions, what):
    inp = make_decode_inputs(w)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    assert int(r.err.item()) == 0
    assert_codes_equal(r, o, inp)
    ref = oracle_decode(o, inp)
    for part in partitions:
        out = library_decode(r, inp, partition=part, out_dtype="f32")
        torch.cuda.synchronize()
        mx, nbad = gate_errors(out, ref, "f32")
        log(f"[{what} {w.k_dtype}/{w.v_dtype} D={w.D}] partition={part} max|err|={mx:.3e}")
        assert nbad == 0
        assert torch.isfinite(out).all()
    return inp, out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kd,vd", PAIRS)
def test_pair_decode_and_verify(kd, vd, D):
    lens = (5, 16, 17, 0, 1, 100, 33)
    inp, out = _check(_workload(kd, vd, D, lens), (0, 16), "decode")
    assert (out[3] == 0).all()                       # seq_len 0 -> zero row
    n_q = 5
    inp, out = _check(_workload(kd, vd, D, (3, 5, 17, 100, 1), n_q=n_q), (0, 16), "verify")
    assert (out[:n_q - 3] == 0).all()                # positions below 0 of the 3-token sequence


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kd,vd", PAIRS)
def test_pair_one_call_step(kd, vd, D):
    w = _workload(kd, vd, D, (5, 16, 17, 1, 100, 33, 64), new_tokens=1, seed=53)
    inp = make_decode_inputs(w)
    # the library's cache with every token but each sequence's last, then the
    # step both ways, on copies
    full = build_library_cache(w, inp)               # calibrated scales and a pool of the right geometry
    last = inp.cu[1:] - 1
    keep = np.ones(int(inp.cu[-1]), bool)
    keep[last] = False
    kb, vb = dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    sl = torch.from_numpy(inp.slot_mapping).cuda()
    it, lt = torch.from_numpy(np.nonzero(keep)[0]).cuda(), torch.from_numpy(last).cuda()

    def prompt_cache():
        c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran)
        for a, b in ((c.k_scale, full.cache.k_scale), (c.v_scale, full.cache.v_scale)):
            if a is not None:
                a.copy_(b)
        kvq.kvq_cache_write(c, kb[it].contiguous(), vb[it].contiguous(), sl[it].contiguous())
        return c

    a, b = prompt_cache(), prompt_cache()
    k_new, v_new, s_new = kb[lt].contiguous(), vb[lt].contiguous(), sl[lt].contiguous()
    ea = torch.zeros(1, dtype=torch.int32, device="cuda")
    eb = torch.zeros_like(ea)
    L, sm = int(inp.max_seq_len), softmax_scale(w.D)
    kvq.kvq_cache_write(a, k_new, v_new, s_new, err_count=ea)
    oa = kvq.kvq_paged_attention_decode(a, full.q, full.bt, full.sl, L, sm, out_dtype="f32", err_count=ea)
    ob = kvq.kvq_paged_attention_decode_write(b, k_new, v_new, s_new, full.q, full.bt, full.sl, L, sm,
                                              out_dtype="f32", err_count=eb)
    torch.cuda.synchronize()
    assert int(ea.item()) == int(eb.item()) == 0
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    assert torch.equal(a.k_pages, b.k_pages) and torch.equal(a.v_pages, b.v_pages)
    # the one-call cache equals the cache written token by token in one pass
    assert torch.equal(b.k_pages, full.cache.k_pages) and torch.equal(b.v_pages, full.cache.v_pages)
    mx, nbad = gate_errors(ob, oracle_decode(build_oracle_cache(w, inp), inp), "f32")
    log(f"[step {kd}/{vd} D={D}] max|err| vs oracle {mx:.3e}")
    assert nbad == 0
