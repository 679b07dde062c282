"""GPU parity of kvq_paged_attention_decode_write, the decode step in one call:
writing each sequence's new token and attending over the cache that holds it must
equal kvq_cache_write followed by kvq_paged_attention_decode, bit for bit (the
output, every page byte and INT4 metadata value, and the error count), for every
format, both head sizes and two splits; and slots that are negative, out of the
pool or not the new token's position behave as documented."""

import copy

import numpy as np
import pytest
import torch

import quantized_paged_kv_absmax_amd as kvq
from tests.kvq_harness import _scale_plan, build_oracle_cache, dev_bf16, gate_errors, log, oracle_decode, softmax_scale
from workloads import WORKLOADS, make_calibration_set, make_decode_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "llama8b_int8": dict(B=12, lens=("uniform", 20, 700)),
    "fp8_e4m3": dict(B=6),
    "fp8_e5m2": dict(B=6),
    "fp8_hybrid": dict(B=6),
    "fp8_e4m3_head": dict(B=6),
    "bf16": dict(B=6, lens=("uniform", 20, 700)),
    "int4": dict(B=6, lens=("uniform", 20, 700)),     # INT4: the row encoder in the pre-pass
    "int4_had": dict(B=6, lens=("uniform", 20, 700)),
    "tiny_int8": dict(B=5, lens=("uniform", 1, 300)),  # head_dim 64, sequences of one token
}


def _prompt_cache(name):
    """The workload's cache with every token written except each sequence's last
    (the step's new token), by the library's own calibration and write."""
    w = WORKLOADS[name]
    if w.calib == "set":
        w = w.with_(calib_set=(8, 512))
    inp = make_decode_inputs(w, **CASES[name])
    c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran)
    kt, vt = _scale_plan(w)
    ck, cv = make_calibration_set(w, inp)
    if kt:
        kvq.kvq_calibrate_scales(dev_bf16(ck), w.k_gran, kt, c.k_absmax, c.k_scale)
    if vt:
        kvq.kvq_calibrate_scales(dev_bf16(cv), w.v_gran, vt, c.v_absmax, c.v_scale)
    last = inp.cu[1:] - 1
    keep = np.ones(int(inp.cu[-1]), bool)
    keep[last] = False
    kd, vd = dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    sl = torch.from_numpy(inp.slot_mapping).cuda()
    it = torch.from_numpy(np.nonzero(keep)[0]).cuda()
    kvq.kvq_cache_write(c, kd[it].contiguous(), vd[it].contiguous(), sl[it].contiguous())
    lt = torch.from_numpy(last).cuda()
    new = (kd[lt].contiguous(), vd[lt].contiguous(), sl[lt].contiguous())
    run = dict(q=dev_bf16(inp.q_bits), bt=torch.from_numpy(inp.block_tables).cuda(),
               sl=torch.from_numpy(inp.seq_lens).cuda(), L=int(inp.max_seq_len), sm=softmax_scale(w.D))
    torch.cuda.synchronize()
    return w, inp, c, new, run


def _clone(c):
    d = copy.copy(c)
    d.k_pages, d.v_pages = c.k_pages.clone(), c.v_pages.clone()
    d.k_meta = None if c.k_meta is None else c.k_meta.clone()
    d.v_meta = None if c.v_meta is None else c.v_meta.clone()
    return d


def _both(c, new, run, partition, slots=None):
    """(two-call output, pages, err), (one-call output, pages, err) from copies of c."""
    k_new, v_new, s_new = new
    s_new = s_new if slots is None else slots
    a, b = _clone(c), _clone(c)
    ea = torch.zeros(1, dtype=torch.int32, device="cuda")
    eb = torch.zeros_like(ea)
    kvq.kvq_cache_write(a, k_new, v_new, s_new, err_count=ea)
    oa = kvq.kvq_paged_attention_decode(a, run["q"], run["bt"], run["sl"], run["L"], run["sm"], partition=partition,
                                        out_dtype="f32", err_count=ea)
    ob = kvq.kvq_paged_attention_decode_write(b, k_new, v_new, s_new, run["q"], run["bt"], run["sl"], run["L"],
                                              run["sm"], partition=partition, out_dtype="f32", err_count=eb)
    torch.cuda.synchronize()
    return (oa, a, int(ea.item())), (ob, b, int(eb.item()))


def _same_cache(a, b):
    assert torch.equal(a.k_pages, b.k_pages)
    assert torch.equal(a.v_pages, b.v_pages)
    for ma, mb in ((a.k_meta, b.k_meta), (a.v_meta, b.v_meta)):
        if ma is not None:
            assert torch.equal(ma.view(torch.int32), mb.view(torch.int32))


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("partition", [0, 64])
def test_one_call_equals_write_then_decode(name, partition):
    w, inp, c, new, run = _prompt_cache(name)
    log(f"[decode_write {name}] partition={partition} lens={inp.seq_lens.tolist()[:8]}")
    (oa, a, ea), (ob, b, eb) = _both(c, new, run, partition)
    assert torch.isfinite(oa).all()
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    _same_cache(a, b)
    assert ea == eb == 0
    # and the step changed the cache: the new rows are in it
    assert not torch.equal(a.k_pages, c.k_pages)
    if partition == 0:
        # against the oracle's cache with every token written, and its decode
        o = build_oracle_cache(w, inp)
        mx, nbad = gate_errors(ob, oracle_decode(o, inp), "f32")
        log(f"[decode_write {name}] max|err| vs oracle {mx:.3e}")
        assert nbad == 0


@pytest.mark.parametrize("name", ["llama8b_int8", "bf16", "tiny_int8", "int4", "int4_had"])
def test_slots_negative_out_of_pool_and_misplaced(name):
    """Sequence 0: slot -1 (neither call writes).  Sequence 1: the slot one past its
    last position on the same page, which attention never reads: the two calls
    write it, the one call counts it and leaves it.  Sequence 2: a slot past the
    pool, counted and skipped by both."""
    w, inp, c, new, run = _prompt_cache(name)
    L = inp.seq_lens.astype(np.int64)
    slots = new[2].clone()
    b1 = [b for b in range(1, len(L)) if L[b] % 16 != 0][0]
    b2 = [b for b in range(1, len(L)) if b != b1][0]
    slots[0] = -1
    slots[b1] = slots[b1] + 1
    slots[b2] = inp.num_blocks * 16 + 5
    log(f"[decode_write slots {name}] misplaced sequence {b1}, out-of-pool sequence {b2}")
    (oa, a, ea), (ob, b, eb) = _both(c, new, run, 0, slots=slots)
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    assert ea == 1 and eb == 2
    # the pages differ exactly at the misplaced slot, where only the two calls wrote
    s1 = int(slots[b1])
    blk, off = s1 // 16, s1 % 16
    for pa, pb in ((a.k_pages, b.k_pages), (a.v_pages, b.v_pages)):
        d = (pa != pb).any(dim=-1).nonzero().tolist()
        assert {tuple(x) for x in d} <= {(blk, h, off) for h in range(w.Hkv)}
        assert len(d) > 0
    # nothing was written for sequence 0 or 2, in either cache
    for x in (a, b):
        for s in (int(new[2][0]), int(new[2][b2])):
            assert torch.equal(x.k_pages[s // 16, :, s % 16], c.k_pages[s // 16, :, s % 16])


@pytest.mark.parametrize("B", [150, 300])
def test_one_call_with_many_short_sequences(B):
    """Many short sequences (0 to 40 tokens): with 2048-token chunks (128 pages) a
    chunk spans more than 64 of them, and with 300 the lengths do not fit the
    registers, so each wave finds the sequences ending in its chunk by rescanning
    them."""
    from tests.kvq_harness import build_library_cache
    lens = tuple((7 * i) % 41 for i in range(B))
    w = WORKLOADS["llama8b_int8"].with_(B=B, lens=("fixed", lens), calib="all")
    inp = make_decode_inputs(w)
    full = build_library_cache(w, inp)
    L = inp.seq_lens.astype(np.int64)
    has = np.nonzero(L > 0)[0]
    last = inp.cu[1:][has] - 1
    keep = np.ones(int(inp.cu[-1]), bool)
    keep[last] = False
    kb, vb = dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    sl = torch.from_numpy(inp.slot_mapping).cuda()
    it = torch.from_numpy(np.nonzero(keep)[0]).cuda()
    rows = np.zeros(B, np.int64)
    rows[has] = last
    slots = np.full(B, -1, np.int64)
    slots[has] = inp.slot_mapping[last]
    nr = torch.from_numpy(rows).cuda()
    new = (kb[nr].contiguous(), vb[nr].contiguous(), torch.from_numpy(slots).cuda())
    c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran)
    c.k_scale.copy_(full.cache.k_scale)
    c.v_scale.copy_(full.cache.v_scale)
    kvq.kvq_cache_write(c, kb[it].contiguous(), vb[it].contiguous(), sl[it].contiguous())
    run = dict(q=full.q, bt=full.bt, sl=full.sl, L=int(inp.max_seq_len), sm=softmax_scale(w.D))
    for partition in (0, 2048):
        (oa, a, ea), (ob, b, eb) = _both(c, new, run, partition)
        log(f"[decode_write B={B}] partition={partition}")
        assert ea == eb == 0
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
        _same_cache(a, b)
        assert torch.equal(b.k_pages, full.cache.k_pages) and torch.equal(b.v_pages, full.cache.v_pages)
    mx, nbad = gate_errors(ob, oracle_decode(build_oracle_cache(w, inp), inp), "f32")
    log(f"[decode_write B={B}] max|err| vs oracle {mx:.3e}")
    assert nbad == 0
