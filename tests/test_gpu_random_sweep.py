"""GPU parity on a seeded sweep of random shapes: format pair, head size, KV and
query heads, batch and length mix (empty, one-token and page-edge lengths among
them), scale granularity, query tokens per sequence, work split, the cache
written token by token or converted from bf16 pages, and the call's output type.
Each case: the cache codes bit-exact against the oracle, and the attention
output within the gate of its output type (f32: 4e-3 absolute; bf16: that or
half a bf16 ulp of the oracle's value plus 1e-4)."""

import numpy as np
import pytest
import torch

from tests.kvq_harness import (assert_codes_equal, build_library_cache, build_oracle_cache, gate_errors,
                               library_decode, log, oracle_decode)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu

PAIRS = [(k, v) for k in ("bf16", "int8", "e4m3", "e5m2") for v in ("bf16", "int8", "e4m3", "e5m2")]
PAIRS += [("int4", "int4"), ("int4h", "int4")]
N_CASES = 160


def _case(i):
    rng = np.random.default_rng(1000 + i)
    kd, vd = PAIRS[int(rng.integers(len(PAIRS)))]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8]))
    B = int(rng.integers(1, 13))
    lens = rng.integers(0, 700, size=B)
    edge = np.array([0, 1, 15, 16, 17, 32, 33])
    pick = rng.random(B) < 0.3
    lens[pick] = rng.choice(edge, size=int(pick.sum()))
    if lens.max() == 0:
        lens[0] = 5                                   # at least one sequence with tokens
    n_q = 1 if rng.random() < 0.6 else int(rng.integers(2, 21))
    partition = int(rng.choice([0, 0, 16, 64, 512]))
    int4 = kd in ("int4", "int4h")
    gran = "per_token_head" if int4 else ("per_kv_head" if rng.random() < 0.3 else "per_tensor")
    mode = lambda dt: "row" if int4 else ("one" if dt == "bf16" or (dt == "e5m2" and rng.random() < 0.5) else "absmax")
    w = WORKLOADS["tiny_int8"].with_(
        name=f"sweep{i}", seed=2000 + i, B=B, Hq=g * Hkv, Hkv=Hkv, D=D, k_dtype=kd, v_dtype=vd,
        lens=("fixed", tuple(int(x) for x in lens)), n_q=n_q, new_tokens=0, partition=partition,
        k_gran="per_tensor" if kd == "bf16" else gran, v_gran="per_tensor" if vd == "bf16" else gran,
        k_scale_mode=mode(kd), v_scale_mode=mode(vd),
        calib="none" if int4 else "all", from_bf16_cache=bool(rng.random() < 0.2))
    out_dtype = "bf16" if rng.random() < 0.3 else "f32"
    return w, out_dtype


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    w, out_dtype = _case(i)
    log(f"[sweep {i}] {w.k_dtype}/{w.v_dtype} D={w.D} Hq={w.Hq} Hkv={w.Hkv} B={w.B} n_q={w.n_q} "
        f"partition={w.partition} gran={w.k_gran} convert={w.from_bf16_cache} out={out_dtype} lens={w.lens[1]}")
    inp = make_decode_inputs(w)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    assert int(r.err.item()) == 0
    assert_codes_equal(r, o, inp)
    out = library_decode(r, inp, partition=w.partition, out_dtype=out_dtype)
    torch.cuda.synchronize()
    mx, nbad = gate_errors(out, oracle_decode(o, inp), out_dtype)
    log(f"[sweep {i}] max|err| = {mx:.3e}")
    assert nbad == 0


N_STEP_CASES = 60


@pytest.mark.parametrize("i", range(N_STEP_CASES))
def test_random_one_call_step(i):
    """The decode step in one call on random shapes: equal, bit for bit, to the
    write then the decode (output, pages, metadata), and within the f32 gate of
    the oracle over the cache holding the new tokens."""
    import quantized_paged_kv_absmax_amd as kvq
    from tests.kvq_harness import dev_bf16, softmax_scale
    w, _ = _case(5000 + i)
    w = w.with_(n_q=1, new_tokens=1, from_bf16_cache=False)
    inp = make_decode_inputs(w)
    log(f"[step sweep {i}] {w.k_dtype}/{w.v_dtype} D={w.D} Hq={w.Hq} Hkv={w.Hkv} B={w.B} "
        f"partition={w.partition} gran={w.k_gran} lens={inp.seq_lens.tolist()}")
    full = build_library_cache(w, inp)          # scales, and the cache with every token written
    L = inp.seq_lens.astype(np.int64)
    has = np.nonzero(L > 0)[0]
    last = inp.cu[1:][has] - 1
    keep = np.ones(int(inp.cu[-1]), bool)
    keep[last] = False
    kb, vb = dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    sl = torch.from_numpy(inp.slot_mapping).cuda()
    it = torch.from_numpy(np.nonzero(keep)[0]).cuda()
    # one new token per sequence: a sequence with no tokens takes slot -1 (its row unused)
    new_rows = np.zeros(w.B, np.int64)
    new_rows[has] = last
    slots = np.full(w.B, -1, np.int64)
    slots[has] = inp.slot_mapping[last]
    nr = torch.from_numpy(new_rows).cuda()
    k_new, v_new = kb[nr].contiguous(), vb[nr].contiguous()
    s_new = torch.from_numpy(slots).cuda()

    def prompt_cache():
        c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran)
        for a, b in ((c.k_scale, full.cache.k_scale), (c.v_scale, full.cache.v_scale)):
            if a is not None:
                a.copy_(b)
        if it.numel():
            kvq.kvq_cache_write(c, kb[it].contiguous(), vb[it].contiguous(), sl[it].contiguous())
        return c

    a, b = prompt_cache(), prompt_cache()
    ea = torch.zeros(1, dtype=torch.int32, device="cuda")
    eb = torch.zeros_like(ea)
    Lmax, sm = int(inp.max_seq_len), softmax_scale(w.D)
    kvq.kvq_cache_write(a, k_new, v_new, s_new, err_count=ea)
    oa = kvq.kvq_paged_attention_decode(a, full.q, full.bt, full.sl, Lmax, sm, partition=w.partition,
                                        out_dtype="f32", err_count=ea)
    ob = kvq.kvq_paged_attention_decode_write(b, k_new, v_new, s_new, full.q, full.bt, full.sl, Lmax, sm,
                                              partition=w.partition, out_dtype="f32", err_count=eb)
    torch.cuda.synchronize()
    assert int(ea.item()) == int(eb.item()) == 0
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    for x, y in ((a.k_pages, b.k_pages), (a.v_pages, b.v_pages), (b.k_pages, full.cache.k_pages),
                 (b.v_pages, full.cache.v_pages)):
        assert torch.equal(x, y)
    for x, y in ((a.k_meta, b.k_meta), (a.v_meta, b.v_meta)):
        if x is not None:
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    mx, nbad = gate_errors(ob, oracle_decode(build_oracle_cache(w, inp), inp), "f32")
    log(f"[step sweep {i}] max|err| = {mx:.3e}")
    assert nbad == 0
