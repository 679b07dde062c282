"""GPU parity of the paged decode (and of the cache it reads) against the oracle,
on every workload at reduced sizes that span several partitions and a ragged
tail, plus the edge cases."""

import numpy as np
import pytest
import torch

import quantized_paged_kv_absmax_amd as kvq
from tests.kvq_harness import (assert_codes_equal, build_library_cache, build_oracle_cache, dev_bf16, gate_errors,
                               library_decode, log, oracle_decode, softmax_scale)
from workloads import WORKLOADS, make_decode_inputs
from oracle import cache as oc

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_int8": {},
    "llama8b_int8": dict(B=8, lens=("uniform", 20, 1500)),
    "fp8_e4m3": dict(B=6),
    "fp8_e4m3_s1": dict(B=6),
    "fp8_e5m2": dict(B=6),
    "fp8_hybrid": dict(B=6),
    "fp8_e4m3_head": dict(B=6),
    "fp8_e5m2_cal": dict(B=6),
    "longctx_int8": dict(B=2, lens=("uniform", 1000, 3000)),
    "int4": dict(B=8, lens=("uniform", 20, 1500)),
    "int4_had": dict(B=8, lens=("uniform", 20, 1500)),
    "bf16": dict(B=6, lens=("uniform", 20, 1500)),
}


def _workload(name):
    w = WORKLOADS[name]
    if w.calib == "set":
        w = w.with_(calib_set=(8, 512))
    return w


_cache = {}


def _setup(name):
    if name not in _cache:
        w = _workload(name)
        inp = make_decode_inputs(w, **CASES[name])
        log(f"[{name}] B={inp.w.B} lens={inp.seq_lens.tolist()[:8]} blocks={inp.num_blocks}")
        r = build_library_cache(w, inp)
        o = build_oracle_cache(w, inp)
        ref = oracle_decode(o, inp)
        _cache.clear()
        _cache[name] = (inp, r, o, ref)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_cache_codes_bit_exact(name):
    inp, r, o, _ = _setup(name)
    assert_codes_equal(r, o, inp)
    assert int(r.err.item()) == 0
    if o.kabs is not None:
        assert np.array_equal(r.cache.k_absmax.cpu().numpy(), o.kabs)
        assert np.array_equal(r.cache.k_scale.cpu().numpy(), o.k_scale)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("partition", [0, 64])
def test_decode_within_tolerance(name, partition):
    inp, r, o, ref = _setup(name)
    for odt in ("f32", "bf16"):
        out = library_decode(r, inp, partition=partition, out_dtype=odt)
        torch.cuda.synchronize()
        mx, nbad = gate_errors(out, ref, odt)
        log(f"[{name}] partition={partition} out={odt} max|err|={mx:.3e} violations={nbad}")
        assert nbad == 0


@pytest.mark.parametrize("name", ["llama8b_int8", "fp8_hybrid", "int4"])
def test_split_matches_unsplit_and_is_deterministic(name):
    inp, r, o, ref = _setup(name)
    a = library_decode(r, inp, partition=0, out_dtype="f32")
    b = library_decode(r, inp, partition=0, out_dtype="f32")
    torch.cuda.synchronize()
    assert torch.equal(a, b)                                  # bit-identical reruns
    # The PV product takes p in fp16, rounded relative to each partition's own
    # running max: per weight a relative error of at most 2^-12, so two
    # partitionings differ by at most 2 * 2^-12 * max|v_hat| (~1e-3 for the
    # values here); both are separately within the oracle gate above.
    vmax = float(np.abs(o.gather(inp.block_tables[0], int(inp.seq_lens[0]), "v")).max())
    for part in (16, 128, 2048):
        s = library_decode(r, inp, partition=part, out_dtype="f32")
        torch.cuda.synchronize()
        d = float((s - a).abs().max())
        log(f"[{name}] split {part} vs unsplit: max|diff|={d:.3e} (bound {2 * 2 ** -12 * vmax:.3e})")
        assert d <= 2 * 2 ** -12 * vmax, part


@pytest.mark.parametrize("name,B", [("llama8b_int8", 16), ("fp8_e4m3", 12), ("int4", 16), ("int4_had", 8)])
def test_repeated_calls_bit_identical(name, B):
    """The automatic split at full sequence lengths, where each wave streams a
    short chunk (a few rounds) and the ring's first waits overlap the length scan:
    eight calls through one workspace are bit-identical and within the oracle gate.
    A load that a ring wait let through before it landed would show up here as a
    piece that changes from call to call."""
    w = _workload(name)
    inp = make_decode_inputs(w, B=B)
    log(f"[repeat {name}] B={B} lens={inp.seq_lens.tolist()}")
    r = build_library_cache(w, inp)
    need = kvq.kvq_decode_workspace_size(B, w.Hq, w.Hkv, w.D, inp.max_seq_len, 0)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(8):
        out = torch.full((B, w.Hq, w.D), float("nan"), device="cuda")
        kvq.kvq_paged_attention_decode(r.cache, r.q, r.bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                       partition=0, workspace=ws, out_dtype="f32", out=out)
        torch.cuda.synchronize()
        outs.append(out)
    for i, out in enumerate(outs[1:], 1):
        d = (out - outs[0]).abs().amax(-1)
        assert torch.equal(out, outs[0]), (i, (d > 0).nonzero().tolist()[:8])
    o = build_oracle_cache(w, inp)
    mx, nbad = gate_errors(outs[0], oracle_decode(o, inp), "f32")
    log(f"[repeat {name}] max|err|={mx:.3e}")
    assert nbad == 0


def _small(Hq=8, Hkv=2, D=128, lens=(5, 16, 17, 0, 1, 512, 513), kd="int8", vd="int8"):
    w = WORKLOADS["tiny_int8"].with_(Hq=Hq, Hkv=Hkv, D=D, k_dtype=kd, v_dtype=vd, B=len(lens),
                                     lens=("fixed", tuple(lens)),
                                     k_scale_mode="absmax" if kd in ("int8", "e4m3", "e5m2") else "one",
                                     v_scale_mode="absmax" if vd in ("int8", "e4m3", "e5m2") else "one",
                                     k_gran="per_token_head" if kd == "int4" else "per_tensor",
                                     v_gran="per_token_head" if vd == "int4" else "per_tensor",
                                     calib="all" if kd != "int4" else "none")
    inp = make_decode_inputs(w)
    return w, inp


@pytest.mark.parametrize("kd,vd,D,Hq,Hkv", [
    ("int8", "int8", 128, 8, 2), ("e5m2", "e4m3", 64, 16, 1), ("int4", "int4", 64, 6, 3),
    ("bf16", "int8", 128, 32, 2), ("e4m3", "bf16", 64, 4, 4), ("int4", "int4", 128, 16, 1),
])
def test_edge_lengths_and_group_sizes(kd, vd, D, Hq, Hkv):
    w, inp = _small(Hq=Hq, Hkv=Hkv, D=D, kd=kd, vd=vd)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    assert_codes_equal(r, o, inp)
    ref = oracle_decode(o, inp)
    for part in (0, 16, 32):
        out = library_decode(r, inp, partition=part, out_dtype="f32")
        torch.cuda.synchronize()
        mx, nbad = gate_errors(out, ref, "f32")
        log(f"[edge {kd}/{vd} D={D} g={Hq // Hkv}] partition={part} max|err|={mx:.3e}")
        assert nbad == 0
        assert (out[3] == 0).all()                 # seq_len 0 -> zero row
        assert torch.isfinite(out).all()           # NaN-coded unused slots never leak


@pytest.mark.parametrize("kd,vd,nseq", [("int8", "int8", 150), ("int4", "int4", 150), ("int8", "int8", 300)])
def test_many_short_sequences(kd, vd, nseq):
    # 150 sequences of 0..40 tokens: more sequences than lanes of a wave, and with
    # 2048-token chunks (128 pages) a chunk spans more than 64 sequences; 300
    # sequences: more than the kernel keeps in registers, so it rescans lengths
    lens = tuple((7 * i) % 41 for i in range(nseq))
    w, inp = _small(Hq=8, Hkv=2, D=128, lens=lens, kd=kd, vd=vd)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    assert_codes_equal(r, o, inp)
    ref = oracle_decode(o, inp)
    zero = [i for i, L in enumerate(lens) if L == 0]
    for part in (0, 16, 2048):
        out = library_decode(r, inp, partition=part, out_dtype="f32")
        torch.cuda.synchronize()
        mx, nbad = gate_errors(out, ref, "f32")
        log(f"[short {kd}/{vd} x{nseq}] partition={part} max|err|={mx:.3e}")
        assert nbad == 0
        assert (out[zero] == 0).all()


def test_workspace_reused_across_calls():
    # one workspace through calls with different queries and splits: no piece of
    # an earlier call may leak into a later one
    from oracle import attention as oa
    inp, r, o, ref = _setup("llama8b_int8")
    w = inp.w
    need = max(kvq.kvq_decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, inp.max_seq_len, part) for part in (0, 16, 64))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    q_neg = inp.q_bits ^ np.uint16(0x8000)
    calls = [(64, inp.q_bits), (64, q_neg), (16, inp.q_bits), (0, q_neg), (0, inp.q_bits)]
    refs = {0: ref, 1: oa.decode(o, q_neg, inp.block_tables, inp.seq_lens, softmax_scale(w.D))}
    firsts = {}
    for part, qb in calls:
        qd = dev_bf16(qb)
        out = kvq.kvq_paged_attention_decode(r.cache, qd, r.bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                             partition=part, workspace=ws, out_dtype="f32")
        torch.cuda.synchronize()
        key = 1 if qb is q_neg else 0
        mx, nbad = gate_errors(out, refs[key], "f32")
        log(f"[reuse] partition={part} q={'neg' if key else 'pos'} max|err|={mx:.3e}")
        assert nbad == 0
        if (part, key) in firsts:
            assert torch.equal(out, firsts[(part, key)])
        firsts[(part, key)] = out


def test_bad_block_ids_are_counted_not_faulted():
    w, inp = _small(lens=(40, 33))
    r = build_library_cache(w, inp)
    bt = r.bt.clone()
    bt[0, 1] = -5
    bt[1, 0] = 10 ** 6
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvq.kvq_paged_attention_decode(r.cache, r.q, bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                         out_dtype="f32", err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) >= 2
    assert torch.isfinite(out[0]).all()


def test_seq_len_clamped_to_max_and_counted():
    w, inp = _small(lens=(40, 33))
    r = build_library_cache(w, inp)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvq.kvq_paged_attention_decode(r.cache, r.q, r.bt, r.sl, 33, softmax_scale(w.D), out_dtype="f32",
                                         err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    o = build_oracle_cache(w, inp)
    from oracle import attention as oa
    ref = oa.decode(o, inp.q_bits, inp.block_tables, np.minimum(inp.seq_lens, 33), softmax_scale(w.D))
    mx, nbad = gate_errors(out, ref, "f32")
    assert nbad == 0


def test_empty_batch_is_a_noop():
    c = kvq.PagedKVCache(2, 2, 128, "int8", "int8")
    q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    out = kvq.kvq_paged_attention_decode(c, q, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                                         torch.zeros(0, dtype=torch.int32, device="cuda"), 0, 0.088)
    assert out.shape == (0, 4, 128)


def test_binding_rejects_mismatched_tensors():
    """The C ABI sees bare pointers; the binding raises on any tensor whose shape,
    dtype or device does not match the cache and the batch, before a launch."""
    c = kvq.PagedKVCache(4, 2, 128, "int8", "int8")
    dev = "cuda"
    B, Hq = 3, 8
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 4), dtype=torch.int32, device=dev)
    sl = torch.full((B,), 5, dtype=torch.int32, device=dev)
    bad = [
        dict(q=torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device=dev)),          # head_dim of another cache
        dict(q=torch.zeros((B - 1, Hq, 128), dtype=torch.bfloat16, device=dev)),     # fewer rows than sequences
        dict(block_tables=torch.zeros((B - 1, 4), dtype=torch.int32, device=dev)),   # fewer tables than sequences
        dict(block_tables=torch.zeros((B, 4), dtype=torch.int64, device=dev)),
        dict(seq_lens=sl.cpu()),
        dict(out=torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)),       # bf16 requested
        dict(err_count=torch.zeros(1, dtype=torch.int64, device=dev)),
        dict(workspace=torch.zeros(64, dtype=torch.float32, device=dev)),
    ]
    for over in bad:
        args = dict(q=q, block_tables=bt, seq_lens=sl, out=None, err_count=None, workspace=None)
        args.update(over)
        with pytest.raises((ValueError, TypeError)):
            kvq.kvq_paged_attention_decode(c, args["q"], args["block_tables"], args["seq_lens"], 16, 0.088,
                                           out=args["out"], err_count=args["err_count"],
                                           workspace=args["workspace"])
    x = torch.zeros((5, 2, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        kvq.kvq_cache_write(c, x, x, torch.arange(4, dtype=torch.int64, device=dev))   # 4 slots for 5 rows
    with pytest.raises(ValueError):
        kvq.kvq_cache_write(c, x[:, :1].contiguous(), x[:, :1].contiguous(), torch.arange(5, dtype=torch.int64,
                                                                                          device=dev))
    with pytest.raises(ValueError):
        kvq.kvq_convert_cache(c, torch.zeros((3, 2, 16, 128), dtype=torch.bfloat16, device=dev),
                              torch.zeros((3, 2, 16, 128), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        kvq.kvq_calibrate_scales(x, "per_kv_head", "int8", torch.zeros(1, device=dev), torch.zeros(1, device=dev))
    torch.cuda.synchronize()


def test_rotated_keys_through_the_c_abi_alone():
    """KVQ_INT4_HAD keys, decode and two-token verify called straight through
    ctypes with the caller's plain query and softmax scale: the library rotates
    the query and folds 1 / head_dim in itself."""
    import ctypes
    from quantized_paged_kv_absmax_amd import _lib
    from oracle import attention as oa
    inp = make_decode_inputs(_workload("int4_had"), B=5, lens=("uniform", 30, 700))
    w = inp.w
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    lib = _lib.load()
    s = r.cache.struct()
    sm = softmax_scale(w.D)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B = w.B
    for n_q in (1, 2):
        inp2 = make_decode_inputs(w.with_(n_q=n_q))
        assert np.array_equal(inp2.k_bits, inp.k_bits)
        q = dev_bf16(inp2.q_bits)
        out = torch.empty((B * n_q, w.Hq, w.D), dtype=torch.float32, device="cuda")
        need = lib.kvq_verify_workspace_size(B, n_q, w.Hq, w.Hkv, w.D, inp.max_seq_len, 64)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
        args = (ctypes.byref(s), ctypes.c_void_p(q.data_ptr()))
        tail = (ctypes.c_void_p(r.bt.data_ptr()), r.bt.shape[1], ctypes.c_void_p(r.sl.data_ptr()), B,
                inp.max_seq_len, w.Hq, sm, 64, ctypes.c_void_p(ws.data_ptr()), ws.numel(), _lib.F32,
                ctypes.c_void_p(out.data_ptr()), None, stream)
        if n_q == 1:
            st = lib.kvq_paged_attention_decode(*args, *tail)
            ref = oa.decode(o, inp2.q_bits, inp.block_tables, inp.seq_lens, sm)
        else:
            st = lib.kvq_paged_attention_verify(*args, n_q, *tail)
            ref = oa.verify(o, inp2.q_bits, n_q, inp.block_tables, inp.seq_lens, sm)
        assert st == _lib.OK
        torch.cuda.synchronize()
        mx, nbad = gate_errors(out, ref, "f32")
        log(f"int4h through the C ABI, n_q={n_q}: max|err|={mx:.3e}")
        assert nbad == 0


def test_side_stream_call_keeps_its_own_temporaries():
    """A decode enqueued on a non-current stream, with the workspace and output
    allocated by the binding: those allocations belong to that stream, so
    tensors allocated and filled on the current stream right after the call
    cannot take their memory before the decode has run."""
    inp, r, o, ref = _setup("llama8b_int8")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        out = kvq.kvq_paged_attention_decode(r.cache, r.q, r.bt, r.sl, inp.max_seq_len, softmax_scale(inp.w.D),
                                             partition=64, out_dtype="f32", stream=side)
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(8)]   # on the current stream
        outs.append(out)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for out in outs:
        mx, nbad = gate_errors(out, ref, "f32")
        assert nbad == 0, mx
