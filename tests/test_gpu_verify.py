"""GPU parity of kvq_paged_attention_verify (several query tokens per sequence,
causal over the paged cache) against the oracle, through the C ABI: format
pairs, group sizes 1 to 16, tiles of 16 (token, head) columns that split a
token's heads, sequences shorter than the query block, and forced splits."""

import pytest
import torch

import quantized_paged_kv_absmax_amd as kvq
from tests.kvq_harness import (build_library_cache, build_oracle_cache, gate_errors, library_decode, log,
                               oracle_decode, softmax_scale)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu


def _small(kd, vd, Hq, Hkv, D, n_q, lens, seed=31):
    w = WORKLOADS["tiny_int8"].with_(B=len(lens), lens=("fixed", lens), Hq=Hq, Hkv=Hkv, D=D, k_dtype=kd,
                                     v_dtype=vd, seed=seed, n_q=n_q, new_tokens=0, calib="all")
    if kd in ("int4", "int4h"):
        w = w.with_(k_gran="per_token_head", v_gran="per_token_head", k_scale_mode="row", v_scale_mode="row",
                    calib="none")
    elif kd == "bf16":
        w = w.with_(k_scale_mode="one", v_scale_mode="one", calib="none")
    return w, make_decode_inputs(w)


# (K, V, Hq, Hkv, D, n_q): g = 4 with 16 tokens (4 tiles), g = 3 (a token's heads
# cut by a tile edge), g = 8 with odd n_q, g = 16 (one token per tile), g = 1,
# and 64 tokens
CASES = [
    ("int8", "int8", 8, 2, 128, 16),
    ("e4m3", "e5m2", 6, 2, 128, 7),
    ("int4", "int4", 16, 2, 128, 5),
    ("int4h", "int4", 8, 2, 128, 16),      # rotated keys: the query rows rotated alike
    ("bf16", "bf16", 16, 1, 64, 3),
    ("e4m3", "int8", 2, 2, 64, 20),
    ("int8", "e4m3", 8, 2, 128, 64),      # a prefill chunk: 16 tiles, 4 workgroups per (chunk, KV head)
]


@pytest.mark.parametrize("kd,vd,Hq,Hkv,D,n_q", CASES)
def test_verify_within_tolerance(kd, vd, Hq, Hkv, D, n_q):
    lens = (3, n_q, 17, 300, 1000, 1)            # shorter than the query block, equal to it, longer
    w, inp = _small(kd, vd, Hq, Hkv, D, n_q, lens)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    ref = oracle_decode(o, inp)
    for part in (0, 16, 64):
        for odt in ("f32", "bf16"):
            out = library_decode(r, inp, partition=part, out_dtype=odt)
            torch.cuda.synchronize()
            mx, bad = gate_errors(out, ref, odt)
            log(f"[verify {kd}/{vd} g={Hq // Hkv} n_q={n_q} D={D}] partition={part} out={odt} max|err|={mx:.3e}")
            assert bad == 0
    # rows whose position is below 0 (sequence 0 has 3 tokens) are zero
    out = library_decode(r, inp, partition=0, out_dtype="f32")
    assert (out[:n_q - 3] == 0).all()


def test_one_query_token_is_decode():
    w, inp = _small("int8", "int8", 8, 2, 128, 1, (5, 40, 700))
    r = build_library_cache(w, inp)
    sm = softmax_scale(w.D)
    for part in (0, 16):
        a = kvq.kvq_paged_attention_verify(r.cache, r.q, 1, r.bt, r.sl, inp.max_seq_len, sm, partition=part,
                                           out_dtype="f32")
        b = kvq.kvq_paged_attention_decode(r.cache, r.q, r.bt, r.sl, inp.max_seq_len, sm, partition=part,
                                           out_dtype="f32")
        assert torch.equal(a, b)


def test_each_query_token_is_a_truncated_decode():
    # token i of a sequence equals a one-token decode of the same query over the
    # first L - n_q + i + 1 positions (the library against itself, both splits)
    n_q = 6
    w, inp = _small("e4m3", "e4m3", 8, 2, 128, n_q, (20, 333, 64))
    r = build_library_cache(w, inp)
    sm = softmax_scale(w.D)
    out = kvq.kvq_paged_attention_verify(r.cache, r.q, n_q, r.bt, r.sl, inp.max_seq_len, sm, out_dtype="f32")
    for i in range(n_q):
        lens = (r.sl - n_q + i + 1).to(torch.int32).contiguous()
        q_i = r.q[i::n_q].contiguous()
        d = kvq.kvq_paged_attention_decode(r.cache, q_i, r.bt, lens, inp.max_seq_len, sm, out_dtype="f32")
        torch.cuda.synchronize()
        diff = (out[i::n_q] - d).abs().max().item()
        assert diff <= 2e-5, (i, diff)


def test_verify16_workload_reduced():
    w = WORKLOADS["verify16_int8"]
    inp = make_decode_inputs(w, B=6, lens=("uniform", 16, 1500))
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    ref = oracle_decode(o, inp)
    for part in (0, 512):
        out = library_decode(r, inp, partition=part, out_dtype="bf16")
        torch.cuda.synchronize()
        mx, bad = gate_errors(out, ref, "bf16")
        log(f"[verify16_int8 B=6] partition={part} max|err|={mx:.3e}")
        assert bad == 0


# many (token, head) rows with few pieces each: the reduce takes one lane group
# per row, workgroups of 8 (D = 128) or 16 (D = 64) rows; the second case leaves
# a partly filled workgroup (138 rows a sequence) and sequences shorter than n_q
ROW_CASES = [
    ("int8", "int8", 32, 8, 128, 16, 24, (1, 700)),
    ("e4m3", "e5m2", 6, 2, 64, 23, 72, (1, 200)),
]


@pytest.mark.parametrize("kd,vd,Hq,Hkv,D,n_q,B,lens", ROW_CASES)
def test_verify_many_rows(kd, vd, Hq, Hkv, D, n_q, B, lens):
    w = WORKLOADS["tiny_int8"].with_(B=B, lens=("uniform",) + lens, Hq=Hq, Hkv=Hkv, D=D, k_dtype=kd, v_dtype=vd,
                                     seed=41, n_q=n_q, new_tokens=0, calib="all")
    inp = make_decode_inputs(w)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    ref = oracle_decode(o, inp)
    for odt in ("f32", "bf16"):
        out = library_decode(r, inp, partition=0, out_dtype=odt)
        torch.cuda.synchronize()
        mx, bad = gate_errors(out, ref, odt)
        log(f"[verify rows {kd}/{vd} B={B} n_q={n_q} Hq={Hq} D={D}] out={odt} max|err|={mx:.3e}")
        assert bad == 0


@pytest.mark.parametrize("B", [64, 9])
def test_verify16_repeated_calls_bit_identical(B):
    """The several-token kernel at the verify16_int8 shape (four waves sharing each
    round through LDS, two barriers per round): eight calls through one workspace
    are bit-identical, and within the oracle gate on a reduced batch.  A round read
    before every wave's share of it had landed, or refilled before every wave had
    read it, would change a piece from call to call."""
    w = WORKLOADS["verify16_int8"]
    inp = make_decode_inputs(w, B=B)
    log(f"[verify16 repeat] B={B} lens={inp.seq_lens.tolist()[:8]}")
    r = build_library_cache(w, inp)
    need = kvq.kvq_verify_workspace_size(B, w.n_q, w.Hq, w.Hkv, w.D, inp.max_seq_len, 0)
    ws = torch.full((max(need, 16),), 0x7F, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(8):
        out = torch.full((B * w.n_q, w.Hq, w.D), float("nan"), device="cuda")
        kvq.kvq_paged_attention_verify(r.cache, r.q, w.n_q, r.bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                       partition=0, workspace=ws, out_dtype="f32", out=out)
        torch.cuda.synchronize()
        outs.append(out)
    for i, out in enumerate(outs[1:], 1):
        assert torch.equal(out, outs[0]), i
    assert torch.isfinite(outs[0]).all()
    if B <= 9:
        o = build_oracle_cache(w, inp)
        mx, nbad = gate_errors(outs[0], oracle_decode(o, inp), "f32")
        log(f"[verify16 repeat] B={B} max|err|={mx:.3e}")
        assert nbad == 0
