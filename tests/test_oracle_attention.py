"""Pins of the oracle's paged decode: closed forms, invariants and torch SDPA."""

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import codecs
from workloads import WORKLOADS, make_decode_inputs


def _cache(inp, kd="int8", vd="int8", ks=0.05, vs=0.04):
    w = inp.w
    c = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, kd, vd, k_scale=ks, v_scale=vs)
    c.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    return c


def _inputs(B=3, lens=("fixed", (1, 40, 77)), Hq=8, Hkv=2, D=64):
    w = WORKLOADS["tiny_int8"].with_(B=B, lens=lens, Hq=Hq, Hkv=Hkv, D=D)
    return make_decode_inputs(w)


def test_zero_query_gives_mean_of_v():
    inp = _inputs()
    c = _cache(inp)
    q0 = np.zeros_like(inp.q_bits)
    out = oa.decode(c, q0, inp.block_tables, inp.seq_lens, 0.125)
    g = inp.w.Hq // inp.w.Hkv
    for b in range(inp.w.B):
        V = c.gather(inp.block_tables[b], int(inp.seq_lens[b]), "v").astype(np.float64)
        for h in range(inp.w.Hq):
            np.testing.assert_allclose(out[b, h], V[:, h // g, :].mean(axis=0), rtol=0, atol=1e-14)


def test_single_token_gives_its_value():
    inp = _inputs(B=2, lens=("fixed", (1, 1)))
    c = _cache(inp, "e4m3", "int4")
    out = oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    g = inp.w.Hq // inp.w.Hkv
    for b in range(2):
        v0 = c.gather(inp.block_tables[b], 1, "v")[0].astype(np.float64)
        for h in range(inp.w.Hq):
            assert np.array_equal(out[b, h], v0[h // g])


def test_constant_logit_shift_changes_nothing():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((50, 64))
    V = rng.standard_normal((50, 64))
    q = rng.standard_normal(64)
    u = rng.standard_normal(64) * 3          # adds softmax_scale * (u . q) to every logit
    a = oa._attend(q, K, V, 0.125)
    b = oa._attend(q, K + u, V, 0.125)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_permuted_pool_is_bit_identical():
    inp = _inputs()
    c1 = _cache(inp)
    o1 = oa.decode(c1, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    # relabel every physical block through a permutation
    rng = np.random.default_rng(8)
    perm = rng.permutation(inp.num_blocks)
    bt = np.where(inp.block_tables >= 0, perm[np.maximum(inp.block_tables, 0)], -1).astype(np.int32)
    slots = perm[inp.slot_mapping // 16] * 16 + inp.slot_mapping % 16
    c2 = oc.PagedCache(inp.num_blocks, inp.w.Hkv, inp.w.D, "int8", "int8", k_scale=0.05, v_scale=0.04)
    c2.write(inp.k_bits, inp.v_bits, slots)
    o2 = oa.decode(c2, inp.q_bits, bt, inp.seq_lens, 0.125)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("kd,vd", [("int8", "int8"), ("e5m2", "e4m3"), ("int4", "int4"), ("bf16", "bf16")])
def test_matches_torch_sdpa_fp64(kd, vd):
    inp = _inputs()
    c = _cache(inp, kd, vd)
    sm = float(np.float32(1 / np.sqrt(64)))
    out = oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, sm)
    g = inp.w.Hq // inp.w.Hkv
    q = torch.from_numpy(codecs.bf16_to_f32(inp.q_bits).astype(np.float64))
    for b in range(inp.w.B):
        L = int(inp.seq_lens[b])
        K = torch.from_numpy(c.gather(inp.block_tables[b], L, "k").astype(np.float64))   # [L][Hkv][D]
        V = torch.from_numpy(c.gather(inp.block_tables[b], L, "v").astype(np.float64))
        K = K.permute(1, 0, 2).repeat_interleave(g, dim=0)                               # [Hq][L][D]
        V = V.permute(1, 0, 2).repeat_interleave(g, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q[b][:, None, :], K, V, scale=sm)[:, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_split_equals_unsplit():
    inp = _inputs(B=4, lens=("fixed", (5, 16, 100, 257)))
    c = _cache(inp, "e4m3", "int8")
    o = oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    for part in (16, 32, 64, 512):
        s = oa.decode_split(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125, part)
        np.testing.assert_allclose(s, o, rtol=1e-12, atol=1e-13)


def test_unused_slots_and_empty_sequences():
    inp = _inputs(B=3, lens=("fixed", (3, 0, 17)))
    c = _cache(inp, "e4m3", "e4m3")
    # every slot not written holds 0xFF, a NaN code for e4m3: it must not leak
    out = oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    assert np.isfinite(out).all()
    assert (out[1] == 0).all()


def test_gqa_equals_repeated_kv_heads():
    inp = _inputs()
    c = _cache(inp)
    out = oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    g = inp.w.Hq // inp.w.Hkv
    rep = oc.PagedCache(inp.num_blocks, inp.w.Hq, inp.w.D, "int8", "int8", k_scale=0.05, v_scale=0.04)
    rep.write(np.repeat(inp.k_bits, g, axis=1), np.repeat(inp.v_bits, g, axis=1), inp.slot_mapping)
    out2 = oa.decode(rep, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125)
    assert np.array_equal(out, out2)


# ---------------------------------------------------------------------------
# several query tokens per sequence (causal)
# ---------------------------------------------------------------------------


def _verify_q(inp, n_q, seed=21):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((inp.w.B * n_q, inp.w.Hq, inp.w.D)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kd,vd", [("int8", "int8"), ("e4m3", "e5m2"), ("int4", "int4")])
def test_verify_matches_torch_sdpa_causal_fp64(kd, vd):
    # torch's scaled_dot_product_attention with an explicit mask: query token i of
    # sequence b (position L - n_q + i) sees cache positions 0..L - n_q + i
    inp = _inputs(B=3, lens=("fixed", (5, 40, 77)))
    c = _cache(inp, kd, vd)
    n_q = 5
    qb = _verify_q(inp, n_q)
    sm = float(np.float32(1 / np.sqrt(64)))
    out = oa.verify(c, qb, n_q, inp.block_tables, inp.seq_lens, sm)
    g = inp.w.Hq // inp.w.Hkv
    q = torch.from_numpy(codecs.bf16_to_f32(qb).astype(np.float64))
    for b in range(inp.w.B):
        L = int(inp.seq_lens[b])
        K = torch.from_numpy(c.gather(inp.block_tables[b], L, "k").astype(np.float64))
        V = torch.from_numpy(c.gather(inp.block_tables[b], L, "v").astype(np.float64))
        K = K.permute(1, 0, 2).repeat_interleave(g, dim=0)                   # [Hq][L][D]
        V = V.permute(1, 0, 2).repeat_interleave(g, dim=0)
        pos = torch.arange(L - n_q, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos                                # [n_q][L]
        qq = q[b * n_q:(b + 1) * n_q].permute(1, 0, 2)                         # [Hq][n_q][D]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, K, V, attn_mask=mask, scale=sm)
        np.testing.assert_allclose(out[b * n_q:(b + 1) * n_q], ref.permute(1, 0, 2).numpy(), rtol=1e-12,
                                   atol=1e-12)


def test_verify_rows_are_truncated_decodes():
    # row i of sequence b is the single-query decode of query i over the first
    # L - n_q + i + 1 positions; one query token per sequence is the decode itself
    inp = _inputs(B=3, lens=("fixed", (3, 40, 77)))
    c = _cache(inp, "e4m3", "int8")
    n_q = 4
    qb = _verify_q(inp, n_q)
    out = oa.verify(c, qb, n_q, inp.block_tables, inp.seq_lens, 0.125)
    for i in range(n_q):
        lens = inp.seq_lens - n_q + i + 1
        ref = oa.decode(c, qb[i::n_q], inp.block_tables, lens, 0.125)
        assert np.array_equal(out[i::n_q], ref), i
    one = oa.verify(c, inp.q_bits, 1, inp.block_tables, inp.seq_lens, 0.125)
    assert np.array_equal(one, oa.decode(c, inp.q_bits, inp.block_tables, inp.seq_lens, 0.125))
    # sequence 0 has 3 tokens: its first query token (position -1) sees nothing
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()


def test_verify_zero_query_gives_prefix_mean():
    inp = _inputs(B=2, lens=("fixed", (20, 33)))
    c = _cache(inp)
    n_q = 3
    q0 = np.zeros((inp.w.B * n_q, inp.w.Hq, inp.w.D), np.uint16)
    out = oa.verify(c, q0, n_q, inp.block_tables, inp.seq_lens, 0.125)
    g = inp.w.Hq // inp.w.Hkv
    for b in range(2):
        L = int(inp.seq_lens[b])
        V = c.gather(inp.block_tables[b], L, "v").astype(np.float64)
        for i in range(n_q):
            for h in range(inp.w.Hq):
                np.testing.assert_allclose(out[b * n_q + i, h], V[:L - n_q + i + 1, h // g].mean(axis=0),
                                           rtol=0, atol=1e-14)


def test_rotated_keys_equal_derotated_attention():
    """An "int4h" cache stores INT4 codes of H k; its decode attends with the
    de-rotated keys H k_hat_rot / D and the query as given.  The same logits come
    from the other side of the identity, (H q) . k_hat_rot / D: torch's
    scaled_dot_product_attention in float64 over the stored rows with the
    rotated query (scipy's Hadamard matrix) and the scale divided by D.  A
    missing 1 / D, an unrotated or transposed rotation fails it."""
    from scipy.linalg import hadamard
    inp = _inputs(B=2, lens=("fixed", (9, 40)), Hq=4, Hkv=2, D=64)
    c = oc.PagedCache(inp.num_blocks, 2, 64, "int4h", "int4")
    c.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    rng = np.random.default_rng(14)
    q = rng.standard_normal(inp.q_bits.shape).astype(np.float32)
    q_bits = codecs.f32_to_bf16_rne(q)
    out = oa.decode(c, q_bits, inp.block_tables, inp.seq_lens, 0.125)
    qf = codecs.bf16_to_f32(q_bits).astype(np.float64)
    H = hadamard(64).astype(np.float64)
    for b in range(2):
        L = int(inp.seq_lens[b])
        Kr = c.gather(inp.block_tables[b], L, "k").astype(np.float64)        # the stored rows: H k, dequantised
        V = c.gather(inp.block_tables[b], L, "v").astype(np.float64)
        hq = qf[b] @ H.T                                                    # H q per head
        for h in range(4):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(hq[h][None, None, None, :]), torch.from_numpy(Kr[None, None, :, h // 2, :]),
                torch.from_numpy(V[None, None, :, h // 2, :]), scale=0.125 / 64).numpy()[0, 0, 0]
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
    # and the stored codes are those of the rotated rows
    plain = oc.PagedCache(inp.num_blocks, 2, 64, "int4", "int4")
    plain.write(codecs.hadamard_rotate_bf16(inp.k_bits), inp.v_bits, inp.slot_mapping)
    assert np.array_equal(plain.k_pages, c.k_pages)
    assert np.array_equal(plain.k_meta, c.k_meta, equal_nan=True)
