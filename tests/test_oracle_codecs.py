"""Pins of the oracle's element codecs against definitions, brute force and torch."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# FP8 decode
# ---------------------------------------------------------------------------

# named codes of the OCP 8-bit formats: (code, value)
E4M3_POINTS = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
               (0x38, 1.0), (0x39, 1.125), (0x7E, 448.0), (0x7D, 416.0), (0xB8, -1.0), (0xFE, -448.0)]
E5M2_POINTS = [(0x00, 0.0), (0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16), (0x04, 2.0 ** -14),
               (0x3C, 1.0), (0x3D, 1.25), (0x7B, 57344.0), (0x7A, 49152.0), (0xBC, -1.0), (0xFB, -57344.0)]


@pytest.mark.parametrize("fmt,points", [("e4m3", E4M3_POINTS), ("e5m2", E5M2_POINTS)])
def test_fp8_named_codes(fmt, points):
    tab = codecs.fp8_decode_table(fmt)
    for code, val in points:
        assert tab[code] == val, (fmt, hex(code))
    assert np.signbit(tab[0x80]) and tab[0x80] == 0.0


def test_fp8_special_code_sets():
    e4 = codecs.fp8_decode_table("e4m3")
    assert set(np.nonzero(np.isnan(e4))[0]) == {0x7F, 0xFF}
    assert not np.isinf(e4).any()
    e5 = codecs.fp8_decode_table("e5m2")
    assert set(np.nonzero(np.isnan(e5))[0]) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert e5[0x7C] == np.inf and e5[0xFC] == -np.inf
    for tab, top in ((e4, 0x7E), (e5, 0x7B)):
        pos = tab[: top + 1]
        assert np.all(np.diff(pos) > 0)                 # positive codes increase strictly
        assert np.array_equal(tab[0x80: 0x80 + top + 1], -pos)  # sign-magnitude


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decode_matches_torch_views(fmt, tdt):
    tab = codecs.fp8_decode_table(fmt)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(tdt).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert np.array_equal(ref[~nan], tab[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(tab[~nan]))


# ---------------------------------------------------------------------------
# FP8 encode: brute-force nearest with even tie rule, over all 65536 bf16 inputs
# ---------------------------------------------------------------------------


def _brute_force_fp8(t, fmt):
    """Nearest finite code of the same sign; ties -> code with LSB 0; NaN -> NaN code."""
    tab = codecs.fp8_decode_table(fmt)
    codes = np.arange(256)
    out = np.zeros(t.shape, np.int64)
    t64 = t.astype(np.float64)
    for sign in (0, 1):
        cand = codes[(np.isfinite(tab)) & ((codes >> 7) == sign)]
        vals = tab[cand]
        sel = (np.signbit(t) == bool(sign)) & np.isfinite(t)
        tt = t64[sel]
        for c0 in range(0, tt.size, 4096):
            chunk = tt[c0:c0 + 4096]
            # |t - v| is exact in float64 while |t| < 2^36; above the largest
            # candidate, t - v = (t - vmax) + (vmax - v) and the first term is
            # common to all candidates, so (vmax - v) ranks them exactly
            vmax = np.abs(vals).max()
            far = np.abs(chunk)[:, None] > vmax
            dist = np.where(far, vmax - np.abs(vals)[None, :], np.abs(chunk[:, None] - vals[None, :]))
            best = dist.min(axis=1, keepdims=True)
            tie = dist == best
            # prefer an even code among the tied minima
            score = np.where(tie, 1 + (cand[None, :] & 1), 99)
            idx = np.argmin(score, axis=1)
            o = np.nonzero(sel)[0][c0:c0 + 4096]
            out[o] = cand[idx]
    return out


ALL_BF16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.75e-3, 17.5])
def test_fp8_encode_exhaustive_bf16(fmt, scale):
    x = ALL_BF16
    got = codecs.fp8_encode(x, np.float32(scale), fmt).astype(np.int64)
    t = np.divide(x, np.float32(scale), dtype=np.float32)
    fin = np.isfinite(t)
    ref = _brute_force_fp8(t, fmt)
    assert np.array_equal(got[fin], ref[fin])
    # infinities saturate to the largest finite code of their sign
    top = codecs.FP8_FORMATS[fmt]["maxcode"]
    inf = np.isinf(t)
    assert np.array_equal(got[inf], np.where(t[inf] > 0, top, 0x80 | top))
    # NaN inputs give a NaN code
    assert codecs.fp8_is_nan_code(got[np.isnan(t)].astype(np.uint8), fmt).all()


def test_fp8_encode_named_ties():
    # ties go to the even code (values between neighbours that differ in the LSB)
    e = lambda v: int(codecs.fp8_encode_value(np.float32(v), "e4m3"))
    assert e(1.0625) == 0x38          # between 1.0 (0x38) and 1.125 (0x39)
    assert e(1.1875) == 0x3A          # between 1.125 (0x39) and 1.25 (0x3A)
    assert e(1.5 * 2.0 ** -9) == 0x02  # subnormal tie between 0x01 and 0x02
    assert e(2.0 ** -10) == 0x00      # half the smallest subnormal -> +0
    assert e(-(2.0 ** -10)) == 0x80   # ... keeps its sign
    assert e(460.0) == 0x7E and e(1e9) == 0x7E and e(-1e9) == 0xFE
    f = lambda v: int(codecs.fp8_encode_value(np.float32(v), "e5m2"))
    assert f(61440.0) == 0x7B         # the tie above the largest finite saturates
    assert f(1.125) == 0x3C           # tie between 1.0 and 1.25 -> even 0x3C
    assert f(-0.0) == 0x80


@pytest.mark.parametrize("fmt,tdt,lim", [("e4m3", torch.float8_e4m3fn, 464.0), ("e5m2", torch.float8_e5m2, 61440.0)])
def test_fp8_encode_matches_torch_cast_in_range(fmt, tdt, lim):
    rng = np.random.default_rng(11)
    t = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(lim / 8),
        rng.standard_normal(200000).astype(np.float32) * np.float32(2.0 ** -8),
        ALL_BF16[np.isfinite(ALL_BF16)],
    ])
    t = t[np.abs(t) < lim]
    got = codecs.fp8_encode_value(t, fmt)
    ref = torch.from_numpy(t).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# INT8
# ---------------------------------------------------------------------------


def test_int8_named_cases():
    x = np.array([2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5, 127.5, 200.0, -127.5, -200.0, np.inf, -np.inf, np.nan], np.float32)
    want = [2, 4, -2, 0, 0, 2, 126, 127, 127, -127, -127, 127, -127, 0]
    assert codecs.int8_encode(x, np.float32(1.0)).tolist() == want
    # -128 is never produced
    assert codecs.int8_encode(np.float32(-1e30), np.float32(1.0)) == -127


def test_int8_division_is_correctly_rounded():
    # the float32 quotient must equal the float64 quotient rounded once to float32
    # (exact for float32 operands: 53 >= 2*24 + 2), not x * (1/s)
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000).astype(np.float32)
    s = np.float32(rng.uniform(0.001, 0.1))
    t = codecs._div32(x, s)
    ref = (x.astype(np.float64) / np.float64(s)).astype(np.float32)
    assert np.array_equal(t, ref)
    # one hand-checked quotient: 1/3 in float32
    q = codecs._div32(np.float32(1.0), np.float32(3.0))
    assert Fraction(float(q)) == Fraction(11184811, 33554432)


def test_int8_round_trip_bound():
    rng = np.random.default_rng(5)
    for s in (np.float32(0.01), np.float32(0.0375), np.float32(1.7)):
        x = (rng.uniform(-127, 127, 50000) * s).astype(np.float32)
        xh = codecs.int8_decode(codecs.int8_encode(x, s), s)
        err = np.abs(x.astype(np.float64) - xh.astype(np.float64))
        assert err.max() <= float(s) / 2 * (1 + 2 ** -20) + np.spacing(np.float32(127 * s))


# ---------------------------------------------------------------------------
# INT4 asymmetric
# ---------------------------------------------------------------------------


def test_int4_hand_example():
    x = np.array([[-1.0, 0.5, 2.0, 2.0]], np.float32)
    codes, s, zp = codecs.int4_encode_rows(x)
    assert s[0] == np.float32(0.2)           # fl32(3 / 15)
    assert zp[0] == 5.0                      # RNE(1 / 0.2f) = RNE(4.99999997)
    assert codes[0].tolist() == [0, 7, 15, 15]
    assert codecs.int4_pack(codes)[0].tolist() == [0x70, 0xFF]


def test_int4_pack_order():
    c = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    p = codecs.int4_pack(c)
    assert p[0].tolist() == [0x21, 0x43, 0x0F]
    assert np.array_equal(codecs.int4_unpack(p), c)


def test_int4_invariants():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3000, 128)).astype(np.float32)
    x[:, 7] *= 8
    x[::7] = np.abs(x[::7]) + np.float32(3.0)   # rows entirely positive -> zero point below 0
    codes, s, zp = codecs.int4_encode_rows(x)
    assert codes.max() <= 15
    rows = np.arange(len(x))
    # RNE is odd-symmetric, so the row minimum always lands on code 0
    assert (codes[rows, x.argmin(axis=1)] == 0).all()
    top = codes[rows, x.argmax(axis=1)]
    assert (top >= 14).all() and (top == 15).mean() > 0.99
    assert (zp[::7] < 0).all()
    xh = codecs.int4_decode(codes, s, zp)
    err = np.abs(x.astype(np.float64) - xh) / s[:, None]
    assert err.max() <= 0.5 + 1e-5


def test_int4_constant_rows_exact():
    x = np.array([[0.0] * 8, [3.5] * 8, [-2.25] * 8, [1e-30] * 8], np.float32)
    codes, s, zp = codecs.int4_encode_rows(x)
    assert np.array_equal(codecs.int4_decode(codes, s, zp), x)


# ---------------------------------------------------------------------------
# byte accounting, pinned to the L4 table of vLLM PR 4893
# ---------------------------------------------------------------------------


def test_bytes_ratios():
    D = 128
    bf = codecs.kv_bytes_per_token_head("bf16", "bf16", D)
    assert bf == 512
    assert codecs.kv_bytes_per_token_head("int8", "int8", D) / bf == 0.5
    assert codecs.kv_bytes_per_token_head("e4m3", "e4m3", D) / bf == 0.5
    assert codecs.kv_bytes_per_token_head("e4m3", "int8", D) / bf == 0.5
    assert codecs.kv_bytes_per_token_head("int4", "int4", D) / bf == 0.28125   # "roughly a quarter"


def test_block_ratio_matches_l4_table():
    rows = json.load(open(os.path.join(GOLDEN, "l4_gpu_blocks.json")))["rows"]
    by = {(r["model_dtype"], r["kv_dtype"]): r["gpu_blocks"] for r in rows}
    printed = [by[("FP16", "FP8_e5m2")] / by[("FP16", "FP16")],
               by[("FP8_e4m3", "FP8_e4m3")] / by[("FP8_e4m3", "FP16")]]
    # Llama-3-8B: 32 layers, 8 KV heads, head dim 128, block 16.  The budget is
    # the FP16-KV pool of the first row; an 8-bit KV pool of equal bytes holds:
    per_fp16_block = codecs.kv_bytes_per_token_head("bf16", "bf16", 128) * 8 * 32 * 16
    for base_blocks, ratio in ((by[("FP16", "FP16")], printed[0]), (by[("FP8_e4m3", "FP16")], printed[1])):
        budget = base_blocks * per_fp16_block
        n16 = codecs.blocks_in_budget(budget, "bf16", "bf16", 128, 8, 32)
        n8 = codecs.blocks_in_budget(budget, "e5m2", "e5m2", 128, 8, 32)
        assert n16 == base_blocks
        assert n8 / n16 == ratio == 2.0


# ---- Hadamard rotation (KVarN's rotation step) ----

def _bf16_bits(x):
    return codecs.f32_to_bf16_rne(np.asarray(x, np.float32))


@pytest.mark.parametrize("D", [64, 128])
def test_hadamard_matches_sylvester_matrix(D):
    from scipy.linalg import hadamard
    H = hadamard(D).astype(np.float64)
    rng = np.random.default_rng(11)
    xi = rng.integers(-2, 3, size=(40, D)).astype(np.float32)        # exact in bf16 and in the sums
    got = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(_bf16_bits(xi))).astype(np.float64)
    assert np.array_equal(got, xi.astype(np.float64) @ H.T)
    xr = codecs.bf16_to_f32(_bf16_bits(rng.standard_normal((200, D)) * 3.0))
    ref = xr.astype(np.float64) @ H.T
    got = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(_bf16_bits(xr))).astype(np.float64)
    # bf16 rounding of the result (2^-9 relative) plus float32 sums (about 2^-24 * D * max|x|)
    bound = np.abs(ref) * 2.0 ** -8 + 2.0 ** -20 * D * np.abs(xr).max(axis=-1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)


def test_hadamard_twice_is_D_times_identity_and_columns():
    D = 128
    rng = np.random.default_rng(12)
    x = rng.integers(-2, 3, size=(30, D)).astype(np.float32)
    once = codecs.hadamard_rotate_bf16(_bf16_bits(x))
    twice = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(once))
    assert np.array_equal(twice, D * x)
    eye = np.eye(D, dtype=np.float32)
    cols = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(_bf16_bits(eye)))
    i, k = np.meshgrid(np.arange(D), np.arange(D), indexing="ij")
    pop = np.vectorize(lambda v: bin(v).count("1"))(i & k)
    assert np.array_equal(cols, np.where(pop % 2 == 0, 1.0, -1.0).astype(np.float32))


def test_hadamard_preserves_dot_products():
    D = 64
    rng = np.random.default_rng(13)
    q = rng.integers(-2, 3, size=(20, D)).astype(np.float32)
    k = rng.integers(-2, 3, size=(20, D)).astype(np.float32)
    hq = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(_bf16_bits(q))).astype(np.float64)
    hk = codecs.bf16_to_f32(codecs.hadamard_rotate_bf16(_bf16_bits(k))).astype(np.float64)
    assert np.array_equal((hq * hk).sum(-1), D * (q.astype(np.float64) * k).sum(-1))
