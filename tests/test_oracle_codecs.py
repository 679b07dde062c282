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


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_exact_ties_follow_the_quotient(fmt):
    """x / s exactly halfway between two adjacent finite codes (x = t s exact in
    float32: t has at most 5 significant bits, s 16) encodes to the code whose
    mantissa LSB is 0.  A product by the rounded reciprocal, x * fl32(1 / s),
    misses some of these ties in the last bit: the cases include such ties, so
    only the correctly rounded quotient passes."""
    tab = codecs.fp8_decode_table(fmt)
    top = 0x7E if fmt == "e4m3" else 0x7B
    rng = np.random.default_rng(13)
    xs, ss, want, flips = [], [], [], 0
    for _ in range(3000):
        c = int(rng.integers(0, top))                 # the tie between codes c and c + 1
        t = Fraction(tab[c]) / 2 + Fraction(tab[c + 1]) / 2
        neg = bool(rng.integers(0, 2))
        m, e = np.frexp(np.float64(rng.uniform(0.001, 0.2)))
        s = np.float32(np.ldexp(np.round(m * 2 ** 16) / 2 ** 16, e))
        x = np.float32(float((-t if neg else t) * Fraction(float(s))))
        assert Fraction(float(x)) == (-t if neg else t) * Fraction(float(s))   # an exact tie
        code = (c if c % 2 == 0 else c + 1) | (0x80 if neg else 0)
        xs.append(x)
        ss.append(s)
        want.append(code)
        flips += int(codecs.fp8_encode_value(np.float32(x * np.float32(np.float32(1.0) / s)), fmt) != code)
    assert flips > 0
    got = codecs.fp8_encode(np.array(xs, np.float32), np.array(ss, np.float32), fmt)
    assert got.tolist() == want


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_round_trip_bound(fmt):
    """Decoding the code of x at scale s gives x back to within half the code
    spacing at x / s, times s: relative 2^-(m+1) for normal values (m mantissa
    bits), half a subnormal step below the normal range (plus the float32
    roundings of the quotient and the product).  Named values: the code of 1.0
    decodes to s itself."""
    f = codecs.FP8_FORMATS[fmt]
    mb, bias, maxval = f["mbits"], f["bias"], f["maxval"]
    rng = np.random.default_rng(21)
    for s in (np.float32(0.013), np.float32(0.25), np.float32(3.5)):
        x = (rng.uniform(-1, 1, 40000) * maxval * s).astype(np.float32)
        x[:100] *= np.float32(2.0 ** -12)          # some in the subnormal range
        xh = codecs.fp8_decode(codecs.fp8_encode(x, s, fmt), s, fmt).astype(np.float64)
        err = np.abs(xh - x.astype(np.float64))
        bound = (np.abs(x.astype(np.float64)) * 2.0 ** -(mb + 1) + float(s) * 2.0 ** (-bias - mb)) * (1 + 2.0 ** -20)
        assert (err <= bound).all()
        one = 0x38 if fmt == "e4m3" else 0x3C
        assert codecs.fp8_decode(np.array([one, one | 0x80], np.uint8), s, fmt).tolist() == [float(s), -float(s)]


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


def test_int8_exact_ties_follow_the_quotient():
    """Codes at exact ties x / s = n + 1/2 (x = (n + 1/2) s exact in float32: s
    has 16 significant bits) round to the even integer.  A product by the
    rounded reciprocal, x * fl32(1 / s), misses some of these ties in the last
    bit and rounds them the other way: the cases below include such ties, so
    only the correctly rounded quotient passes."""
    rng = np.random.default_rng(11)
    xs, ss, want, flips = [], [], [], 0
    for _ in range(4000):
        m, e = np.frexp(np.float64(rng.uniform(0.001, 0.2)))
        s = np.float32(np.ldexp(np.round(m * 2 ** 16) / 2 ** 16, e))
        n = int(rng.integers(-127, 127))
        x = np.float32((n + 0.5) * float(s))
        assert Fraction(float(x)) == (n + Fraction(1, 2)) * Fraction(float(s))   # an exact tie
        xs.append(x)
        ss.append(s)
        want.append(n if n % 2 == 0 else n + 1)                                   # the even neighbour
        flips += int(np.rint(np.float32(x * np.float32(np.float32(1.0) / s))) != want[-1])
    assert flips > 0
    got = codecs.int8_encode(np.array(xs, np.float32), np.array(ss, np.float32))
    assert got.tolist() == want


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


def test_int4_zero_zero_point_is_positive_zero():
    """Rows whose minimum is a zero (either sign, or both present) store zp = +0."""
    x = np.array([[-0.0, 0.0, 1.0, 2.0], [0.0, -0.0, 3.0, 0.5], [-0.0, -0.0, 1.0, 1.0]], np.float32)
    _, s, zp = codecs.int4_encode_rows(x)
    assert (zp.view(np.uint32) == 0).all()


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


def test_blocks_in_budget_counts_whole_blocks():
    """Only whole blocks count: one byte short of n blocks holds n - 1."""
    per = codecs.kv_bytes_per_token_head("int8", "int8", 128) * 8 * 32 * 16    # 1 MiB a block
    assert per == 1 << 20
    assert codecs.blocks_in_budget(5 * per, "int8", "int8", 128, 8, 32) == 5
    assert codecs.blocks_in_budget(5 * per - 1, "int8", "int8", 128, 8, 32) == 4
    assert codecs.blocks_in_budget(per - 1, "int8", "int8", 128, 8, 32) == 0


# ---- Hadamard rotation (KVarN's rotation step) ----

def _bf16_bits(x):
    return codecs.f32_to_bf16_rne(np.asarray(x, np.float32))


ALL_BF16_BITS = np.arange(65536, dtype=np.uint32).astype(np.uint16)
_FIN = ALL_BF16_BITS[((ALL_BF16_BITS >> 7) & 0xFF) != 0xFF]
_FIN_VALS = codecs.bf16_to_f32(_FIN).astype(np.float64)


def _nearest_bf16_brute(y):
    """bf16 bits nearest to the exact rational y (a Fraction), found by search
    over every finite bf16 value; ties go to the pattern with an even last
    mantissa bit; at or beyond the halfway point above the largest finite
    value, +-Inf.  Zero gives +0."""
    if y == 0:
        return 0
    big = Fraction(2) ** 128 - Fraction(2) ** 119      # halfway between the largest finite and 2^128
    if y >= big:
        return 0x7F80
    if y <= -big:
        return 0xFF80
    fy = float(y)
    # candidates: the finite values around float(y) (float(y) is within an ulp of y)
    idx = np.argsort(np.abs(_FIN_VALS - fy))[:6]
    best, bestd = None, None
    for i in idx:
        v = Fraction(float(_FIN_VALS[i]))
        d = abs(y - v)
        b = int(_FIN[i])
        if v == 0 and b == 0x8000:
            continue
        if best is None or d < bestd or (d == bestd and (b & 1) == 0 and (best & 1) == 1):
            best, bestd = b, d
    return best


def _exact_rotation(bits):
    """y = H x in exact rational arithmetic with scipy's Hadamard matrix."""
    from scipy.linalg import hadamard
    D = bits.shape[-1]
    H = hadamard(D)
    x = [Fraction(float(v)) for v in codecs.bf16_to_f32(bits).astype(np.float64)]
    return [sum((int(H[j, i]) * x[i] for i in range(D)), Fraction(0)) for j in range(D)]


@pytest.mark.parametrize("D", [64, 128])
def test_hadamard_matches_library_matrix_and_torch_rounding(D):
    """Rows of multiples of 2^-6 below 4 in magnitude: every exact H x is then an
    integer multiple of 2^-6 below 2^9, exact in float64 and in float32, so
    scipy's Hadamard matrix in float64 gives it and torch's float32 -> bf16 cast
    (round to nearest even) is the single rounding.  Many results are exact
    ties at bf16's 8 significant bits."""
    from scipy.linalg import hadamard
    rng = np.random.default_rng(11)
    k = rng.integers(-255, 256, size=(400, D))
    xr = (k * 2.0 ** -6).astype(np.float32)
    bits = _bf16_bits(xr)
    assert np.array_equal(codecs.bf16_to_f32(bits), xr)          # inputs exact in bf16
    ref64 = xr.astype(np.float64) @ hadamard(D).T.astype(np.float64)
    ref32 = ref64.astype(np.float32)
    assert np.array_equal(ref32.astype(np.float64), ref64)       # exact in float32
    want = torch.from_numpy(ref32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = np.where(ref32 == 0, np.uint16(0), want)              # an exact zero is +0
    got = codecs.hadamard_rotate_bf16(bits)
    assert np.array_equal(got, want)
    # ties were exercised: results exactly halfway between two bf16 values
    r = ref32.view(np.uint32)
    assert ((r & 0xFFFF) == 0x8000).sum() > 100


def test_hadamard_brute_force_on_wide_rows():
    """Rows whose magnitudes span up to 2^120 (beyond any float64 evaluation,
    through the arbitrary-precision path) and ordinary rows: each output equals
    the nearest bf16 of the exact rational result, found by search."""
    rng = np.random.default_rng(21)
    D = 64
    rows = []
    for t in range(6):
        x = rng.standard_normal(D).astype(np.float32)
        if t % 2 == 0:
            x *= np.float32(2.0) ** rng.integers(-60, 60, size=D).astype(np.float32)
        rows.append(x)
    bits = _bf16_bits(np.stack(rows))
    got = codecs.hadamard_rotate_bf16(bits)
    for r in range(bits.shape[0]):
        want = [_nearest_bf16_brute(y) for y in _exact_rotation(bits[r])]
        assert got[r].tolist() == want, r


def test_hadamard_named_ties_subnormals_and_overflow():
    """Two nonzero inputs a, b at positions 0 and 1 give outputs a + b (H[j][1] =
    1) and a - b (H[j][1] = -1) in alternate positions."""
    D = 64

    def pair(a, b):
        x = np.zeros(D, np.float32)
        x[0], x[1] = a, b
        bits = _bf16_bits(x)
        assert codecs.bf16_to_f32(bits)[0] == np.float32(a) and codecs.bf16_to_f32(bits)[1] == np.float32(b)
        y = codecs.hadamard_rotate_bf16(bits)
        return int(y[0]), int(y[1])

    one = 0x3F80
    assert pair(1.0, 2.0 ** -8) == (one, 0x3F7F)                 # 1 + 2^-8: tie -> even 1.0; 1 - 2^-8 exact
    assert pair(1.0 + 2.0 ** -7, 2.0 ** -8) == (0x3F82, 0x3F80)  # tie above an odd value rounds up; 1 exact
    t = 2.0 ** -125 * (1 + 2.0 ** -7)                            # normal, last bit 2^-132
    up, dn = pair(t, 2.0 ** -133)                                # +- half its last bit: both ties
    assert up == 0x0102 and dn == 0x0100                        # odd last bit: ties to mantissas 2 and 0
    assert pair(2.0 ** -130, 2.0 ** -133) == (0x0009, 0x0007)    # subnormal sums are exact
    mx = float(codecs.bf16_to_f32(np.uint16(0x7F7F)))
    # the last binade's ulp is 2^120: max + 2^119 is the tie with 2^128, which
    # goes to the even pattern, the overflow; max - 2^119 ties to even 0x7F7E
    assert pair(mx, 2.0 ** 120) == (0x7F80, 0x7F7E)
    assert pair(mx, 2.0 ** 119) == (0x7F80, 0x7F7E)
    assert pair(mx, 2.0 ** 118) == (0x7F7F, 0x7F7F)              # below halfway: stays finite
    assert pair(-mx, -(2.0 ** 119)) == (0xFF80, 0xFF7E)
    assert pair(0.0, 0.0) == (0x0000, 0x0000)
    negz = np.full(D, 0x8000, np.uint16)                         # -0 everywhere: exact zeros are +0
    assert (codecs.hadamard_rotate_bf16(negz) == 0).all()


def test_hadamard_non_finite_rules():
    from scipy.linalg import hadamard
    D = 64
    H = hadamard(D)
    x = np.zeros(D, np.float32)
    x[0] = np.inf
    y = codecs.hadamard_rotate_bf16(_bf16_bits(x))
    assert (y == 0x7F80).all()                                   # column 0 of H is all +1
    x[1] = -np.inf                                               # +Inf and -Inf meet where H[j][1] = +1
    y = codecs.hadamard_rotate_bf16(_bf16_bits(x))
    assert np.array_equal(y, np.where(H[:, 1] > 0, 0x7FC0, 0x7F80).astype(np.uint16))
    x[1] = 1.0
    x[5] = np.nan
    assert (codecs.hadamard_rotate_bf16(_bf16_bits(x)) == 0x7FC0).all()


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


def test_hadamard_matrix_is_scipys():
    from scipy.linalg import hadamard
    for D in (2, 16, 64, 128):
        assert np.array_equal(codecs.hadamard_matrix(D), hadamard(D))


# ---- helpers that decide what the GPU comparison accepts ----

@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_is_nan_code_matches_torch(fmt, tdt):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(tdt).to(torch.float32).isnan().numpy()
    assert np.array_equal(codecs.fp8_is_nan_code(codes, fmt), ref)


def test_f32_to_bf16_rne_matches_torch():
    rng = np.random.default_rng(31)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 10.0 ** rng.uniform(-40, 38, 50000)).astype(np.float32),
        rng.integers(0, 2 ** 32, size=100000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    # exact ties: low half 0x8000 above an even and an odd bf16, both signs
    hi = rng.integers(0, 0x7F7F, size=20000).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([3.4028235e38, -3.4028235e38, 3.3961e38, np.inf, -np.inf,
                                                      0.0, -0.0, 1e-45, -1e-45])])
    fin = ~np.isnan(x)
    got = codecs.f32_to_bf16_rne(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[fin], want[fin])
    assert (got[~fin] == 0x7FC0).all()
    wt = torch.from_numpy(ties).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.f32_to_bf16_rne(ties), wt)
    assert ((wt & 1) == 0).all()                                 # every tie went to an even pattern


def test_int4_nan_elements_are_left_out():
    """A NaN element does not enter the row's min / max and gets code 0; a row of
    only NaNs keeps (NaN, NaN) and zero codes (the fmin / fmax rule of the
    calibration)."""
    x = np.array([[-1.0, np.nan, 2.0, 2.0], [np.nan] * 4, [0.5, np.nan, np.nan, 0.5]], np.float32)
    codes, s, zp = codecs.int4_encode_rows(x)
    c0, s0, z0 = codecs.int4_encode_rows(np.array([[-1.0, 2.0, 2.0]], np.float32))
    assert s[0] == s0[0] and zp[0] == z0[0]
    assert codes[0].tolist() == [c0[0][0], 0, c0[0][1], c0[0][2]]
    assert np.isnan(s[1]) and np.isnan(zp[1]) and (codes[1] == 0).all()
    # constant row guard: s = |min| = 0.5, zp = -1, both 0.5 entries at code 0 and exact
    assert s[2] == np.float32(0.5) and zp[2] == -1.0 and codes[2].tolist() == [0, 0, 0, 0]
    assert codecs.int4_decode(codes[2:3], s[2:3], zp[2:3])[0, 0] == np.float32(0.5)
