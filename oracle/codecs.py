"""Oracle codecs — TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Element formats of the KV cache and their encode / decode rules, written from
the definitions, in NumPy.  Floating-point steps that decide an integer code
(x / s, the rounding) are done in float32 exactly as the GPU kernels do them
(IEEE correctly-rounded division, round-to-nearest-even), so codes can be
compared bit for bit.

Pins (tests/test_oracle_codecs.py):
  fp8_decode_table  - closed-form values of the OCP 8-bit formats at named codes,
                      and torch's float8_e4m3fn / float8_e5m2 views of all 256
                      codes (library routine).
  fp8_encode        - brute-force nearest search over the 256 decoded values with
                      the even-code tie rule, exhaustively over all 65536 bf16
                      inputs; torch's cast inside its non-saturating range.
  int8_encode       - hand-derived special cases (ties, saturation, NaN) and the
                      round-trip bound |x - x_hat| <= s/2 inside the range.
  int4_encode_rows  - q(min) == 0, max code <= 15, round-trip <= s/2, exact
                      constant rows, hand-packed nibble order.
  kv_bytes_per_token_head - the 2.00x GPU-block ratios printed in the L4 table
                      of vLLM PR 4893 (FP16 vs FP8 KV at equal memory).
  hadamard_rotate_bf16 - scipy's Sylvester Hadamard matrix in float64 (exact on
                      integer rows, within the bf16 rounding otherwise), H H = D I,
                      the closed-form columns (-1)^popcount(i & k), and preserved
                      dot products.
"""

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------


def bf16_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to float32 exactly.

    bf16 is the upper half of an IEEE binary32, so widening is a 16-bit shift.
    Used for every bf16 input (Q, K, V, bf16 cache pages).
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bits.

    Only used to express a float32 result as bf16 for the bf16-output check.
    NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), r)


# ---------------------------------------------------------------------------
# INT8 symmetric
# ---------------------------------------------------------------------------

INT8_QMAX = 127


def _div32(x, s):
    """fl32(x / s): IEEE float32 division, correctly rounded (NumPy float32 ufunc)."""
    return np.divide(np.asarray(x, dtype=F32), np.asarray(s, dtype=F32), dtype=F32)


def int8_encode(x, s):
    """INT8 symmetric code of float32 values ``x`` for scale ``s``.

    Reading (the tiny INT8 reference workload: per-tensor scale absmax/127,
    codes RNE, clamped to [-127, 127]; the sm86 INT8 project summary gives the
    format only):
        t = fl32(x / s)          (IEEE division, not x * (1/s))
        q = clamp(RNE(t), -127, 127)
        NaN -> 0, +-Inf -> +-127 (saturation).
    ``s`` broadcasts against ``x`` (scalar, or per-KV-head with a trailing axis
    arranged by the caller).
    """
    t = _div32(x, s)
    q = np.rint(t)
    q = np.clip(q, -INT8_QMAX, INT8_QMAX)
    q = np.where(np.isnan(q), 0.0, q)
    return q.astype(np.int8)


def int8_decode(q, s):
    """x_hat = fl32(q * s) for INT8 codes ``q`` (int8) and float32 scale ``s``."""
    return np.multiply(np.asarray(q, dtype=np.int8).astype(F32), np.asarray(s, dtype=F32), dtype=F32)


# ---------------------------------------------------------------------------
# FP8, OCP 8-bit floating point (E4M3 "fn": no infinities; E5M2: IEEE-like)
# ---------------------------------------------------------------------------

# (exponent bits, mantissa bits, bias, largest finite magnitude, its code)
FP8_FORMATS = {
    "e4m3": dict(ebits=4, mbits=3, bias=7, maxval=448.0, maxcode=0x7E),
    "e5m2": dict(ebits=5, mbits=2, bias=15, maxval=57344.0, maxcode=0x7B),
}

FP8_QMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def fp8_decode_code(code, fmt):
    """Value of one 8-bit code, from the OCP 8-bit floating-point definition.

    e4m3: bias 7, 3 mantissa bits; exponent field 15 with mantissa 7 is NaN
          (no infinities); field 0 is subnormal: +-M/8 * 2^-6.
    e5m2: bias 15, 2 mantissa bits; exponent field 31 is +-Inf (M = 0) or NaN;
          field 0 is subnormal: +-M/4 * 2^-14.
    Otherwise +-(1 + M/2^m) * 2^(E - bias).  Returned as a Python float (exact).
    The vLLM PR 4893 description names the two formats (fp8_e4m3, fp8_e5m2).
    """
    f = FP8_FORMATS[fmt]
    eb, mb, bias = f["ebits"], f["mbits"], f["bias"]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    E = (code >> mb) & ((1 << eb) - 1)
    M = code & ((1 << mb) - 1)
    emax_field = (1 << eb) - 1
    if fmt == "e4m3":
        if E == emax_field and M == (1 << mb) - 1:
            return float("nan")
    else:
        if E == emax_field:
            return sign * float("inf") if M == 0 else float("nan")
    if E == 0:
        return sign * (M / (1 << mb)) * 2.0 ** (1 - bias)
    return sign * (1.0 + M / (1 << mb)) * 2.0 ** (E - bias)


def fp8_decode_table(fmt):
    """All 256 code values of ``fmt`` as float64 (NaN / +-Inf where defined)."""
    return np.array([fp8_decode_code(c, fmt) for c in range(256)], dtype=np.float64)


def fp8_encode_value(t, fmt):
    """Nearest fp8 code to float32 values ``t`` with ties to even, saturating.

    Reading (the FP8 workload asks for saturating conversion; rounding is not
    printed anywhere, so round-to-nearest-even is taken as for INT8):
      * NaN -> NaN code 0x7F with the input's sign bit (0xFF if negative);
      * otherwise sign = sign bit of t (so -0 encodes as 0x80);
      * |t| >= largest finite (this includes +-Inf) -> the largest finite code;
      * else the finite nonnegative code nearest to |t|, ties to the code with
        mantissa LSB 0.
    The nearest value is found arithmetically: within the binade of |t| the
    representable values are integer multiples of quantum = 2^(e - mbits) (for
    the subnormal range the quantum is 2^(1 - bias - mbits)); RNE on |t|/quantum
    (exact in float64, a power-of-two scaling) picks the nearest multiple, and
    an even multiple has mantissa LSB 0, including the carry into the next
    binade.  Returns uint8 codes.
    """
    f = FP8_FORMATS[fmt]
    mb, bias, maxval, maxcode = f["mbits"], f["bias"], f["maxval"], f["maxcode"]
    t = np.asarray(t, dtype=F32)
    a = np.abs(t.astype(np.float64))
    neg = np.signbit(t)
    min_normal = 2.0 ** (1 - bias)
    # exponent of a in [min_normal, maxval): a = fr * 2^ex with fr in [0.5, 1)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        _, ex = np.frexp(np.where(a >= min_normal, a, min_normal))
        e = ex.astype(np.int64) - 1
        quantum = np.ldexp(1.0, (e - mb))
        quantum = np.where(a >= min_normal, quantum, 2.0 ** (1 - bias - mb))
        n = np.rint(a / quantum)
        val = n * quantum
    # value -> code magnitude
    with np.errstate(invalid="ignore", divide="ignore"):
        _, vex = np.frexp(np.where(val >= min_normal, val, min_normal))
        ve = vex.astype(np.int64) - 1
        efield = np.where(val >= min_normal, ve + bias, 0)
        mant = np.where(
            val >= min_normal,
            val / np.ldexp(1.0, ve) * (1 << mb) - (1 << mb),
            val / 2.0 ** (1 - bias - mb),
        )
    mag = (efield << mb) + np.rint(np.nan_to_num(mant)).astype(np.int64)
    mag = np.where(a >= maxval, maxcode, mag)
    code = (np.where(neg, 0x80, 0) + mag).astype(np.int64)
    code = np.where(np.isnan(t), np.where(neg, 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def fp8_encode(x, s, fmt):
    """FP8 code of float32 ``x`` for scale ``s``: fp8_encode_value(fl32(x / s))."""
    return fp8_encode_value(_div32(x, s), fmt)


def fp8_decode(code, s, fmt):
    """x_hat = fl32(decode(code) * s).  decode(code) is exact in float32."""
    tab = fp8_decode_table(fmt).astype(F32)
    v = tab[np.asarray(code, dtype=np.uint8)]
    with np.errstate(invalid="ignore", over="ignore"):
        return np.multiply(v, np.asarray(s, dtype=F32), dtype=F32)


def fp8_is_nan_code(code, fmt):
    c = np.asarray(code, dtype=np.uint8) & 0x7F
    if fmt == "e4m3":
        return c == 0x7F
    return c > 0x7C


# ---------------------------------------------------------------------------
# INT4 asymmetric, one (scale, zero point) per (token, KV head) row
# ---------------------------------------------------------------------------


def int4_row_params(x):
    """Scale and zero point of each row of float32 ``x`` (last axis = head_dim).

    Reading of vLLM issue 4025, methods item 1 ("calculate the scale and zero
    point") with the asymmetric INT4 workload's formulas:
        mn = min(x), mx = max(x)                (exact)
        s  = fl32(fl32(mx - mn) / 15)
        if s == 0 or s is not finite:  s = |mn| if mn != 0 else 1.0
        zp = RNE(fl32(-mn / s))                 (an integer held in float32,
                                                 not clamped)
    Returns (s, zp), float32 arrays over the leading axes.
    """
    x = np.asarray(x, dtype=F32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore"):
        rng = np.subtract(mx, mn, dtype=F32)
        s = np.divide(rng, F32(15.0), dtype=F32)
    bad = (s == 0) | ~np.isfinite(s)
    guard = np.where(mn != 0, np.abs(mn), F32(1.0)).astype(F32)
    s = np.where(bad, guard, s).astype(F32)
    zp = np.rint(_div32(-mn, s)).astype(F32)
    return s, zp


def int4_encode_rows(x):
    """INT4 codes of float32 rows ``x`` [..., D]: returns (codes uint8 [..., D], s, zp).

    q = clamp(RNE(fl32(x / s)) + zp, 0, 15); the zero point is added after
    rounding, as an integer.
    """
    x = np.asarray(x, dtype=F32)
    s, zp = int4_row_params(x)
    t = _div32(x, s[..., None])
    q = np.clip(np.rint(t) + zp[..., None], 0, 15)
    return q.astype(np.uint8), s, zp


def int4_pack(codes):
    """Pack codes [..., D] (D even) two per byte: byte j = q[2j] | q[2j+1] << 4."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def int4_unpack(packed):
    """Inverse of int4_pack: bytes [..., D/2] -> codes [..., D]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def int4_decode(codes, s, zp):
    """x_hat = fl32((q - zp) * s); (q - zp) is exact in float32 for |zp| < 2^24."""
    q = np.asarray(codes, dtype=np.uint8).astype(F32)
    d = np.subtract(q, np.asarray(zp, dtype=F32)[..., None], dtype=F32)
    with np.errstate(invalid="ignore", over="ignore"):
        return np.multiply(d, np.asarray(s, dtype=F32)[..., None], dtype=F32)


# ---------------------------------------------------------------------------
# byte accounting
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# Hadamard rotation of a row (the rotation step of KVarN: techfi24's KVarN
# article, "Contexte Technique").  Reading: the unnormalised Sylvester-Hadamard
# transform of the row's D values, H x with H[i][k] = (-1)^popcount(i & k), taken
# in float32 by the fast Walsh-Hadamard butterfly (stages h = 1, 2, 4, ..., D/2;
# the pair at indices (i, i + h), i & h == 0, becomes (a + b, a - b)) and rounded
# to bf16.  H H = D I, so (H q) . (H k) = D (q . k): the logit scale takes 1 / D.
# ---------------------------------------------------------------------------


def hadamard_rotate_bf16(x_bits):
    """bf16 rows [..., D] (D a power of two) -> bf16 bits of H x, as above."""
    x = bf16_to_f32(np.asarray(x_bits, np.uint16)).astype(F32).copy()
    D = x.shape[-1]
    assert D & (D - 1) == 0
    lead = x.shape[:-1]
    h = 1
    while h < D:
        y = x.reshape(lead + (D // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b          # float32 arithmetic, round to nearest even
        y[..., 1, :] = a - b
        x = y.reshape(lead + (D,))
        h *= 2
    return f32_to_bf16_rne(x)


INT4_META_BYTES = 8  # float32 scale + float32 zero point per (token, KV head)


def elem_bytes_per_row(dtype, D):
    """Bytes one (token, KV head) row of K (or of V) takes in the cache."""
    if dtype == "bf16":
        return 2 * D
    if dtype in ("int8", "e4m3", "e5m2"):
        return D
    if dtype in ("int4", "int4h"):
        return D // 2 + INT4_META_BYTES
    raise ValueError(dtype)


def kv_bytes_per_token_head(k_dtype, v_dtype, D):
    """Bytes of K plus V per token per KV head (scales of per-tensor / per-head
    granularity are O(heads) and excluded)."""
    return elem_bytes_per_row(k_dtype, D) + elem_bytes_per_row(v_dtype, D)


def blocks_in_budget(budget_bytes, k_dtype, v_dtype, D, num_kv_heads, num_layers, block_size=16):
    """Whole cache blocks (block_size tokens, all layers and KV heads) that fit in
    ``budget_bytes`` — the "GPU blocks" count of the L4 table in vLLM PR 4893."""
    per_block = kv_bytes_per_token_head(k_dtype, v_dtype, D) * num_kv_heads * num_layers * block_size
    return budget_bytes // per_block
