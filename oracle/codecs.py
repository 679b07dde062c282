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
  hadamard_rotate_bf16 - scipy's Sylvester Hadamard matrix (library routine) in
                      float64 on rows whose products are exact there, with torch's
                      float32 -> bf16 rounding of results exact in float32; a
                      brute-force nearest-bf16 search (ties to even) on exact
                      rational results, including halfway cases, subnormals and
                      overflow; H H = D I; preserved dot products; IEEE infinity
                      and NaN rules.
  fp8_is_nan_code   - torch's float8_e4m3fn / float8_e5m2 isnan over all codes.
  f32_to_bf16_rne   - torch's float32 -> bfloat16 cast on random values, exact
                      ties, overflow and NaN.
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
                                                 not clamped; +0 when zero, since
                                                 a row holding -0 and +0 has
                                                 either as its minimum)
    NaN elements are left out of min and max (fmin / fmax, as the calibration
    does); a row of only NaNs gets (NaN, NaN).
    Returns (s, zp), float32 arrays over the leading axes.
    """
    x = np.asarray(x, dtype=F32)
    with np.errstate(invalid="ignore"):
        mn = np.fmin.reduce(x, axis=-1)       # NaN elements are left out (a row
        mx = np.fmax.reduce(x, axis=-1)       # of only NaNs gives NaN)
    with np.errstate(over="ignore", invalid="ignore"):
        rng = np.subtract(mx, mn, dtype=F32)
        s = np.divide(rng, F32(15.0), dtype=F32)
    bad = (s == 0) | ~np.isfinite(s)
    guard = np.where(mn != 0, np.abs(mn), F32(1.0)).astype(F32)
    s = np.where(bad, guard, s).astype(F32)
    zp = (np.rint(_div32(-mn, s)) + F32(0.0)).astype(F32)   # a zero zero point is +0
    return s, zp


def int4_encode_rows(x):
    """INT4 codes of float32 rows ``x`` [..., D]: returns (codes uint8 [..., D], s, zp).

    q = clamp(RNE(fl32(x / s)) + zp, 0, 15); the zero point is added after
    rounding, as an integer.  A NaN element (or any element of an all-NaN row)
    gets code 0, as the clamp's lower bound does for an unordered value.
    """
    x = np.asarray(x, dtype=F32)
    s, zp = int4_row_params(x)
    with np.errstate(invalid="ignore"):
        t = _div32(x, s[..., None])
        q = np.clip(np.rint(t) + zp[..., None], 0, 15)
    q = np.where(np.isnan(q), 0, q)
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
# transform of the row's D values, y = H x with H[i][k] = (-1)^popcount(i & k),
# computed exactly and rounded once to bf16 (round to nearest, ties to even).
# H H = D I, so a key stored as H k is recovered as H (H k) / D.
# ---------------------------------------------------------------------------

BF16_MIN_LSB_EXP = -133      # exponent of the smallest bf16 subnormal, 2^-133
BF16_MAX_EXP = 127           # largest binade of a finite bf16 (values < 2^128)


def hadamard_matrix(D):
    """The Sylvester-Hadamard matrix of order D (a power of two), from its closed
    form H[i][k] = (-1)^popcount(i & k), as int64."""
    assert D > 0 and D & (D - 1) == 0
    i = np.arange(D, dtype=np.int64)
    a = i[:, None] & i[None, :]
    pop = np.zeros_like(a)
    while a.any():
        pop += a & 1
        a >>= 1
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def _round_int_to_bf16(Y, e0):
    """bf16 bits of the exact value Y * 2^e0 (Y a Python int), round to nearest,
    ties to even, overflowing to +-Inf; an exact zero gives +0."""
    if Y == 0:
        return 0
    sign = 0x8000 if Y < 0 else 0
    A = -Y if Y < 0 else Y
    msb = A.bit_length() - 1 + e0                   # exponent of the leading bit
    qe = max(msb - 7, BF16_MIN_LSB_EXP)             # exponent of the result's last bit
    sh = qe - e0
    if sh <= 0:
        R = A << (-sh)
    else:
        R = A >> sh
        rem = A - (R << sh)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and (R & 1)):
            R += 1
    # R * 2^qe with R <= 256: renormalise a carry out of the top bit
    if R == 256:
        R, qe = 128, qe + 1
    if R == 0:
        return sign
    if R >= 128:                                    # normal: R = 1.mmmmmmm * 2^7
        e = qe + 7
        if e > BF16_MAX_EXP:
            return sign | 0x7F80
        return sign | ((e + 127) << 7) | (R & 0x7F)
    return sign | R                                 # subnormal: qe == -133


def _fwht_int64(X):
    """H X over the last axis in exact integer arithmetic, by the fast
    Walsh-Hadamard factorisation of H into log2(D) stages, each pairing (i, i + h)
    into (a + b, a - b).  Integer sums are exact in any order, so this is the
    matrix product itself; callers keep |X| small enough for int64."""
    X = np.array(X, np.int64)
    D = X.shape[-1]
    h = 1
    while h < D:
        y = X.reshape(X.shape[:-1] + (D // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        X = y.reshape(X.shape)
        h *= 2
    return X


def _round_int64_to_bf16(Y, e0):
    """_round_int_to_bf16 over an int64 array Y (|Y| < 2^62) with exponents e0
    broadcast against it, in integer arithmetic throughout."""
    Y = np.asarray(Y, np.int64)
    e0 = np.broadcast_to(np.asarray(e0, np.int64), Y.shape)
    sign = np.where(Y < 0, 0x8000, 0).astype(np.int64)
    A = np.abs(Y)
    # bit length of A: frexp of the float64 value, corrected where the
    # conversion rounded A up to the next power of two
    _, n = np.frexp(A.astype(np.float64))
    n = n.astype(np.int64)
    n = np.where((n > 0) & ((A >> np.maximum(n - 1, 0)) == 0), n - 1, n)
    msb = n - 1 + e0
    qe = np.maximum(msb - 7, BF16_MIN_LSB_EXP)
    sh = qe - e0
    up_sh = np.clip(-sh, 0, 62)
    dn_sh = np.clip(sh, 0, 62)
    Rdn = A >> dn_sh
    rem = A - (Rdn << dn_sh)
    half = np.where(dn_sh > 0, np.int64(1) << np.maximum(dn_sh - 1, 0), 0)
    rup = (dn_sh > 0) & ((rem > half) | ((rem == half) & ((Rdn & 1) == 1)))
    R = np.where(sh <= 0, A << up_sh, Rdn + rup)
    carry = R == 256
    R = np.where(carry, 128, R)
    qe = np.where(carry, qe + 1, qe)
    e = qe + 7
    normal = R >= 128
    bits = np.where(normal, ((e + 127) << 7) | (R & 0x7F), R)
    bits = np.where(normal & (e > BF16_MAX_EXP), 0x7F80, bits)
    bits = np.where(A == 0, 0, bits | sign)
    return bits.astype(np.uint16)


def hadamard_rotate_bf16(x_bits):
    """bf16 rows [..., D] (D a power of two) -> bf16 bits of y = H x, as above.

    Every finite bf16 value is an integer multiple of 2^-133, so with e0 the
    smallest exponent of a last significand bit in the row, X_i = x_i / 2^e0
    is an integer and y_j = 2^e0 * sum_i H[j][i] X_i is evaluated exactly in
    integer arithmetic (int64 where the row's magnitudes allow it, Python
    integers otherwise), then rounded once.  Non-finite rows: a NaN anywhere
    makes every output NaN (0x7FC0); otherwise an output whose signed terms
    hold both +Inf and -Inf is NaN, one holding only one sign of infinity is
    that infinity.
    """
    bits = np.asarray(x_bits, np.uint16)
    D = bits.shape[-1]
    assert D & (D - 1) == 0
    lead = bits.shape[:-1]
    b = bits.reshape(-1, D).astype(np.int64)
    H = hadamard_matrix(D)
    E8 = (b >> 7) & 0xFF
    man = b & 0x7F
    fin = E8 != 0xFF
    sig = np.where(E8 != 0, man | 0x80, man)                 # integer significand
    sig = np.where(fin, sig, 0)
    sig = np.where((b >> 15) == 1, -sig, sig)
    lsb = np.maximum(E8, 1) - 127 - 7                        # exponent of the last bit
    nz = sig != 0
    e0 = np.where(nz, lsb, 10 ** 6).min(axis=1)
    e0 = np.where(nz.any(axis=1), e0, 0)
    spread = np.where(nz, lsb - e0[:, None], 0).max(axis=1)
    out = np.zeros(b.shape, np.uint16)
    # int64 fast path: |X_i| < 2^(spread + 8), sums of D terms below 2^62
    fast = spread + 8 + int(np.log2(D)) <= 62
    rows = np.nonzero(fast)[0]
    if rows.size:
        X = sig[rows] << (lsb[rows] - e0[rows, None]) * nz[rows]
        Y = _fwht_int64(X)                                   # exact int64 sums
        out[rows] = _round_int64_to_bf16(Y, e0[rows, None])
    for r in np.nonzero(~fast)[0]:
        X = [int(s) << int(l - e0[r]) if s else 0 for s, l in zip(sig[r], lsb[r])]
        out[r] = [_round_int_to_bf16(sum(int(H[j, i]) * X[i] for i in range(D)), int(e0[r])) for j in range(D)]
    # non-finite inputs
    for r in np.nonzero((~fin).any(axis=1))[0]:
        if (~fin[r] & (man[r] != 0)).any():
            out[r] = 0x7FC0
            continue
        pos_inf = (~fin[r] & ((b[r] >> 15) == 0)).astype(np.int64)
        neg_inf = (~fin[r] & ((b[r] >> 15) == 1)).astype(np.int64)
        has_pos = ((H > 0) @ pos_inf + (H < 0) @ neg_inf) > 0      # y_j's terms that are +Inf
        has_neg = ((H < 0) @ pos_inf + (H > 0) @ neg_inf) > 0      # ... and -Inf
        out[r] = np.where(has_pos & has_neg, 0x7FC0,
                          np.where(has_pos, 0x7F80, np.where(has_neg, 0xFF80, out[r])))
    return out.reshape(lead + (D,))


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
