"""Planted mistakes in the oracle: each pin set must catch them.

Every case below rewrites one line of an oracle function into a plausible
mistake (a wrong rounding or tie rule, a dropped term, a flipped sign, an
off-by-one index, a swapped operand), installs the rewritten function in place
of the original for the duration of the test, and runs the pins that guard that
part of the oracle.  At least one pin must fail; a mistake that every pin lets
through would mean the oracle is not pinned where it matters.  The oracle's own
source is never modified: the rewrite is compiled from its text in memory.
"""

import functools
import inspect
import textwrap

import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import codecs
from tests import test_oracle_attention as ta
from tests import test_oracle_cache as tca
from tests import test_oracle_codecs as tc

P = functools.partial
EXHAUSTIVE = [P(tc.test_fp8_encode_exhaustive_bf16, f, s) for f in ("e4m3", "e5m2") for s in (1.0, 0.0123, 3.75e-3, 17.5)]
SDPA = [P(ta.test_matches_torch_sdpa_fp64, kd, vd) for kd, vd in (("int8", "int8"), ("e5m2", "e4m3"), ("int4", "int4"))]
CAUSAL = [P(ta.test_verify_matches_torch_sdpa_causal_fp64, "int8", "int8"), ta.test_verify_rows_are_truncated_decodes]

# (name, owner, function, line as written, the planted mistake, pins)
MUTANTS = [
    ("int8 ties round up", codecs, "int8_encode", "q = np.rint(t)", "q = np.floor(t + 0.5)",
     [tc.test_int8_named_cases]),
    ("int8 code -128 allowed", codecs, "int8_encode", "q = np.clip(q, -INT8_QMAX, INT8_QMAX)",
     "q = np.clip(q, -INT8_QMAX - 1, INT8_QMAX)", [tc.test_int8_named_cases]),
    ("int8 quotient by reciprocal", codecs, "int8_encode", "t = _div32(x, s)",
     "t = np.multiply(np.asarray(x, F32), np.divide(F32(1.0), np.asarray(s, F32), dtype=F32), dtype=F32)",
     [tc.test_int8_exact_ties_follow_the_quotient]),
    ("fp8 ties away from zero", codecs, "fp8_encode_value", "n = np.rint(a / quantum)",
     "n = np.floor(a / quantum + 0.5)", [tc.test_fp8_encode_named_ties] + EXHAUSTIVE[:1]),
    ("fp8 no saturation", codecs, "fp8_encode_value", "mag = np.where(a >= maxval, maxcode, mag)", "mag = mag",
     [tc.test_fp8_encode_named_ties] + EXHAUSTIVE),
    ("fp8 subnormal mantissa scale", codecs, "fp8_encode_value", "val / 2.0 ** (1 - bias - mb),",
     "val / 2.0 ** (0 - bias - mb),", EXHAUSTIVE),
    ("fp8 quotient by reciprocal", codecs, "fp8_encode", "return fp8_encode_value(_div32(x, s), fmt)",
     "return fp8_encode_value(np.multiply(np.asarray(x, F32), np.divide(F32(1.0), np.asarray(s, F32), dtype=F32),"
     " dtype=F32), fmt)", [P(tc.test_fp8_exact_ties_follow_the_quotient, f) for f in ("e4m3", "e5m2")] + EXHAUSTIVE),
    ("fp8 normal exponent off by one", codecs, "fp8_decode_code",
     "return sign * (1.0 + M / (1 << mb)) * 2.0 ** (E - bias)",
     "return sign * (1.0 + M / (1 << mb)) * 2.0 ** (E - bias - 1)",
     [P(tc.test_fp8_named_codes, "e4m3", tc.E4M3_POINTS), P(tc.test_fp8_named_codes, "e5m2", tc.E5M2_POINTS)]),
    ("fp8 subnormal exponent off by one", codecs, "fp8_decode_code",
     "return sign * (M / (1 << mb)) * 2.0 ** (1 - bias)", "return sign * (M / (1 << mb)) * 2.0 ** (0 - bias)",
     [P(tc.test_fp8_named_codes, "e4m3", tc.E4M3_POINTS), P(tc.test_fp8_named_codes, "e5m2", tc.E5M2_POINTS)]),
    ("e4m3 top binade all NaN", codecs, "fp8_decode_code", "if E == emax_field and M == (1 << mb) - 1:",
     "if E == emax_field:", [tc.test_fp8_special_code_sets]),
    ("e5m2 infinity counted as NaN", codecs, "fp8_is_nan_code", "return c > 0x7C", "return c >= 0x7C",
     [P(tc.test_fp8_is_nan_code_matches_torch, "e5m2", torch.float8_e5m2)]),
    ("int4 scale over 16 steps", codecs, "int4_row_params", "s = np.divide(rng, F32(15.0), dtype=F32)",
     "s = np.divide(rng, F32(16.0), dtype=F32)", [tc.test_int4_hand_example, tc.test_int4_invariants]),
    ("int4 zero point sign", codecs, "int4_row_params", "zp = (np.rint(_div32(-mn, s)) + F32(0.0)).astype(F32)",
     "zp = (np.rint(_div32(mn, s)) + F32(0.0)).astype(F32)", [tc.test_int4_hand_example, tc.test_int4_invariants]),
    ("int4 NaN taken into the minimum", codecs, "int4_row_params", "mn = np.fmin.reduce(x, axis=-1)",
     "mn = np.min(x, axis=-1)", [tc.test_int4_nan_elements_are_left_out]),
    ("int4 constant-row guard", codecs, "int4_row_params",
     "guard = np.where(mn != 0, np.abs(mn), F32(1.0)).astype(F32)", "guard = np.ones_like(mn)",
     [tc.test_int4_constant_rows_exact]),
    ("int4 zero point added before rounding", codecs, "int4_encode_rows",
     "q = np.clip(np.rint(t) + zp[..., None], 0, 15)", "q = np.clip(np.rint(t + zp[..., None]), 0, 15)",
     [tc.test_int4_hand_example]),
    ("int4 nibble order", codecs, "int4_pack", "(c[..., 0::2] | (c[..., 1::2] << 4))",
     "(c[..., 1::2] | (c[..., 0::2] << 4))", [tc.test_int4_pack_order]),
    ("int4 metadata bytes", codecs, "elem_bytes_per_row", "INT4_META_BYTES", "INT4_META_BYTES // 2",
     [tc.test_bytes_ratios]),
    ("fp8 dequantisation divides", codecs, "fp8_decode", "return np.multiply(v, np.asarray(s, dtype=F32), dtype=F32)",
     "return np.divide(v, np.asarray(s, dtype=F32), dtype=F32)",
     [P(tc.test_fp8_round_trip_bound, f) for f in ("e4m3", "e5m2")]),
    ("int8 dequantisation divides", codecs, "int8_decode",
     "return np.multiply(np.asarray(q, dtype=np.int8).astype(F32), np.asarray(s, dtype=F32), dtype=F32)",
     "return np.divide(np.asarray(q, dtype=np.int8).astype(F32), np.asarray(s, dtype=F32), dtype=F32)",
     [tc.test_int8_round_trip_bound]),
    ("int4 dequantisation adds the zero point", codecs, "int4_decode",
     "d = np.subtract(q, np.asarray(zp, dtype=F32)[..., None], dtype=F32)",
     "d = np.add(q, np.asarray(zp, dtype=F32)[..., None], dtype=F32)", [tc.test_int4_invariants]),
    ("capacity rounds blocks up", codecs, "blocks_in_budget", "return budget_bytes // per_block",
     "return -(-budget_bytes // per_block)", [tc.test_blocks_in_budget_counts_whole_blocks]),
    ("capacity without the layer count", codecs, "blocks_in_budget", "* num_kv_heads * num_layers *",
     "* num_kv_heads *", [tc.test_block_ratio_matches_l4_table, tc.test_blocks_in_budget_counts_whole_blocks]),
    ("bf16 narrowing truncates", codecs, "f32_to_bf16_rne", "r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)",
     "r = (u >> 16).astype(np.uint16)", [tc.test_f32_to_bf16_rne_matches_torch]),
    ("hadamard sign from i | k", codecs, "hadamard_matrix", "a = i[:, None] & i[None, :]",
     "a = i[:, None] | i[None, :]", [tc.test_hadamard_matrix_is_scipys]),
    ("hadamard butterfly difference flipped", codecs, "_fwht_int64", "y[..., 1, :] = a - b", "y[..., 1, :] = b - a",
     [P(tc.test_hadamard_matches_library_matrix_and_torch_rounding, 64),
      tc.test_hadamard_twice_is_D_times_identity_and_columns]),
    ("hadamard rounding ties away", codecs, "_round_int64_to_bf16",
     "rup = (dn_sh > 0) & ((rem > half) | ((rem == half) & ((Rdn & 1) == 1)))", "rup = (dn_sh > 0) & (rem >= half)",
     [tc.test_hadamard_named_ties_subnormals_and_overflow,
      P(tc.test_hadamard_matches_library_matrix_and_torch_rounding, 64)]),
    ("calibration of the signed maximum", oc, "calibrate", "x = np.abs(codecs.bf16_to_f32(x_bits))",
     "x = codecs.bf16_to_f32(x_bits)", [tca.test_calibrate_hand_example]),
    ("calibration of a zero group", oc, "calibrate", "s = np.where(a == 0, F32(1.0), s).astype(F32)",
     "s = s.astype(F32)", [tca.test_calibrate_zero_and_nan]),
    ("calibration groups by token", oc, "calibrate", "groups = x.transpose(1, 0, 2).reshape(H, -1)",
     "groups = x.reshape(H, -1)", [tca.test_calibrate_hand_example, tca.test_calibrate_order_free_and_running]),
    ("per-head scales collapsed to head 0", oc, "_head_scale", "    return s\n", "    return np.full(H, s[0], F32)\n",
     [P(tca.test_write_places_rows_at_slots, "int8", "int8")]),
    ("convert slot order", oc.PagedCache, "convert_from_bf16",
     "r = rows.transpose(0, 2, 1, 3).reshape(-1, self.H, self.D)", "r = rows.reshape(-1, self.H, self.D)",
     [tca.test_convert_equals_write_of_every_slot]),
    ("write offset off by one", oc.PagedCache, "write", "blk, off = slots[idx] // self.bs, slots[idx] % self.bs",
     "blk, off = slots[idx] // self.bs, (slots[idx] + 1) % self.bs",
     [P(tca.test_write_places_rows_at_slots, "int8", "int8")]),
    ("gather offset off by one", oc.PagedCache, "gather", "off = p % self.bs", "off = (p + 1) % self.bs",
     [tca.test_gather_of_permuted_pool_equals_contiguous, ta.test_single_token_gives_its_value] + SDPA[:1]),
    ("softmax scale dropped", oa, "_attend", "z = softmax_scale * (K @ qv)", "z = K @ qv", SDPA[:1]),
    ("keys in place of values", oa, "_attend", "return (e @ V) / e.sum()", "return (e @ K) / e.sum()", SDPA[:1]),
    ("grouped heads mapped by remainder", oa, "decode", "c = col[h // g]", "c = col[h % cache.H]",
     SDPA[:1] + [ta.test_gqa_equals_repeated_kv_heads]),
    ("one position past the end", oa, "decode", "L = int(seq_lens[b])",
     "L = min(int(seq_lens[b]) + 1, 16 * len(block_tables[b])) if int(seq_lens[b]) > 0 else 0",
     [ta.test_unused_slots_and_empty_sequences] + SDPA[:1]),
    ("empty sequence row not zero", oa, "decode", "out[b, h] = 0.0", "out[b, h] = 1.0",
     [ta.test_unused_slots_and_empty_sequences]),
    ("causal limit one past", oa, "verify", "K[:pos + 1, c, :], V[:pos + 1, c, :]",
     "K[:pos + 2, c, :], V[:pos + 2, c, :]", CAUSAL),
    ("causal tokens counted from the start", oa, "verify", "t, pos = b * n_q + i, L - n_q + i",
     "t, pos = b * n_q + i, min(i, L - 1)", CAUSAL),
    ("merge without the weight on l", oa, "combine", "den = (w * l).sum(axis=-1)", "den = l.sum(axis=-1)",
     [ta.test_split_equals_unsplit]),
    ("partition sums against the global maximum", oa, "decode_partials", "e = np.exp(z[sl] - mj)",
     "e = np.exp(z[sl] - z.max())", [ta.test_split_equals_unsplit]),
    ("rotated keys not scaled back by D", oa, "_keys", "K = (K @ H.T) / cache.D", "K = K @ H.T",
     [ta.test_rotated_keys_equal_derotated_attention]),
]


def _plant(monkeypatch, owner, name, line, mistake):
    fn = inspect.getattr_static(owner, name)
    src = textwrap.dedent(inspect.getsource(fn))
    assert line in src, f"{name} no longer holds the line {line!r}"
    mod = inspect.getmodule(fn)
    ns = dict(vars(mod))
    exec(compile(src.replace(line, mistake), f"<planted mistake in {name}>", "exec"), ns)
    monkeypatch.setattr(owner, name, ns[name])


@pytest.mark.parametrize("case", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, case):
    _, owner, name, line, mistake, pins = case
    _plant(monkeypatch, owner, name, line, mistake)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:   # a pin's check failed: the mistake is caught
            caught += 1
    assert caught, "no pin caught the planted mistake"


def test_pins_pass_on_the_oracle_as_written():
    """The same pins, without a planted mistake, pass (so a caught mistake is the
    mistake's doing)."""
    seen = set()
    for *_, pins in MUTANTS:
        for pin in pins:
            key = (getattr(pin, "func", pin), repr(getattr(pin, "args", ())))
            if key in seen:
                continue
            seen.add(key)
            pin()
