"""Pins of the oracle's calibration, paged write, conversion and gather."""

import numpy as np
import pytest

from oracle import cache as oc
from oracle import codecs
from workloads import WORKLOADS, make_decode_inputs, f32_to_bf16_bits, scatter_rows_to_pages


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


# ---------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------


def test_calibrate_hand_example():
    x = np.zeros((3, 2, 4), np.float32)
    x[0, 0, 1] = -12.7
    x[2, 1, 3] = 4.48
    x[1, 1, 0] = -3.0
    a, s = oc.calibrate(_bits(x), "per_tensor", 127.0)
    a12 = float(codecs.bf16_to_f32(_bits(np.float32(-12.7))))
    assert a[0] == np.float32(abs(a12))
    assert s[0] == np.float32(abs(a12)) / np.float32(127.0)
    a, s = oc.calibrate(_bits(x), "per_kv_head", 448.0)
    assert a[0] == np.float32(abs(a12))
    assert a[1] == codecs.bf16_to_f32(_bits(np.float32(4.48)))
    # absmax equal to qmax gives scale exactly 1
    y = np.zeros((1, 1, 2), np.float32)
    y[0, 0, 0] = 448.0
    assert oc.calibrate(_bits(y), "per_tensor", 448.0)[1][0] == 1.0
    y[0, 0, 0] = 127.0
    assert oc.calibrate(_bits(y), "per_tensor", 127.0)[1][0] == 1.0


def test_calibrate_zero_and_nan():
    z = np.zeros((4, 2, 8), np.float32)
    a, s = oc.calibrate(_bits(z), "per_kv_head", 127.0)
    assert (a == 0).all() and (s == 1.0).all()
    b = _bits(z)
    b[1, 0, 3] = 0x7FC0     # NaN is ignored
    b[2, 0, 4] = _bits(np.float32(-2.0))
    a, s = oc.calibrate(b, "per_kv_head", 127.0)
    assert a[0] == 2.0 and a[1] == 0.0 and s[1] == 1.0


def test_calibrate_order_free_and_running():
    rng = np.random.default_rng(0)
    x = _bits(rng.standard_normal((257, 8, 64)).astype(np.float32) * 3)
    a1, s1 = oc.calibrate(x, "per_kv_head", 127.0)
    a2, s2 = oc.calibrate(x[rng.permutation(257)], "per_kv_head", 127.0)
    assert np.array_equal(a1, a2) and np.array_equal(s1, s2)
    run = None
    for c in np.array_split(np.arange(257), 5):
        run, sr = oc.calibrate(x[c], "per_kv_head", 127.0, run)
    assert np.array_equal(run, a1) and np.array_equal(sr, s1)
    at, _ = oc.calibrate(x, "per_tensor", 127.0)
    assert at[0] == a1.max()


# ---------------------------------------------------------------------------
# write by slot mapping
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("kd,vd", [("int8", "int8"), ("e4m3", "e5m2"), ("e4m3", "int8"), ("int4", "int4"), ("bf16", "bf16")])
def test_write_places_rows_at_slots(kd, vd):
    rng = np.random.default_rng(1)
    nb, H, D, bs = 5, 3, 16, 16
    T = 23
    k = _bits(rng.standard_normal((T, H, D)).astype(np.float32))
    v = _bits(rng.standard_normal((T, H, D)).astype(np.float32))
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[4] = -1                 # skipped
    slots[9] = nb * bs + 7        # beyond the pool: skipped and counted
    ks = np.array([0.02, 0.03, 0.05], np.float32)
    c = oc.PagedCache(nb, H, D, kd, vd, k_scale=ks, v_scale=np.float32(0.04), block_size=bs)
    bad = c.write(k, v, slots)
    assert bad == 1
    # expected: loop over tokens and heads, one codec call per row
    for i in range(T):
        s = int(slots[i])
        if s < 0 or s >= nb * bs:
            continue
        blk, off = divmod(s, bs)
        for h in range(H):
            for which, rows, dt, sc in (("k", k, kd, ks[h]), ("v", v, vd, np.float32(0.04))):
                x = codecs.bf16_to_f32(rows[i, h])
                page = getattr(c, which + "_pages")[blk, h, off]
                if dt == "int8":
                    assert np.array_equal(page.view(np.int8), codecs.int8_encode(x, sc))
                elif dt in ("e4m3", "e5m2"):
                    assert np.array_equal(page, codecs.fp8_encode(x, sc, dt))
                elif dt == "bf16":
                    assert np.array_equal(page.view(np.uint16), rows[i, h])
                else:
                    q, s4, z4 = codecs.int4_encode_rows(x[None])
                    assert np.array_equal(page, codecs.int4_pack(q)[0])
                    assert np.array_equal(getattr(c, which + "_meta")[blk, h, off], [s4[0], z4[0]])
    # untouched slots keep the fill
    used = set(int(s) for s in slots if 0 <= s < nb * bs)
    for s in range(nb * bs):
        if s not in used:
            assert (c.k_pages[s // bs, :, s % bs] == 0xFF).all()


def test_convert_equals_write_of_every_slot():
    rng = np.random.default_rng(2)
    nb, H, D, bs = 6, 2, 32, 16
    src_k = _bits(rng.standard_normal((nb, H, bs, D)).astype(np.float32))
    src_v = _bits(rng.standard_normal((nb, H, bs, D)).astype(np.float32))
    a = oc.PagedCache(nb, H, D, "int4", "int4", block_size=bs)
    a.convert_from_bf16(src_k, src_v, 1, 4)
    b = oc.PagedCache(nb, H, D, "int4", "int4", block_size=bs)
    slots = np.arange(1 * bs, 5 * bs, dtype=np.int64)
    rows_k = src_k.transpose(0, 2, 1, 3).reshape(nb * bs, H, D)[slots]
    rows_v = src_v.transpose(0, 2, 1, 3).reshape(nb * bs, H, D)[slots]
    b.write(rows_k, rows_v, slots)
    assert np.array_equal(a.k_pages, b.k_pages) and np.array_equal(a.v_pages, b.v_pages)
    assert np.array_equal(a.k_meta, b.k_meta, equal_nan=True)
    assert np.array_equal(a.v_meta, b.v_meta, equal_nan=True)


def test_gather_of_permuted_pool_equals_contiguous():
    w = WORKLOADS["tiny_int8"]
    inp = make_decode_inputs(w)
    c = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, "bf16", "bf16")
    c.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    for b in range(w.B):
        L = int(inp.seq_lens[b])
        got = c.gather(inp.block_tables[b], L, "k")
        ref = codecs.bf16_to_f32(inp.k_bits[inp.cu[b]:inp.cu[b + 1]])
        assert np.array_equal(got, ref)


def test_scatter_rows_to_pages_roundtrip():
    w = WORKLOADS["tiny_int8"]
    inp = make_decode_inputs(w)
    pages = scatter_rows_to_pages(inp.k_bits, inp.slot_mapping, inp.num_blocks)
    c = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, "bf16", "bf16")
    c.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    assert np.array_equal(c.k_pages.view(np.uint16), pages)
