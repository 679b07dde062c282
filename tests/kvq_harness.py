"""Shared drivers for the GPU parity tests: run one workload through the HIP
library (via the C ABI binding) and through the oracle, from the same seeded
inputs, and compare."""

import math

import numpy as np
import torch

import quantized_paged_kv_absmax_amd as kvq
from oracle import attention as oa
from oracle import cache as oc
from workloads import make_calibration_set, scatter_rows_to_pages

QMAX = {"int8": 127.0, "e4m3": 448.0, "e5m2": 57344.0}


def dev_bf16(bits, device="cuda"):
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def softmax_scale(D):
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


def _scale_plan(w):
    """(K target dtype or None, V target dtype or None) for absmax calibration."""
    kt = w.k_dtype if (w.k_scale_mode == "absmax" and w.k_dtype in QMAX) else None
    vt = w.v_dtype if (w.v_scale_mode == "absmax" and w.v_dtype in QMAX) else None
    return kt, vt


def _writes(w, inp):
    """Order of cache writes: the set-up tokens, then one call per decode-step token."""
    mask = inp.prompt_mask()
    steps = [np.nonzero(mask)[0]]
    if w.new_tokens:
        L = inp.seq_lens.astype(np.int64)
        for i in range(w.new_tokens):
            pos = L - w.new_tokens + i
            steps.append(inp.cu[:-1] + pos)
    return [s for s in steps if s.size]


# ---------------------------------------------------------------------------
# library side
# ---------------------------------------------------------------------------


class LibRun:
    pass


def build_library_cache(w, inp, device="cuda", calib=None):
    r = LibRun()
    c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran,
                         device=device)
    kt, vt = _scale_plan(w)
    ck, cv = make_calibration_set(w, inp) if calib is None else calib
    if kt:
        kvq.kvq_calibrate_scales(dev_bf16(ck, device), w.k_gran, kt, c.k_absmax, c.k_scale)
    if vt:
        kvq.kvq_calibrate_scales(dev_bf16(cv, device), w.v_gran, vt, c.v_absmax, c.v_scale)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    if w.from_bf16_cache:
        kp = dev_bf16(scatter_rows_to_pages(inp.k_bits, inp.slot_mapping, inp.num_blocks), device)
        vp = dev_bf16(scatter_rows_to_pages(inp.v_bits, inp.slot_mapping, inp.num_blocks), device)
        kvq.kvq_convert_cache(c, kp, vp, 0, inp.num_blocks)
        del kp, vp
    else:
        kd, vd = dev_bf16(inp.k_bits, device), dev_bf16(inp.v_bits, device)
        sl = torch.from_numpy(inp.slot_mapping).to(device)
        for idx in _writes(w, inp):
            it = torch.from_numpy(idx).to(device)
            kvq.kvq_cache_write(c, kd[it].contiguous(), vd[it].contiguous(), sl[it].contiguous(), err_count=err)
        del kd, vd
    torch.cuda.synchronize()
    r.cache, r.err = c, err
    r.q = dev_bf16(inp.q_bits, device)
    r.bt = torch.from_numpy(inp.block_tables).to(device)
    r.sl = torch.from_numpy(inp.seq_lens).to(device)
    return r


def library_decode(r, inp, partition=0, out_dtype="f32", err=None):
    """The workload's attention call: decode, or verify with its n_q query tokens."""
    w = inp.w
    if w.n_q > 1:
        return kvq.kvq_paged_attention_verify(r.cache, r.q, w.n_q, r.bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                              partition=partition, out_dtype=out_dtype, err_count=err)
    return kvq.kvq_paged_attention_decode(r.cache, r.q, r.bt, r.sl, inp.max_seq_len, softmax_scale(w.D),
                                          partition=partition, out_dtype=out_dtype, err_count=err)


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------


def build_oracle_cache(w, inp):
    kt, vt = _scale_plan(w)
    ck, cv = make_calibration_set(w, inp)
    ks = vs = None
    kabs = vabs = None
    if kt:
        kabs, ks = oc.calibrate(ck, w.k_gran, QMAX[kt])
    if vt:
        vabs, vs = oc.calibrate(cv, w.v_gran, QMAX[vt])
    if w.k_scale_mode == "one" and w.k_dtype in QMAX:
        ks = np.ones(1, np.float32)
    if w.v_scale_mode == "one" and w.v_dtype in QMAX:
        vs = np.ones(1, np.float32)
    c = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_scale=ks, v_scale=vs)
    if w.from_bf16_cache:
        c.convert_from_bf16(scatter_rows_to_pages(inp.k_bits, inp.slot_mapping, inp.num_blocks),
                            scatter_rows_to_pages(inp.v_bits, inp.slot_mapping, inp.num_blocks), 0, inp.num_blocks)
    else:
        c.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    c.kabs, c.vabs = kabs, vabs
    return c


def seq_token_rows(inp, seqs):
    """Token-major row indices of the given sequences."""
    return np.concatenate([np.arange(inp.cu[b], inp.cu[b + 1]) for b in seqs]) if len(seqs) else np.zeros(0, np.int64)


def build_oracle_cache_sampled(w, inp, seqs, calib=None):
    """The oracle cache at full pool size holding only the tokens of ``seqs``.

    Scales are calibrated on the workload's whole calibration set, as the
    library does; only the sampled sequences' rows are encoded (a bf16 source
    cache is converted block by block over those sequences' blocks).
    """
    kt, vt = _scale_plan(w)
    ck, cv = make_calibration_set(w, inp) if calib is None else calib
    ks = vs = None
    kabs = vabs = None
    if kt:
        kabs, ks = oc.calibrate(ck, w.k_gran, QMAX[kt])
    if vt:
        vabs, vs = oc.calibrate(cv, w.v_gran, QMAX[vt])
    del ck, cv
    if w.k_scale_mode == "one" and w.k_dtype in QMAX:
        ks = np.ones(1, np.float32)
    if w.v_scale_mode == "one" and w.v_dtype in QMAX:
        vs = np.ones(1, np.float32)
    c = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_scale=ks, v_scale=vs)
    rows = seq_token_rows(inp, seqs)
    if w.from_bf16_cache:
        kp = scatter_rows_to_pages(inp.k_bits[rows], inp.slot_mapping[rows], inp.num_blocks)
        vp = scatter_rows_to_pages(inp.v_bits[rows], inp.slot_mapping[rows], inp.num_blocks)
        for blk in np.unique(inp.slot_mapping[rows] // 16):
            c.convert_from_bf16(kp, vp, int(blk), 1)
    else:
        c.write(inp.k_bits[rows], inp.v_bits[rows], inp.slot_mapping[rows])
    c.kabs, c.vabs = kabs, vabs
    return c


# ---------------------------------------------------------------------------
# comparisons
# ---------------------------------------------------------------------------


def valid_slot_mask(inp):
    m = np.zeros((inp.num_blocks, 16), bool)
    s = inp.slot_mapping
    m[s // 16, s % 16] = True
    return m


def assert_codes_equal(r, oracle_cache, inp, seqs=None):
    """Bit-exact comparison of every written slot (codes and INT4 metadata), or,
    with ``seqs``, of the slots of those sequences only."""
    if seqs is None:
        vm = valid_slot_mask(inp)
        blocks = None
    else:
        slots = inp.slot_mapping[seq_token_rows(inp, seqs)]
        blocks = np.unique(slots // 16)
        pos = np.searchsorted(blocks, slots // 16)
        vm = np.zeros((blocks.size, 16), bool)
        vm[pos, slots % 16] = True

    def pick(t, host):
        if blocks is None:
            return t.cpu().numpy() if not host else t
        if host:
            return t[blocks]
        return t[torch.from_numpy(blocks).to(t.device)].cpu().numpy()

    for which in ("k", "v"):
        got = pick(getattr(r.cache, which + "_pages"), False)
        ref = pick(getattr(oracle_cache, which + "_pages"), True)
        dt = getattr(oracle_cache, which + "_dtype")
        g = got.transpose(0, 2, 1, 3)[vm]      # [slots][H][rb]
        e = ref.transpose(0, 2, 1, 3)[vm]
        if dt in ("e4m3", "e5m2"):
            from oracle.codecs import fp8_is_nan_code
            both_nan = fp8_is_nan_code(g, dt) & fp8_is_nan_code(e, dt)
            bad = (g != e) & ~both_nan
        else:
            bad = g != e
        assert not bad.any(), f"{which}: {int(bad.sum())} code bytes differ (first at {np.argwhere(bad)[:3].tolist()})"
        if dt in ("int4", "int4h"):
            gm = pick(getattr(r.cache, which + "_meta"), False).transpose(0, 2, 1, 3)[vm]
            em = pick(getattr(oracle_cache, which + "_meta"), True).transpose(0, 2, 1, 3)[vm]
            assert meta_equal(gm, em), f"{which} int4 metadata differs"


def meta_equal(got, ref):
    """INT4 (scale, zero point) metadata: bit-equal float32 patterns, or NaN on
    both sides (an all-NaN row's NaNs may differ in sign and payload)."""
    g, e = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    both_nan = np.isnan(g) & np.isnan(e)
    return bool(np.all((g.view(np.uint32) == e.view(np.uint32)) | both_nan))


def bf16_half_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def gate_errors(out, ref, out_dtype):
    """Max abs error, and the violations of the tolerance for this output dtype.

    f32 output: |o - ref| <= 4e-3.  bf16 output: |o - ref| <= max(4e-3, half a bf16
    ulp of ref + 1e-4) — bf16 itself cannot hold |ref| >= 2 within 4e-3.
    """
    o = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    if out_dtype == "f32":
        tol = np.full_like(ref, 4e-3)
    else:
        tol = np.maximum(4e-3, bf16_half_ulp(ref) + 1e-4)
    fin = np.isfinite(ref)
    bad = (err > tol) | ~np.isfinite(o)
    return float(np.max(err[fin], initial=0.0)), int(bad[fin].sum())


def oracle_decode(oracle_cache, inp, heads=None, seqs=None):
    if inp.w.n_q > 1:
        return oa.verify(oracle_cache, inp.q_bits, inp.w.n_q, inp.block_tables, inp.seq_lens,
                         softmax_scale(inp.w.D), heads=heads, seqs=seqs)
    return oa.decode(oracle_cache, inp.q_bits, inp.block_tables, inp.seq_lens, softmax_scale(inp.w.D),
                     heads=heads, seqs=seqs)


def query_rows(inp, seqs):
    """Rows of q / out that belong to the given sequences (n_q per sequence)."""
    n = inp.w.n_q
    return [b * n + i for b in seqs for i in range(n)]


def sample_rows(inp, n_seqs, heads_per_seq, seed=0):
    rng = np.random.default_rng(seed)
    seqs = sorted(rng.choice(inp.w.B, size=min(n_seqs, inp.w.B), replace=False).tolist())
    heads = sorted(rng.choice(inp.w.Hq, size=min(heads_per_seq, inp.w.Hq), replace=False).tolist())
    return seqs, heads


def log(msg):
    print(msg, flush=True)


def ceil_div(a, b):
    return -(-a // b)


__all__ = ["dev_bf16", "meta_equal", "build_library_cache", "library_decode", "build_oracle_cache", "build_oracle_cache_sampled",
           "query_rows",
           "seq_token_rows", "assert_codes_equal",
           "gate_errors", "oracle_decode", "sample_rows", "log", "softmax_scale", "math", "ceil_div"]
