"""Workload definitions and seeded generators (no method arithmetic here).

Workloads (sizes as the library is measured on; every one single-layer decode,
block_size 16):

  tiny_int8      B=2, lengths {17, 33}, Hq=Hkv=4, D=64; INT8 per-tensor
                 absmax/127 scales over all tokens; 2 of the 256 (head, dim) K
                 channels scaled x10.
  llama8b_int8   B=64, lengths U[512, 4096], Hq=32, Hkv=8, D=128; INT8
                 per-tensor scales over the prompt (all but the last token); 10
                 (= 1% of Hkv*D) K channels x8; the last token of each sequence is
                 written by the decode step itself (1 new token / sequence).
  fp8_*          B=256, L=768 (512 prompt + 256 decoded), 32/8/128; K channels as
                 above; e4m3/e4m3 (scale 1.0 or absmax/448), e5m2/e5m2 (1.0),
                 e4m3-K (1.0 or absmax/448) with int8-V (absmax/127).
  fp8_e4m3_head  as fp8_e4m3, with per-KV-head absmax/448 scales for K and V over
                 the prompt; every (K or V, head, channel) has its own standard
                 deviation from LogNormal(0, 0.5), so the heads' scales differ.
  fp8_e5m2_cal   as fp8_e5m2, with per-tensor absmax/57344 scales over the prompt.
  verify16_int8  the llama8b_int8 cache with 16 query tokens per sequence (the
                 last 16 positions, written by the step), attending causally:
                 a prefill chunk or a speculative verification of 15 drafts.
  longctx_int8   B=8, lengths U[32768, 131072], Hq=64, Hkv=8, D=128, INT8
                 per-KV-head scales calibrated on 64 synthetic 2048-token
                 sequences; every (K or V, head, channel) has its own standard
                 deviation drawn once from LogNormal(0, 0.5); decoded with
                 512-token work chunks (32 pages) and the merge pass.
  int4_had       as int4, with the keys Hadamard-rotated before their INT4 codes
                 (KVarN's rotation step); the query is rotated alike.
  int4           B=128, lengths U[1024, 8192], 32/8/128, INT4 asymmetric per
                 (token, KV head); K channels as above, V plain N(0,1); the cache
                 starts as bf16 pages and is converted.

The shapes follow Llama-3-8B's attention (32 query heads, 8 KV heads, head
dim 128), which is the model of the L4 benchmark in vLLM PR 4893; its
512-token prompts / 256 decoded tokens are the fp8 workload's context.  Those
benchmarks used trained weights and real prompts; normally distributed
synthetic values with a few large channels stand in for them here.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
import os

import numpy as np

BLOCK = 16


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    lens: tuple                 # ("fixed", (l0, l1, ...)) or ("uniform", lo, hi)
    k_dtype: str = "int8"
    v_dtype: str = "int8"
    k_gran: str = "per_tensor"  # per_tensor | per_kv_head | per_token_head
    v_gran: str = "per_tensor"
    k_scale_mode: str = "absmax"  # absmax | one | row (int4)
    v_scale_mode: str = "absmax"
    k_outliers: tuple = (0, 1.0)  # (number of (head, dim) channels, factor)
    lognormal_sigma: float = 0.0  # >0: per-channel std ~ LogNormal(0, sigma)
    calib: str = "prompt"         # prompt | all | set | none
    calib_set: tuple = (0, 0)     # (sequences, tokens each) for calib == "set"
    new_tokens: int = 1           # tokens written by the decode step itself
    n_q: int = 1                  # query tokens per sequence (>1: the last n_q positions, causally)
    partition: int = 0            # decode work split: 0 = the library's automatic chunks
    from_bf16_cache: bool = False  # cache starts as bf16 pages, then converted
    block_size: int = BLOCK

    def with_(self, **kw):
        return replace(self, **kw)


def _outliers(Hkv, D, frac):
    return (int(round(frac * Hkv * D)), 8.0)


WORKLOADS = {
    "tiny_int8": Workload("tiny_int8", 1, 2, 4, 4, 64, ("fixed", (17, 33)),
                          k_outliers=(2, 10.0), calib="all", new_tokens=0),
    "llama8b_int8": Workload("llama8b_int8", 2, 64, 32, 8, 128, ("uniform", 512, 4096),
                             k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=1),
    "fp8_e4m3": Workload("fp8_e4m3", 3, 256, 32, 8, 128, ("fixed", (768,)), "e4m3", "e4m3",
                         k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=256),
    "fp8_e4m3_s1": Workload("fp8_e4m3_s1", 3, 256, 32, 8, 128, ("fixed", (768,)), "e4m3", "e4m3",
                            k_scale_mode="one", v_scale_mode="one",
                            k_outliers=_outliers(8, 128, 0.01), calib="none", new_tokens=256),
    "fp8_e5m2": Workload("fp8_e5m2", 3, 256, 32, 8, 128, ("fixed", (768,)), "e5m2", "e5m2",
                         k_scale_mode="one", v_scale_mode="one",
                         k_outliers=_outliers(8, 128, 0.01), calib="none", new_tokens=256),
    "fp8_hybrid": Workload("fp8_hybrid", 3, 256, 32, 8, 128, ("fixed", (768,)), "e4m3", "int8",
                           k_scale_mode="absmax", v_scale_mode="absmax",
                           k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=256),
    "fp8_e4m3_head": Workload("fp8_e4m3_head", 6, 256, 32, 8, 128, ("fixed", (768,)), "e4m3", "e4m3",
                              k_gran="per_kv_head", v_gran="per_kv_head", lognormal_sigma=0.5,
                              k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=256),
    "fp8_e5m2_cal": Workload("fp8_e5m2_cal", 7, 256, 32, 8, 128, ("fixed", (768,)), "e5m2", "e5m2",
                             k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=256),
    "verify16_int8": Workload("verify16_int8", 8, 64, 32, 8, 128, ("uniform", 512, 4096),
                              k_outliers=_outliers(8, 128, 0.01), calib="prompt", new_tokens=16, n_q=16),
    "longctx_int8": Workload("longctx_int8", 4, 8, 64, 8, 128, ("uniform", 32768, 131072),
                             k_gran="per_kv_head", v_gran="per_kv_head", lognormal_sigma=0.5,
                             calib="set", calib_set=(64, 2048), new_tokens=1, partition=512),
    "int4": Workload("int4", 5, 128, 32, 8, 128, ("uniform", 1024, 8192), "int4", "int4",
                     k_gran="per_token_head", v_gran="per_token_head",
                     k_scale_mode="row", v_scale_mode="row",
                     k_outliers=_outliers(8, 128, 0.01), calib="none", new_tokens=0,
                     from_bf16_cache=True),
    "int4_had": Workload("int4_had", 9, 128, 32, 8, 128, ("uniform", 1024, 8192), "int4h", "int4",
                         k_gran="per_token_head", v_gran="per_token_head",
                         k_scale_mode="row", v_scale_mode="row",
                         k_outliers=_outliers(8, 128, 0.01), calib="none", new_tokens=0,
                         from_bf16_cache=True),
    "bf16": Workload("bf16", 2, 64, 32, 8, 128, ("uniform", 512, 4096), "bf16", "bf16",
                     k_scale_mode="one", v_scale_mode="one",
                     k_outliers=_outliers(8, 128, 0.01), calib="none", new_tokens=1),
}


# ---------------------------------------------------------------------------
# bf16 bit helpers (input preparation only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x):
    """float32 samples -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# generated inputs
# ---------------------------------------------------------------------------


@dataclass
class DecodeInputs:
    w: Workload
    seq_lens: np.ndarray        # int32 [B]
    q_bits: np.ndarray          # uint16 [B * n_q][Hq][D] (token-major within a sequence)
    k_bits: np.ndarray          # uint16 [Ntok][Hkv][D], token-major, sequences concatenated
    v_bits: np.ndarray          # uint16 [Ntok][Hkv][D]
    cu: np.ndarray              # int64 [B+1] token offsets of each sequence
    pos: np.ndarray             # int32 [Ntok] position of the token in its sequence
    block_tables: np.ndarray    # int32 [B][max_blocks], -1 past the end
    slot_mapping: np.ndarray    # int64 [Ntok]
    num_blocks: int
    outlier_channels: np.ndarray  # int64 [n][2] (head, dim) of the scaled K channels
    sigma_k: np.ndarray = None  # float32 [Hkv][D] or None
    sigma_v: np.ndarray = None

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def prompt_mask(self):
        """True for tokens written at set-up, False for the tokens of the decode step(s)."""
        L = self.seq_lens.astype(np.int64)
        return self.pos < np.repeat(L - self.w.new_tokens, L)


def _streams(seed, n=8):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _lengths(w, rng):
    kind = w.lens[0]
    if kind == "fixed":
        vals = list(w.lens[1])
        return np.array([vals[i % len(vals)] for i in range(w.B)], np.int32)
    lo, hi = w.lens[1], w.lens[2]
    return rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)


_CHUNK_ROWS = 1 << 14


def _chunked_bf16(rng, shape, chan_scale):
    """[chan_scale *] N(0,1) float32 draws rounded to bf16, in row chunks.

    Each chunk of _CHUNK_ROWS rows draws from its own PCG64 generator, seeded
    from ``rng`` in chunk order, so the values do not depend on how many
    threads fill the chunks (the draws run in parallel; numpy releases the GIL
    for them).
    """
    rows = shape[0]
    out = np.empty(shape, np.uint16)
    inner = int(np.prod(shape[1:]))
    n_chunks = -(-rows // _CHUNK_ROWS)
    seeds = rng.integers(0, 2 ** 63, size=n_chunks, dtype=np.int64)
    cs = None if chan_scale is None else np.asarray(chan_scale, np.float32)

    def fill(k):
        r0 = k * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        g = np.random.Generator(np.random.PCG64(int(seeds[k])))
        x = g.standard_normal((r1 - r0) * inner, dtype=np.float32).reshape((r1 - r0,) + tuple(shape[1:]))
        out[r0:r1] = f32_to_bf16_bits(x if cs is None else x * cs)

    if n_chunks <= 1:
        for k in range(n_chunks):
            fill(k)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _normal_bf16(rng, shape):
    """N(0,1) float32 draws rounded to bf16."""
    return _chunked_bf16(rng, shape, None)


def _scaled_normal_bf16(rng, shape, chan_scale):
    """chan_scale [Hkv][D] * N(0,1), rounded to bf16 once (the product is the sample)."""
    return _chunked_bf16(rng, shape, chan_scale)


def _channel_scales(w, streams):
    """Per-(head, dim) multipliers for K and V: outlier factors and/or LogNormal std."""
    r_out, r_sig = streams[4], streams[5]
    ck = np.ones((w.Hkv, w.D), np.float32)
    cv = np.ones((w.Hkv, w.D), np.float32)
    n, fac = w.k_outliers
    chans = np.zeros((0, 2), np.int64)
    if n:
        flat = r_out.choice(w.Hkv * w.D, size=n, replace=False)
        chans = np.stack([flat // w.D, flat % w.D], axis=1)
        ck[chans[:, 0], chans[:, 1]] *= np.float32(fac)
    sk = sv = None
    if w.lognormal_sigma > 0:
        sk = r_sig.lognormal(0.0, w.lognormal_sigma, size=(w.Hkv, w.D)).astype(np.float32)
        sv = r_sig.lognormal(0.0, w.lognormal_sigma, size=(w.Hkv, w.D)).astype(np.float32)
        ck *= sk
        cv *= sv
    return ck, cv, chans, sk, sv


def make_decode_inputs(w, B=None, lens=None):
    """All inputs of one workload.  ``B`` / ``lens`` override the batch for
    reduced-size parity cases (the draws keep the same generator recipe)."""
    if B is not None or lens is not None:
        w = w.with_(B=B if B is not None else w.B, lens=lens if lens is not None else w.lens)
    st = _streams(w.seed)
    seq_lens = _lengths(w, st[0])
    L64 = seq_lens.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(L64)]).astype(np.int64)
    ntok = int(cu[-1])
    q_bits = _normal_bf16(st[1], (w.B * w.n_q, w.Hq, w.D))
    ck, cv, chans, sk, sv = _channel_scales(w, st)
    shape = (ntok, w.Hkv, w.D)
    k_bits = _scaled_normal_bf16(st[2], shape, ck) if (ck != 1).any() else _normal_bf16(st[2], shape)
    v_bits = _scaled_normal_bf16(st[3], shape, cv) if (cv != 1).any() else _normal_bf16(st[3], shape)
    # pages: a pool of exactly sum ceil(L / bs) blocks, handed out in a seeded random order
    bs = w.block_size
    nblk_seq = -(-L64 // bs)
    num_blocks = int(nblk_seq.sum())
    perm = st[6].permutation(num_blocks).astype(np.int32)
    max_blocks = int(nblk_seq.max()) if w.B else 0
    bt = np.full((w.B, max(max_blocks, 1)), -1, np.int32)
    o = 0
    for b in range(w.B):
        n = int(nblk_seq[b])
        bt[b, :n] = perm[o:o + n]
        o += n
    pos = (np.arange(ntok, dtype=np.int64) - np.repeat(cu[:-1], L64)).astype(np.int32)
    seq_of = np.repeat(np.arange(w.B), L64)
    slot = bt[seq_of, pos // bs].astype(np.int64) * bs + (pos % bs)
    return DecodeInputs(w, seq_lens, q_bits, k_bits, v_bits, cu, pos, bt, slot, num_blocks,
                        chans, sk, sv)


def make_calibration_set(w, inp):
    """The calibration tokens of workload ``w`` as bf16 (K [T][Hkv][D], V [T][Hkv][D]).

    calib == "all":    every token of the cache;
    calib == "prompt": every token written at set-up (not the decode-step tokens);
    calib == "set":    a separate synthetic set of calib_set = (n, T) sequences drawn
                       with the same per-channel scales as the cache, from its own
                       stream;
    calib == "none":   no calibration (scales 1.0 or per-row).
    """
    if w.calib == "all":
        return inp.k_bits, inp.v_bits
    if w.calib == "prompt":
        m = inp.prompt_mask()
        return inp.k_bits[m], inp.v_bits[m]
    if w.calib == "set":
        st = _streams(w.seed)
        ck, cv, _, _, _ = _channel_scales(w, st)
        n, T = w.calib_set
        shape = (n * T, w.Hkv, w.D)
        return _scaled_normal_bf16(st[7], shape, ck), _scaled_normal_bf16(st[7], shape, cv)
    return None, None


def scatter_rows_to_pages(rows_bits, slot_mapping, num_blocks, block_size=BLOCK, fill=0xFFFF):
    """Lay token-major bf16 rows [T][Hkv][D] out as bf16 pages [num_blocks][Hkv][bs][D].

    Used to build an existing bf16 cache as the input of the conversion; unused
    slots hold ``fill`` (0xFFFF, a NaN).
    """
    T, H, D = rows_bits.shape
    pages = np.full((num_blocks, H, block_size, D), fill, np.uint16)
    s = np.asarray(slot_mapping, np.int64)
    pages[s // block_size, :, s % block_size, :] = rows_bits
    return pages
