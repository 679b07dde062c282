"""Oracle paged-attention decode — TEST INFRASTRUCTURE ONLY.

The pages name the operation only: decode runs a paged-attention kernel over
the cache (vLLM PR 4893, side note on attention backends), and that kernel,
given the quantisation parameters, reads the stored codes, converts them back
and computes (vLLM issue 4025, methods item 3).  What it computes is the
textbook single-query softmax attention, written out here:

  for sequence b and query head h, KV head kv = h // g  (g = Hq / Hkv; consecutive
  query heads share a KV head — the plainest grouped-query reading),
      z_i = softmax_scale * sum_c q_c * k_hat_{i,c}        for i < L_b
      o   = sum_i exp(z_i - max z) * v_hat_i / sum_i exp(z_i - max z)

in float64 over exact float32 q (bf16 widened), k_hat and v_hat (the decoded
cache values).  Positions >= L_b are excluded, never multiplied by zero: an
unused slot may hold a NaN code.  L_b <= 0 gives a zero row.

Split form: positions are cut into partitions of ``partition`` tokens; each
gives (m_j, l_j, acc_j) = (max z, sum exp(z - m_j), sum exp(z - m_j) v_hat), and
      o = sum_j exp(m_j - M) acc_j / sum_j exp(m_j - M) l_j,   M = max_j m_j.

Several query tokens per sequence (``verify``): token i of the last n_q
positions attends causally to positions 0..L_b - n_q + i.

Rotated keys (K dtype "int4h", KVarN's rotation step, techfi24's KVarN article,
"Contexte Technique"): the cache holds INT4 codes of H k (H the Sylvester-Hadamard
matrix, H H = D I).  The key such a slot holds is the de-rotated row
k_hat = H k_hat_rot / D, and attention is the plain formula above over those keys
with the caller's query and softmax scale as given.

Pins (tests/test_oracle_attention.py): q = 0 gives the mean of v_hat; one
token gives v_hat_0; adding a constant to every logit changes nothing; a
permuted page pool gives bit-identical output to the contiguous order; g = 1
and repeated KV heads agree; torch's scaled_dot_product_attention in float64
on the same decoded tensors; split == unsplit.
"""

import numpy as np

from . import codecs


def _keys(cache, block_table_row, L, heads=None):
    """Dequantised keys of one sequence's first L positions, float64 [L][h][D].
    A rotated-key ("int4h") slot holds H k; its key is H (H k) / D, taken in
    float64 (a product of at most 128 float32 terms per element)."""
    K = cache.gather(block_table_row, L, "k", heads).astype(np.float64)
    if cache.k_dtype == "int4h":
        H = codecs.hadamard_matrix(cache.D).astype(np.float64)
        K = (K @ H.T) / cache.D
    return K


def _attend(qv, K, V, softmax_scale):
    """One query head: qv [D] f64, K/V [L][D] f64 -> o [D] f64."""
    z = softmax_scale * (K @ qv)
    m = z.max()
    e = np.exp(z - m)
    return (e @ V) / e.sum()


def decode(cache, q_bits, block_tables, seq_lens, softmax_scale, heads=None, seqs=None):
    """Paged decode of every (sequence, query head) -> float64 [B][Hq][D].

    cache: oracle.cache.PagedCache; q_bits: bf16 [B][Hq][D]; block_tables int
    [B][max_blocks]; seq_lens int [B]; softmax_scale: the float32 value the
    caller passes (used exactly).  ``heads`` / ``seqs`` restrict the work to a
    subset (other rows are left NaN), for sampled checks at large sizes.
    """
    q = codecs.bf16_to_f32(np.asarray(q_bits, np.uint16)).astype(np.float64)
    B, Hq, D = q.shape
    g = Hq // cache.H
    sm = float(np.float32(softmax_scale))
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        hs = range(Hq) if heads is None else heads
        if L <= 0:
            for h in hs:
                out[b, h] = 0.0
            continue
        kvs = sorted({h // g for h in hs})
        K = _keys(cache, block_tables[b], L, kvs)                         # [L][len(kvs)][D]
        V = cache.gather(block_tables[b], L, "v", kvs).astype(np.float64)
        col = {kv: i for i, kv in enumerate(kvs)}
        for h in hs:
            c = col[h // g]
            out[b, h] = _attend(q[b, h], K[:, c, :], V[:, c, :], sm)
    return out


def verify(cache, q_bits, n_q, block_tables, seq_lens, softmax_scale, heads=None, seqs=None):
    """Several query tokens per sequence over the paged cache, causally
    -> float64 [B * n_q][Hq][D].

    The multi-token form of the same paged attention (the row of the survey's
    next steps built on vLLM PR 4893's side note on attention backends, which
    leaves quantised-KV attention with several query tokens to the paged
    kernel): speculative verification or a prefill chunk.  The last n_q
    positions of sequence b are its query tokens; row t = b * n_q + i is token
    i, at position p = L_b - n_q + i, and attends to positions 0..p of the cache
    (its own and every earlier one), exactly as ``decode`` with L = p + 1.
    p < 0 (a sequence shorter than n_q) gives a zero row.  ``heads`` / ``seqs``
    restrict the work (other rows NaN).
    """
    q = codecs.bf16_to_f32(np.asarray(q_bits, np.uint16)).astype(np.float64)
    T, Hq, D = q.shape
    B = T // n_q
    g = Hq // cache.H
    sm = float(np.float32(softmax_scale))
    out = np.full((T, Hq, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        hs = range(Hq) if heads is None else heads
        kvs = sorted({h // g for h in hs})
        col = {kv: i for i, kv in enumerate(kvs)}
        if L > 0:
            K = _keys(cache, block_tables[b], L, kvs)
            V = cache.gather(block_tables[b], L, "v", kvs).astype(np.float64)
        for i in range(n_q):
            t, pos = b * n_q + i, L - n_q + i
            for h in hs:
                if pos < 0:
                    out[t, h] = 0.0
                    continue
                c = col[h // g]
                out[t, h] = _attend(q[t, h], K[:pos + 1, c, :], V[:pos + 1, c, :], sm)
    return out


def decode_partials(cache, q_bits, block_tables, seq_lens, softmax_scale, partition):
    """Per-partition (m, l, acc) of the split form.

    Returns m, l float64 [B][Hq][P] and acc float64 [B][Hq][P][D], P = number of
    partitions of the longest sequence.  Partitions with no tokens hold
    m = -inf, l = 0, acc = 0.
    """
    q = codecs.bf16_to_f32(np.asarray(q_bits, np.uint16)).astype(np.float64)
    B, Hq, D = q.shape
    g = Hq // cache.H
    sm = float(np.float32(softmax_scale))
    Lmax = max(int(x) for x in seq_lens) if len(seq_lens) else 0
    P = max(1, -(-Lmax // partition))
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    acc = np.zeros((B, Hq, P, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = _keys(cache, block_tables[b], L)
        V = cache.gather(block_tables[b], L, "v").astype(np.float64)
        for h in range(Hq):
            z = sm * (K[:, h // g, :] @ q[b, h])
            for j in range(-(-L // partition)):
                sl = slice(j * partition, min(L, (j + 1) * partition))
                mj = z[sl].max()
                e = np.exp(z[sl] - mj)
                m[b, h, j], l[b, h, j] = mj, e.sum()
                acc[b, h, j] = e @ V[sl, h // g, :]
    return m, l, acc


def combine(m, l, acc):
    """Merge partitions: o = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j."""
    M = m.max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(m), np.exp(m - M), 0.0)
        num = (w[..., None] * acc).sum(axis=-2)
        den = (w * l).sum(axis=-1)
        out = num / den[..., None]
    return np.where(den[..., None] > 0, out, 0.0)


def decode_split(cache, q_bits, block_tables, seq_lens, softmax_scale, partition):
    return combine(*decode_partials(cache, q_bits, block_tables, seq_lens, softmax_scale, partition))
