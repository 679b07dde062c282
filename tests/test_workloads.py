"""The seeded input generators: deterministic, and the paging inputs are consistent."""

import numpy as np

from workloads import WORKLOADS, make_decode_inputs, make_calibration_set


def test_deterministic_and_valid_paging():
    for name in ("tiny_int8", "fp8_hybrid"):
        w = WORKLOADS[name]
        kw = {} if name == "tiny_int8" else dict(B=5, lens=("fixed", (40,)))
        a = make_decode_inputs(w, **kw)
        b = make_decode_inputs(w, **kw)
        assert np.array_equal(a.k_bits, b.k_bits) and np.array_equal(a.block_tables, b.block_tables)
        # the pool is exactly sum ceil(L/16) blocks, each used once
        used = np.concatenate([a.block_tables[i, : -(-int(L) // 16)] for i, L in enumerate(a.seq_lens)])
        assert sorted(used.tolist()) == list(range(a.num_blocks))
        # slots of sequence b point into its own blocks at position order
        for i in range(a.w.B):
            s = a.slot_mapping[a.cu[i]:a.cu[i + 1]]
            p = np.arange(a.seq_lens[i])
            assert np.array_equal(s // 16, a.block_tables[i, p // 16]) and np.array_equal(s % 16, p % 16)


def test_tiny_lengths_and_outliers():
    a = make_decode_inputs(WORKLOADS["tiny_int8"])
    assert a.seq_lens.tolist() == [17, 33]
    assert a.outlier_channels.shape == (2, 2)
    k, v = make_calibration_set(a.w, a)
    assert k.shape[0] == 50


def test_uniform_lengths_in_range():
    w = WORKLOADS["llama8b_int8"]
    a = make_decode_inputs(w, B=16, lens=("uniform", 20, 70))
    assert a.seq_lens.min() >= 20 and a.seq_lens.max() <= 70
    assert a.outlier_channels.shape == (10, 2)
    m = a.prompt_mask()
    assert m.sum() == a.seq_lens.sum() - 16
