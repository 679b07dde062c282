"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module holds no arithmetic of the method: it draws random bf16 Q/K/V,
sequence lengths, outlier channels, per-channel standard deviations and a
page permutation, and lays the draws out as the inputs the library takes
(token-major rows, block tables, slot mappings, bf16 pages).  Quantisation,
calibration and attention live in the oracle and in the HIP library, never here.

Generator: numpy.random.Generator(PCG64) seeded with the workload number; each
kind of draw uses its own child stream of SeedSequence(seed).spawn(...), so
changing one draw's size does not move the others.  Samples are float32,
rounded to bf16 (round-to-nearest-even on the bit pattern).
"""

from .configs import (  # noqa: F401
    WORKLOADS, Workload, DecodeInputs, make_decode_inputs, make_calibration_set,
    f32_to_bf16_bits, bf16_bits_to_f32, scatter_rows_to_pages,
)
