"""CPU oracle for the quantized paged KV cache — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct definition of what the GPU
library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, links or calls anything here, and
this package imports nothing from the product package.

Sources (cited by page title and section):

* "vllm-int8-kv-cache-for-ampere-sm86" project summary: INT8 KV cache with
  per-layer scaling values calibrated offline; FP8-E4M3 emulated for one part
  of the cache.
* vLLM PR 4893 "[Misc] Load FP8 kv-cache scaling factors from checkpoints":
  the KV dtype set {auto, fp8, fp8_e4m3, fp8_e5m2} and the default scale 1.0
  (description, items 1-2); the L4 benchmark table (GPU blocks per dtype);
  decode runs a paged-attention kernel (the side note on backends).
* vLLM issue 4025 "[Feature]: Support for 4-bit KV Cache in paged-attention
  op", section "methods": compute scale + zero point and convert an existing
  bf16 cache to int4 (item 1); store 4-bit KV in the paged-cache write (item 2);
  paged attention with optional k_scale, k_zeropoint, v_scale, v_zeropoint that
  converts the stored codes back to 16-bit and computes (item 3).
* modelium "vLLM FP8 KV-кеш: калибровка и проверка памяти и качества",
  section on scale schemes: per-tensor and per-attention-head scales.

The pages print no formula, rounding rule or bit layout; the readings taken
where they are silent are listed in each function's docstring.

Modules:
  codecs    - bf16 widening, INT8 / FP8 (OCP e4m3, e5m2) / INT4-asymmetric
              encode and decode, byte accounting.
  cache     - absmax calibration, paged cache write by slot mapping, bf16 cache
              conversion, page gather.
  attention - fp64 paged decode, its split (partition + combine) form.

Every function here is pinned by a CPU test against something other than
itself (closed forms, brute force, invariants, a library routine, or the
numbers printed on the pages).  See the pin table in each module header.
"""

from . import codecs, cache, attention  # noqa: F401
