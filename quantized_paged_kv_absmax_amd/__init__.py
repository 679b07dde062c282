"""Quantized paged KV cache with paged-attention decode for AMD MI355X (gfx950).

The work runs in libkvq.so (hand-written HIP; C ABI in include/kvq.h); this
package is its thin Python binding.  Importing the binding does not load the
library; the first call does, and raises ImportError if it has not been built
(`python -m quantized_paged_kv_absmax_amd.build`).
"""

from ._lib import (  # noqa: F401
    BF16, INT8, FP8_E4M3, FP8_E5M2, INT4_ASYM, INT4_HAD, F32, PER_TENSOR, PER_KV_HEAD, PER_TOKEN_HEAD,
    KvqError, LIB_PATH, load,
)
from .api import (  # noqa: F401
    PagedKVCache, kvq_calibrate_scales, kvq_cache_write, kvq_convert_cache, kvq_decode_workspace_size,
    kvq_paged_attention_decode, kvq_paged_attention_verify, kvq_verify_workspace_size, kvq_cache_block_bytes,
    kvq_blocks_in_budget, kvq_hadamard_rotate, kvq_paged_attention_decode_noalloc, kvq_paged_attention_decode_write,
    row_bytes,
)
