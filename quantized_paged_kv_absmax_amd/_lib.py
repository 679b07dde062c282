"""ctypes loader for libkvq.so (the C ABI declared in include/kvq.h).

Only argument marshalling lives here.  If the library has not been built the
import of the binding fails loudly: there is no fallback implementation.
"""

import ctypes
import os

# KVQ_LIBRARY may name another build of the same C ABI (the host sanitizer build
# lib/libkvq_hostsan.so, loaded by its test)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                          "libkvq.so")

# kvq_status
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)
# kvq_dtype
BF16, INT8, FP8_E4M3, FP8_E5M2, INT4_ASYM, F32, INT4_HAD = range(7)
# kvq_granularity
PER_TENSOR, PER_KV_HEAD, PER_TOKEN_HEAD = range(3)

DTYPES = {"bf16": BF16, "auto": BF16, "int8": INT8, "e4m3": FP8_E4M3, "fp8": FP8_E4M3, "fp8_e4m3": FP8_E4M3,
          "e5m2": FP8_E5M2, "fp8_e5m2": FP8_E5M2, "int4": INT4_ASYM, "f32": F32, "int4h": INT4_HAD}
DECODE_SCRATCH_BYTES = 64 << 20   # KVQ_DECODE_SCRATCH_BYTES
GRANULARITIES = {"per_tensor": PER_TENSOR, "per_kv_head": PER_KV_HEAD, "per_token_head": PER_TOKEN_HEAD}

EXPORTS = ("kvq_calibrate_scales", "kvq_cache_write", "kvq_convert_cache", "kvq_decode_workspace_size",
           "kvq_paged_attention_decode", "kvq_paged_attention_verify", "kvq_verify_workspace_size",
           "kvq_cache_block_bytes", "kvq_blocks_in_budget", "kvq_status_string", "kvq_abi_version",
           "kvq_hadamard_rotate", "kvq_paged_attention_decode_noalloc", "kvq_paged_attention_decode_write")


class KvqCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32),
        ("k_gran", ctypes.c_int32), ("v_gran", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load libkvq.so once and declare the prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkvq.so not built ({LIB_PATH}); run `python -m quantized_paged_kv_absmax_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    CP = ctypes.POINTER(KvqCacheStruct)
    lib.kvq_calibrate_scales.argtypes = [P, I64, I32, I32, I32, I32, P, P, P]
    lib.kvq_calibrate_scales.restype = I32
    lib.kvq_cache_write.argtypes = [CP, P, P, P, I64, P, P]
    lib.kvq_cache_write.restype = I32
    lib.kvq_convert_cache.argtypes = [CP, P, P, I32, I32, P]
    lib.kvq_convert_cache.restype = I32
    lib.kvq_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.kvq_decode_workspace_size.restype = SZ
    lib.kvq_paged_attention_decode.argtypes = [CP, P, P, I32, P, I32, I32, I32, F, I32, P, SZ, I32, P, P, P]
    lib.kvq_paged_attention_decode.restype = I32
    lib.kvq_paged_attention_decode_noalloc.argtypes = [CP, P, P, I32, P, I32, I32, I32, F, I32, I32, P, P, P]
    lib.kvq_paged_attention_decode_noalloc.restype = I32
    lib.kvq_paged_attention_decode_write.argtypes = [CP, P, P, P, P, P, I32, P, I32, I32, I32, F, I32, P, SZ, I32,
                                                     P, P, P]
    lib.kvq_paged_attention_decode_write.restype = I32
    lib.kvq_paged_attention_verify.argtypes = [CP, P, I32, P, I32, P, I32, I32, I32, F, I32, P, SZ, I32, P, P, P]
    lib.kvq_paged_attention_verify.restype = I32
    lib.kvq_verify_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.kvq_verify_workspace_size.restype = SZ
    lib.kvq_cache_block_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.kvq_cache_block_bytes.restype = ctypes.c_uint64
    lib.kvq_blocks_in_budget.argtypes = [ctypes.c_uint64, I32, I32, I32, I32, I32, I32]
    lib.kvq_blocks_in_budget.restype = ctypes.c_int64
    lib.kvq_hadamard_rotate.argtypes = [P, I64, I32, P, P]
    lib.kvq_hadamard_rotate.restype = I32
    lib.kvq_status_string.argtypes = [I32]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_abi_version.argtypes = []
    lib.kvq_abi_version.restype = I32
    _lib = lib
    return lib


class KvqError(RuntimeError):
    def __init__(self, status, fn):
        msg = load().kvq_status_string(status).decode()
        super().__init__(f"{fn}: {msg}")
        self.status = status


def check(status, fn):
    if status != OK:
        raise KvqError(status, fn)
