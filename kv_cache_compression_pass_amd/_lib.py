"""ctypes declarations of libkvc's C ABI (include/kvc.h).

Loading fails loudly: there is no fallback of any kind when the library is missing.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK = 0
STATUS_NAMES = {
    0: "KVC_OK", 1: "KVC_ERR_INVALID_ARG", 2: "KVC_ERR_UNSUPPORTED", 3: "KVC_ERR_WORKSPACE",
    4: "KVC_ERR_NO_DEVICE", 5: "KVC_ERR_HIP", 6: "KVC_ERR_DEVICE_DATA",
}

OP_ROW_LSE, OP_SCORE_TOKENS, OP_CHANNEL_WEIGHTS, OP_ALLOCATE_BITS, OP_QUANTIZE_PACK, \
    OP_COMPRESSED_ATTEND, OP_RIDGE_FIT = range(7)
SCORE_SUM, SCORE_MAX = 0, 1
ALLOC_V_TOKENS, ALLOC_K_CHANNELS, ALLOC_TOPK = 0, 1, 2
PK_NBUF = 9
PK_NAMES = ("header", "v_idx", "v_words", "v_par", "k_keep", "k_vloc", "k_words", "k_par",
            "k_width")
HDR_GLOBAL = 16
HDR_PER_HEAD = 24
DEV_BAD_WIDTH = 1
DEV_BAD_CACHE = 2
DEV_NOT_SPD = 4

EXPORTED = (
    "kvc_workspace_size", "kvc_row_lse", "kvc_row_lse_noalloc", "kvc_score_tokens", "kvc_channel_weights",
    "kvc_allocate_bits", "kvc_keep_threshold", "kvc_packed_capacity", "kvc_quantize_pack",
    "kvc_compressed_attend", "kvc_compressed_attend_append", "kvc_fidelity_terms", "kvc_pilot_budgets",
    "kvc_ridge_value_fit", "kvc_get_device_status", "kvc_status_string", "kvc_last_error", "kvc_version",
)


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("n_keys", ctypes.c_int64),
        ("n_queries", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


class KvzipArgs(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_void_p),
        ("w_o", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("hidden_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class AllocResult(ctypes.Structure):
    _fields_ = [
        ("lambda_", ctypes.c_double),
        ("budget_bits", ctypes.c_int64),
        ("used_bits", ctypes.c_int64),
        ("distortion", ctypes.c_double),
    ]


class PackedCacheC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PK_NAMES]


_lib = None


def load():
    """Load libkvc.so from the package directory; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libkvc.so not found at {LIB_PATH}; build it first "
            "(python -m kv_cache_compression_pass_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.c_size_t
    I32 = ctypes.c_int32
    D = ctypes.POINTER(LayerDesc)
    lib.kvc_workspace_size.argtypes = [I32, D, I32]
    lib.kvc_workspace_size.restype = S
    lib.kvc_row_lse.argtypes = [D, P, P, P, P, S, P]
    lib.kvc_row_lse_noalloc.argtypes = [D, P, P, P, P]
    lib.kvc_score_tokens.argtypes = [D, I32, P, P, P, ctypes.POINTER(KvzipArgs), P, P, S, P]
    lib.kvc_channel_weights.argtypes = [D, P, P, P, P, S, P]
    lib.kvc_allocate_bits.argtypes = [D, I32, P, P, P, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_uint8, P, P, P, S, P]
    lib.kvc_keep_threshold.argtypes = [D, P, ctypes.c_float, ctypes.c_int64, ctypes.c_uint8, P, P, P]
    lib.kvc_packed_capacity.argtypes = [D, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvc_quantize_pack.argtypes = [D, P, P, P, P, I32, ctypes.POINTER(PackedCacheC), P, S, P]
    lib.kvc_compressed_attend.argtypes = [D, P, ctypes.POINTER(PackedCacheC), P, P, P, S, P]
    lib.kvc_compressed_attend_append.argtypes = [D, P, ctypes.POINTER(PackedCacheC), P, P, ctypes.c_int64,
                                                 P, P, P, S, P]
    lib.kvc_fidelity_terms.argtypes = [D, P, P, P, P, P, P]
    lib.kvc_pilot_budgets.argtypes = [ctypes.POINTER(ctypes.c_double), I32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.kvc_ridge_value_fit.argtypes = [D, ctypes.c_int64, P, P, P, P, ctypes.c_double, P, P, S, P]
    lib.kvc_get_device_status.argtypes = [P, ctypes.POINTER(I32), P]
    for name in ("kvc_row_lse", "kvc_row_lse_noalloc", "kvc_score_tokens", "kvc_channel_weights", "kvc_allocate_bits", "kvc_keep_threshold",
                 "kvc_packed_capacity", "kvc_quantize_pack", "kvc_compressed_attend",
                 "kvc_compressed_attend_append", "kvc_fidelity_terms", "kvc_pilot_budgets",
                 "kvc_ridge_value_fit", "kvc_get_device_status"):
        getattr(lib, name).restype = I32
    lib.kvc_status_string.argtypes = [I32]
    lib.kvc_status_string.restype = ctypes.c_char_p
    lib.kvc_last_error.argtypes = []
    lib.kvc_last_error.restype = ctypes.c_char_p
    lib.kvc_version.argtypes = []
    lib.kvc_version.restype = ctypes.c_char_p
    _lib = lib
    return lib
