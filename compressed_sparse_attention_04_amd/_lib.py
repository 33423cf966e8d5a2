"""ctypes loader of libcsa.so and the C declarations of include/csa.h.

Only argument marshalling lives here.  The library is the in-tree build of
csrc/ (``python -m compressed_sparse_attention_04_amd.build``); when it is
missing every call raises: there is no fallback path.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA_LIB_PATH selects another build of the same library (the sanitized
# host build of the checked CPU tests); there is no fallback either way.
LIB_PATH = os.environ.get("CSA_LIB_PATH") or os.path.join(_HERE, "libcsa.so")

c_void_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_size = ctypes.c_size_t


class CsaLayerArgs(ctypes.Structure):
    """Mirror of ``csa_layer_args`` in include/csa.h (field order matters)."""
    _fields_ = [
        ("codes", c_void_p), ("scales", c_void_p), ("kv_rows", c_i64),
        ("k_fp8", c_void_p), ("k_rows", c_i64), ("n_entries", c_i64),
        ("win", c_void_p), ("win_cap", c_i64),
        ("n_seq", c_i64), ("q_per_seq", c_i64),
        ("q_pos", c_void_p), ("q_attn", c_void_p), ("q_idx", c_void_p), ("w_idx", c_void_p),
        ("sm_scale", c_f32), ("top_k", c_i32), ("build_pool", c_i32), ("n_pool_blocks", c_i32),
        ("pool_blocks", c_void_p), ("idx", c_void_p), ("out", c_void_p),
        ("ws", c_void_p), ("ws_bytes", c_size), ("attn_after", c_void_p),
    ]


# name -> (restype, argtypes); must match include/csa.h
SIGNATURES = {
    "csa_status_string": (ctypes.c_char_p, [c_i32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_version": (c_i32, []),
    "csa_quantize": (c_i32, [c_void_p, c_i64, c_void_p, c_void_p, c_void_p]),
    "csa_dequantize": (c_i32, [c_void_p, c_void_p, c_i64, c_void_p, c_void_p]),
    "csa_compress_quant_workspace_size": (c_size, [c_i64]),
    "csa_compress_quant": (c_i32, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i32, c_f32,
                                   c_void_p, c_void_p, c_i64, c_void_p, c_void_p, c_size, c_void_p]),
    "csa_window_append": (c_i32, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p]),
    "csa_compress_quant_append": (c_i32, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i32, c_f32,
                                          c_void_p, c_void_p, c_i64, c_void_p, c_void_p, c_size,
                                          c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p]),
    "csa_window_rebuild": (c_i32, [c_void_p, c_i64, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p]),
    "csa_kv_save": (c_i32, [ctypes.c_char_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_void_p, c_size,
                            c_void_p]),
    "csa_kv_load": (c_i32, [ctypes.c_char_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_size,
                            c_void_p]),
    "csa_kv_file_info": (c_i32, [ctypes.c_char_p, c_void_p, c_void_p]),
    "csa_probe_mfma_f16": (c_i32, [c_void_p, c_i32, c_i32, c_void_p]),
    "csa_probe_mfma_f8": (c_i32, [c_void_p, c_i32, c_i32, c_i32, c_void_p]),
    "csa_probe_read": (c_i32, [c_void_p, c_i64, c_void_p, c_void_p]),
    "csa_index_score": (c_i32, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_i64, c_i64,
                                c_void_p, c_i32, c_void_p, c_void_p, c_void_p]),
    "csa_topk_workspace_size": (c_size, [c_i64, c_i64, c_i32]),
    "csa_topk": (c_i32, [c_void_p, c_i64, c_i64, c_void_p, c_i32, c_void_p, c_void_p, c_size, c_void_p]),
    "csa_block_pool_workspace_size": (c_size, [c_i64, c_i64, c_i32, c_i32]),
    "csa_block_pool": (c_i32, [c_void_p, c_i32, c_i64, c_i64, c_i32, c_void_p, c_void_p, c_size,
                               c_void_p]),
    "csa_sparse_attn_workspace_size": (c_size, [c_i64, c_i32]),
    "csa_sparse_attn": (c_i32, [c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p,
                                c_i32, c_void_p, c_i64, c_f32, c_void_p, c_void_p, c_size, c_void_p]),
    "csa_noalloc_scratch_bytes": (c_size, []),
    "csa_sparse_attn_noalloc": (c_i32, [c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_i64, c_void_p,
                                        c_i32, c_void_p, c_i64, c_f32, c_void_p, c_void_p]),
    "csa_layer_workspace_size": (c_size, [c_i32, ctypes.POINTER(CsaLayerArgs)]),
    "csa_layer_full": (c_i32, [ctypes.POINTER(CsaLayerArgs), c_void_p]),
    "csa_layer_reindex": (c_i32, [ctypes.POINTER(CsaLayerArgs), c_void_p]),
    "csa_layer_reuse": (c_i32, [ctypes.POINTER(CsaLayerArgs), c_void_p]),
}

_lib = None


def load():
    """Load libcsa.so once (after torch, so that torch's HIP runtime is the one used)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads the HIP runtime the library links against
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m compressed_sparse_attention_04_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
