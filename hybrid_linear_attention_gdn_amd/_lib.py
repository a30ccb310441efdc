"""ctypes declarations of the C ABI in include/sanawm_gdn.h and include/sanawm_attn.h
(argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsanawm_gdn.so")

GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP, GDN_ERR_INTERNAL = range(6)
GDN_F32, GDN_BF16, GDN_FP8_E4M3 = 0, 1, 2
GDN_FLAG_BETA_IS_PROB, GDN_FLAG_QK_PRENORMALIZED, GDN_FLAG_REVERSE = 1, 2, 8

# every symbol include/sanawm_gdn.h declares
EXPORTED = ("gdn_chunk_len", "gdn_workspace_bytes", "gdn_fwd", "gdn_chunk_step", "gdn_workspace_layout",
            "gdn_fwd_no_alloc",
            "gdn_bidir_workspace_bytes", "gdn_bidir_fwd",
            "gdn_in_proj", "gdn_out_proj", "gdn_layer_workspace_bytes", "gdn_layer_fwd",
            "gdn_status_string", "gdn_last_error", "gdn_version")
GDN_LAYER_BIDIRECTIONAL = 16
GDN_NO_ALLOC_SCRATCH_BYTES = 64 << 20
# every symbol include/sanawm_attn.h declares
EXPORTED_ATTN = ("attn_cache_bytes", "attn_block_fwd")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class LayerProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("frame_tokens", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class AttnProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frame_tokens", ctypes.c_int32), ("frames_per_block", ctypes.c_int32),
                ("cached_blocks", ctypes.c_int32), ("sink_frames", ctypes.c_int32), ("o_dtype", ctypes.c_int32)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_size_t), ("rq", ctypes.c_size_t), ("rk", ctypes.c_size_t),
                ("gcum", ctypes.c_size_t), ("rec", ctypes.c_size_t), ("rec_bytes", ctypes.c_size_t),
                ("carry", ctypes.c_size_t), ("range_cap", ctypes.c_int32), ("first_range", ctypes.c_int32),
                ("total", ctypes.c_size_t), ("mfma", ctypes.c_int32)]


_lib = None


def load():
    """Open libsanawm_gdn.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m hybrid_linear_attention_gdn_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(Problem)
    lib.gdn_chunk_len.restype = ctypes.c_int32
    lib.gdn_chunk_len.argtypes = []
    lib.gdn_version.restype = ctypes.c_int32
    lib.gdn_version.argtypes = []
    lib.gdn_workspace_bytes.restype = ctypes.c_int
    lib.gdn_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
    lib.gdn_workspace_layout.restype = ctypes.c_int
    lib.gdn_workspace_layout.argtypes = [P, ctypes.POINTER(WorkspaceLayout)]
    for fn in (lib.gdn_fwd, lib.gdn_chunk_step):
        fn.restype = ctypes.c_int
        fn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_fwd_no_alloc.restype = ctypes.c_int
    lib.gdn_fwd_no_alloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_bidir_workspace_bytes.restype = ctypes.c_int
    lib.gdn_bidir_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
    lib.gdn_bidir_fwd.restype = ctypes.c_int
    lib.gdn_bidir_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    LP = ctypes.POINTER(LayerProblem)
    lib.gdn_in_proj.restype = ctypes.c_int
    lib.gdn_in_proj.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_out_proj.restype = ctypes.c_int
    lib.gdn_out_proj.argtypes = [LP, vp, vp, vp, vp]
    lib.gdn_layer_workspace_bytes.restype = ctypes.c_int
    lib.gdn_layer_workspace_bytes.argtypes = [LP, ctypes.POINTER(sz)]
    lib.gdn_layer_fwd.restype = ctypes.c_int
    lib.gdn_layer_fwd.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    A = ctypes.POINTER(AttnProblem)
    lib.attn_cache_bytes.restype = ctypes.c_int
    lib.attn_cache_bytes.argtypes = [A, ctypes.POINTER(sz)]
    lib.attn_block_fwd.restype = ctypes.c_int
    lib.attn_block_fwd.argtypes = [A, ctypes.c_int32, vp, vp, vp, vp, sz, vp, vp]
    _lib = lib
    return lib
