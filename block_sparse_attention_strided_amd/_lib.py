"""ctypes declarations of libxattn.so (the C ABI in include/xattn.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Loading fails loudly if the library has not been built.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libxattn.so")

XATTN_OK = 0
XATTN_ERR_INVALID = -1
XATTN_ERR_UNSUPPORTED = -2
XATTN_ERR_HIP = -3
XATTN_ERR_WORKSPACE = -4
XATTN_ERR_NOT_PINNED = -5

DTYPE_BF16 = 0
DTYPE_F32 = 1
SELECT_PER_KVHEAD = 0
SELECT_CHUNK_VOTE = 1
SELECT_CHUNK_VOTE_SPARSE = 2
GQA_ANY = 0
GQA_MAJORITY = 1

EXPORTED = (
    "xattn_workspace_size",
    "xattn_estimate",
    "xattn_select",
    "xattn_sparse_attn",
    "xattn_attn_plan",
    "xattn_attn_run",
    "xattn_merge_attn",
    "xattn_prefill_chunk",
    "xattn_prefill_chunk_static",
    "xattn_ring_create",
    "xattn_ring_destroy",
    "xattn_ring_create_staged",
    "xattn_ring_set_copy_delay_us",
    "xattn_ring_offload_chunk",
    "xattn_ring_offload_wait",
    "xattn_kernel_timing",
    "xattn_kernel_timing_read",
    "xattn_last_error",
)

_i32p = ctypes.POINTER(ctypes.c_int32)


class XattnShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int),
        ("num_q_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("cu_q_host", _i32p),
        ("cu_k_host", _i32p),
        ("cu_q", ctypes.c_void_p),
        ("cu_k", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int),
        ("num_phys_blocks", ctypes.c_int),
    ]


class XattnParams(ctypes.Structure):
    _fields_ = [
        ("stride", ctypes.c_int),
        ("block_size", ctypes.c_int),
        ("threshold", ctypes.c_float),
        ("est_scale", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("kv_chunk_tokens", ctypes.c_int),
        ("select_mode", ctypes.c_int),
        ("group_agg", ctypes.c_int),
        ("num_to_choose", ctypes.c_int),
        ("reuse_selection", ctypes.c_int),
    ]


class XattnAux(ctypes.Structure):
    _fields_ = [
        ("block_sums", ctypes.c_void_p),
        ("mask_kv", ctypes.c_void_p),
        ("hist_sel", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load libxattn.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libxattn.so is not built (%s); run `python -m block_sparse_attention_strided_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    sp = ctypes.POINTER(XattnShape)
    pp = ctypes.POINTER(XattnParams)
    vp = ctypes.c_void_p
    lib.xattn_workspace_size.argtypes = [sp, pp]
    lib.xattn_workspace_size.restype = ctypes.c_size_t
    lib.xattn_estimate.argtypes = [sp, pp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.xattn_estimate.restype = ctypes.c_int
    lib.xattn_select.argtypes = [sp, pp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.xattn_select.restype = ctypes.c_int
    lib.xattn_sparse_attn.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.xattn_sparse_attn.restype = ctypes.c_int
    lib.xattn_attn_plan.argtypes = [sp, pp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.xattn_attn_plan.restype = ctypes.c_int
    lib.xattn_attn_run.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.xattn_attn_run.restype = ctypes.c_int
    lib.xattn_merge_attn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    lib.xattn_merge_attn.restype = ctypes.c_int
    lib.xattn_prefill_chunk.argtypes = [vp, sp, pp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                        ctypes.POINTER(XattnAux), vp, ctypes.c_size_t, vp]
    lib.xattn_prefill_chunk.restype = ctypes.c_int
    lib.xattn_prefill_chunk_static.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(XattnAux), vp]
    lib.xattn_prefill_chunk_static.restype = ctypes.c_int
    lib.xattn_ring_create.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(vp)]
    lib.xattn_ring_create.restype = ctypes.c_int
    lib.xattn_ring_destroy.argtypes = [vp]
    lib.xattn_ring_create_staged.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_void_p)]
    lib.xattn_ring_create_staged.restype = ctypes.c_int
    lib.xattn_ring_destroy.restype = None
    lib.xattn_ring_set_copy_delay_us.argtypes = [vp, ctypes.c_int]
    lib.xattn_ring_offload_chunk.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.xattn_ring_offload_chunk.restype = ctypes.c_int
    lib.xattn_ring_offload_wait.argtypes = [vp, vp]
    lib.xattn_kernel_timing.argtypes = [ctypes.c_int]
    lib.xattn_kernel_timing.restype = ctypes.c_int
    lib.xattn_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.xattn_kernel_timing_read.restype = ctypes.c_int
    lib.xattn_ring_offload_wait.restype = ctypes.c_int
    lib.xattn_ring_set_copy_delay_us.restype = ctypes.c_int
    lib.xattn_last_error.argtypes = []
    lib.xattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error():
    return load().xattn_last_error().decode()
