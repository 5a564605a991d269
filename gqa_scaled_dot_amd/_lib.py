"""ctypes view of libattn.so (declared in include/attn.h). Marshalling only."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_DEVICE = 0, 1, 2, 3
ATTN_ALIBI_NONE, ATTN_ALIBI_BLOOM, ATTN_ALIBI_MPT, ATTN_ALIBI_EXPLICIT = 0, 1, 2, 3
ATTN_ALIBI_MAX_HEADS = 256
ATTN_PB_MAX_BUCKETS, ATTN_PB_MAX_DIST = 128, 512
ATTN_BIAS_NONE, ATTN_BIAS_TS, ATTN_BIAS_HTS = 0, 1, 2
ATTN_PATH_EMPTY, ATTN_PATH_ZERO, ATTN_PATH_GENERIC, ATTN_PATH_DECODE, ATTN_PATH_PREFILL = 0, 1, 2, 3, 4
ATTN_PATH_MLA = 5
PATH_NAMES = {0: "empty", 1: "zero", 2: "generic", 3: "decode", 4: "prefill", 5: "mla"}
(ATTN_ROPE_DEFAULT, ATTN_ROPE_LINEAR, ATTN_ROPE_LLAMA3, ATTN_ROPE_YARN, ATTN_ROPE_LONGROPE,
 ATTN_ROPE_DYNAMIC) = range(6)
ATTN_ROPE_MAX_ROTARY_DIM = 256
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20
ROPE_SCALING = {"default": ATTN_ROPE_DEFAULT, "linear": ATTN_ROPE_LINEAR, "llama3": ATTN_ROPE_LLAMA3,
                "yarn": ATTN_ROPE_YARN, "longrope": ATTN_ROPE_LONGROPE, "dynamic": ATTN_ROPE_DYNAMIC}

# Every symbol include/attn.h declares.
EXPORTS = (
    "attn_params_init", "attn_validate", "attn_workspace_size", "attn_forward",
    "attn_forward_append", "attn_cache_write", "attn_cache_write2", "attn_last_error", "attn_plan",
    "attn_set_option", "attn_timing_enable", "attn_timing_collect",
    "attn_rope_params_init", "attn_rope_table", "attn_rope", "attn_rope_cache_write",
    "attn_mla_params_init", "attn_mla_validate", "attn_mla_workspace_size", "attn_mla_plan",
    "attn_mla_forward", "attn_forward_noalloc",
)


class AttnRopeParams(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int64), ("rotary_dim", ctypes.c_int64), ("offset", ctypes.c_int64),
        ("interleaved", ctypes.c_int32), ("scaling", ctypes.c_int32),
        ("base", ctypes.c_double),
        ("inv_freq", ctypes.POINTER(ctypes.c_float)),
        ("has_attention_factor", ctypes.c_int32), ("attention_factor", ctypes.c_float),
        ("factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double), ("high_freq_factor", ctypes.c_double),
        ("original_max_positions", ctypes.c_int64), ("max_positions", ctypes.c_int64),
        ("beta_fast", ctypes.c_double), ("beta_slow", ctypes.c_double),
        ("mscale", ctypes.c_double), ("mscale_all_dim", ctypes.c_double),
        ("truncate", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("short_factor", ctypes.POINTER(ctypes.c_double)),
        ("long_factor", ctypes.POINTER(ctypes.c_double)),
        ("scaling_attention_factor", ctypes.c_double),
    ]


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("S", ctypes.c_int64),
        ("heads", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64), ("v_head_dim", ctypes.c_int64),
        ("pos_offset", ctypes.c_int64), ("window", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("has_scale", ctypes.c_int32),
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
        ("alibi", ctypes.c_int32), ("alibi_max", ctypes.c_float),
        ("alibi_slopes", ctypes.POINTER(ctypes.c_float)),
        ("bias_kind", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("q_rope", ctypes.POINTER(AttnRopeParams)),
        ("sinks", ctypes.c_int64),
        ("pb_weight", ctypes.c_void_p), ("pb_buckets", ctypes.POINTER(ctypes.c_int64)),
        ("pb_n", ctypes.c_int64), ("pb_bidirectional", ctypes.c_int32), ("reserved2", ctypes.c_int32),
        ("rel_k", ctypes.c_void_p), ("rel_v", ctypes.c_void_p), ("rel_max", ctypes.c_int64),
    ]


class AttnMlaParams(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("S", ctypes.c_int64),
        ("heads", ctypes.c_int64), ("kv_rank", ctypes.c_int64), ("qk_nope", ctypes.c_int64),
        ("qk_rope", ctypes.c_int64), ("v_head_dim", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("has_scale", ctypes.c_int32),
        ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("pos_offset", ctypes.c_int64), ("window", ctypes.c_int64), ("sinks", ctypes.c_int64),
    ]


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("tile_q", ctypes.c_int32), ("variant", ctypes.c_int32)]


class LibraryMissing(ImportError):
    pass


_lib = None


def lib():
    """The loaded library. Raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m gqa_scaled_dot_amd.build` "
            "(there is no fallback implementation)")
    # torch ships its own HIP runtime with the same soname as the system one.
    # Loading torch first makes libattn.so bind to that one runtime, so device
    # pointers and streams from torch mean the same thing to the library.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(AttnParams)
    vp = ctypes.c_void_p
    L.attn_params_init.argtypes = [P]
    L.attn_params_init.restype = None
    L.attn_validate.argtypes = [P]
    L.attn_validate.restype = ctypes.c_int
    L.attn_workspace_size.argtypes = [P]
    L.attn_workspace_size.restype = ctypes.c_size_t
    L.attn_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_forward.restype = ctypes.c_int
    L.attn_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.attn_forward_noalloc.restype = ctypes.c_int
    L.attn_forward_append.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    L.attn_forward_append.restype = ctypes.c_int
    L.attn_cache_write.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int64,
                                   ctypes.c_int64, vp]
    L.attn_cache_write.restype = ctypes.c_int
    L.attn_cache_write2.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                    vp, ctypes.c_int64, ctypes.c_int64, vp]
    L.attn_cache_write2.restype = ctypes.c_int
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_plan.argtypes = [P, ctypes.POINTER(AttnPlanInfo)]
    L.attn_plan.restype = ctypes.c_int
    L.attn_set_option.argtypes = [ctypes.c_char_p, ctypes.c_int64]
    L.attn_set_option.restype = ctypes.c_int
    L.attn_timing_enable.argtypes = [ctypes.c_int]
    L.attn_timing_enable.restype = ctypes.c_int
    L.attn_timing_collect.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
    L.attn_timing_collect.restype = ctypes.c_int
    R = ctypes.POINTER(AttnRopeParams)
    L.attn_rope_params_init.argtypes = [R]
    L.attn_rope_params_init.restype = None
    L.attn_rope_table.argtypes = [R, ctypes.c_int64, ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_float)]
    L.attn_rope_table.restype = ctypes.c_int
    L.attn_rope.argtypes = [R, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
    L.attn_rope.restype = ctypes.c_int
    L.attn_rope_cache_write.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, ctypes.c_int64,
                                        ctypes.c_int64, R, vp]
    L.attn_rope_cache_write.restype = ctypes.c_int
    M = ctypes.POINTER(AttnMlaParams)
    L.attn_mla_params_init.argtypes = [M]
    L.attn_mla_params_init.restype = None
    L.attn_mla_validate.argtypes = [M]
    L.attn_mla_validate.restype = ctypes.c_int
    L.attn_mla_workspace_size.argtypes = [M]
    L.attn_mla_workspace_size.restype = ctypes.c_size_t
    L.attn_mla_plan.argtypes = [M, ctypes.POINTER(AttnPlanInfo)]
    L.attn_mla_plan.restype = ctypes.c_int
    L.attn_mla_forward.argtypes = [M, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_mla_forward.restype = ctypes.c_int
    _lib = L
    return L
