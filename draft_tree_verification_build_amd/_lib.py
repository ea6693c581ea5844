"""ctypes loader for libdtv.so and the signatures of its C entry points (include/dtv.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdtv.so")

c_int, c_i32, c_i64, c_f32, c_f64 = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
c_size, c_vp, c_char_p = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p


class DtvTree(ctypes.Structure):
    _fields_ = [
        ("n_cap", c_i32), ("words", c_i32),
        ("n_nodes", c_vp), ("parent", c_vp), ("token", c_vp), ("depth", c_vp),
        ("row", c_vp), ("score", c_vp), ("anc", c_vp), ("layers", c_vp),
    ]


PTREE = ctypes.POINTER(DtvTree)


class DtvKvCache(ctypes.Structure):
    _fields_ = [
        ("k", c_vp), ("v", c_vp), ("P", c_vp), ("P_new", c_vp),
        ("P_cap", c_i32), ("Hkv", c_i32), ("D", c_i32),
    ]


PKV = ctypes.POINTER(DtvKvCache)


class DtvBuildParams(ctypes.Structure):
    _fields_ = [
        ("mode", c_i32), ("B", c_i32), ("K", c_i32), ("alpha", c_f64),
        ("n", c_i32), ("delta", c_f64), ("max_layers", c_i32),
    ]


PBP = ctypes.POINTER(DtvBuildParams)

# name -> (restype, argtypes)
SIGNATURES = {
    "dtv_status_str": (c_char_p, [c_int]),
    "dtv_last_error": (c_char_p, []),
    "dtv_ws_status": (c_int, [c_vp, c_vp]),
    "dtv_row_stats_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_int]),
    "dtv_row_stats": (c_int, [c_vp, c_int, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                              c_vp, c_size, c_vp]),
    "dtv_tree_build_given_ws_bytes": (c_size, [c_i32]),
    "dtv_tree_build_given": (c_int, [PTREE, c_i32, c_vp, c_size, c_vp]),
    "dtv_tree_build_talon_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_build_talon": (c_int, [PTREE, c_i32, c_vp, c_int, c_i32, c_i32, c_i32, c_i32, c_f64,
                                     c_vp, c_size, c_vp]),
    "dtv_tree_build_spine_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_build_spine": (c_int, [PTREE, c_i32, c_vp, c_i32, c_vp, c_i32, c_vp, c_int, c_i32, c_i32,
                                     c_vp, c_size, c_vp]),
    "dtv_tree_build_opt_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_build_opt": (c_int, [PTREE, c_i32, c_vp, c_int, c_i32, c_i32, c_i32, c_f64, c_i32,
                                   c_vp, c_size, c_vp]),
    "dtv_tree_build_layered_ws_bytes": (c_size, [PBP, c_i32, c_i32, c_int]),
    "dtv_tree_build_begin": (c_int, [PTREE, c_i32, PBP, c_vp, c_int, c_i32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "dtv_tree_build_step": (c_int, [PTREE, c_i32, PBP, c_i32, c_vp, c_i32, c_int, c_i32, c_vp, c_vp, c_vp, c_size,
                                    c_vp]),
    "dtv_tree_attn_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_attn": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, PTREE, c_i32, c_i32, c_i32,
                              c_i32, c_int, c_f32, c_vp, c_vp, c_size, c_vp]),
    "dtv_tree_attn_noalloc": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, PTREE, c_i32, c_i32, c_i32,
                                      c_i32, c_int, c_f32, c_vp, c_vp]),
    "dtv_tree_verify_greedy_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_verify_greedy": (c_int, [PTREE, c_i32, c_vp, c_int, c_i32, c_i32, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, c_size, c_vp]),
    "dtv_tree_verify_greedy_compact": (c_int, [PTREE, c_i32, c_vp, c_int, c_i32, c_i32, c_vp, c_vp, c_vp,
                                               c_vp, PKV, c_vp, c_size, c_vp]),
    "dtv_tree_verify_sample_compact": (c_int, [PTREE, c_i32, c_vp, c_vp, c_int, c_i32, c_i32, c_vp, c_vp,
                                               c_vp, c_vp, c_vp, PKV, c_vp, c_size, c_vp]),
    "dtv_tree_verify_sample_ws_bytes": (c_size, [c_i32, c_i32, c_i32, c_int]),
    "dtv_tree_verify_sample": (c_int, [PTREE, c_i32, c_vp, c_vp, c_int, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, c_size, c_vp]),
    "dtv_tree_verify_sample_plan": (c_int, [c_i32, c_i32, c_i32, c_int, c_i32, c_i32, c_vp]),
    "dtv_kv_compact": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                               c_i32, c_int, c_vp]),
    "dtv_kernel_timing": (c_int, [c_int, c_int]),
    "dtv_kernel_times": (c_int, [c_i32, c_vp, c_i32, c_vp, c_vp]),
    "dtv_bookkeeping": (c_int, [c_vp, c_i32, c_i64, c_f64, c_vp]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdtv.so once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m draft_tree_verification_build_amd.build_lib` "
            "(the draft-tree step has no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
