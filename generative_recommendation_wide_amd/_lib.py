"""ctypes binding of libgrw.so (argument marshalling only).

The functions here have the names of the C ABI in include/grw.h and pass raw device
pointers (torch tensors' data_ptr()) and the current HIP stream.  No arithmetic of the
decode step happens in Python.  Loading fails loudly when the library was not built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgrw.so")

GRW_OK, GRW_EINVAL, GRW_ENOMEM, GRW_EDEVICE, GRW_EUNSUPPORTED, GRW_ESTATE = range(6)
GRW_F32, GRW_BF16, GRW_FP8_E4M3 = 0, 1, 2
FLAG_NAN_LOGPROB, FLAG_POS_LOGPROB, FLAG_BAD_NODE, FLAG_BAD_PARENT, FLAG_CHILD_MISSING = 1, 2, 4, 8, 16
FLAG_POOL_CORRUPT = 32
FLAG_BAD_NOISE = 64
STAGE_SHARED, STAGE_UNSHARED, STAGE_MERGE = 1, 2, 4
SELFTEST_WORDS = 3584

EXPORTED = ["grw_ws_create", "grw_ws_destroy", "grw_ws_bind_batch", "grw_beams_init",
            "beam_attn_decode", "beam_attn_decode_stages", "beam_attn_decode_overlap", "beam_select", "beam_select_gumbel",
            "beam_select_logits", "beam_select_ex", "grw_trie_dense_build", "grw_plan_batches", "grw_backtrack",
            "grw_ws_error",
            "grw_ws_splits", "grw_ws_pool_size", "grw_ws_set_wait_limit", "grw_status_str",
            "beam_select_noalloc", "grw_selftest_lanes"]


class GrwLimits(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_requests", "max_total_beams", "max_W", "max_K", "max_C", "max_S", "max_P",
        "Hq", "Hkv", "D", "q_dtype", "kv_dtype", "max_splits")]


class GrwTrie(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("code", ctypes.c_void_p), ("n_internal", ctypes.c_int32),
                ("dense_slot", ctypes.c_void_p), ("dense_mask", ctypes.c_void_p)]


class GrwSelectOpts(ctypes.Structure):
    _fields_ = [("noise", ctypes.c_void_p), ("temperature", ctypes.c_float), ("raw_logits", ctypes.c_int32),
                ("first_step_fanout", ctypes.c_int32)]


class GrwError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgrw.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python generative_recommendation_wide_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i32, i32p, fp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    sig = {
        "grw_ws_create": [ctypes.POINTER(GrwLimits), ctypes.POINTER(vp)],
        "grw_ws_destroy": [vp],
        "grw_ws_bind_batch": [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32), vp],
        "grw_beams_init": [vp, fp, i32p, vp],
        "beam_attn_decode": [vp, vp, vp, vp, fp, fp, vp, vp, i32p, i32, fp, vp],
        "beam_attn_decode_stages": [vp, vp, vp, vp, fp, fp, vp, vp, i32p, i32, fp, i32, vp],
        "beam_attn_decode_overlap": [vp, vp, vp, vp, fp, fp, vp, vp, i32p, i32, fp, vp, vp],
        "beam_select": [vp, fp, fp, i32p, i32p, i32p, i32, i32, i32, i32, i32p, i32p, fp, i32p, vp],
        "beam_select_gumbel": [vp, fp, fp, ctypes.c_float, fp, i32p, i32p, i32p, i32, i32, i32, i32, i32p, i32p, fp,
                               i32p, vp],
        "beam_select_logits": [vp, fp, fp, ctypes.c_float, fp, i32p, i32p, i32p, i32, i32, i32, i32, i32p, i32p, fp,
                               i32p, vp],
        "beam_select_ex": [vp, fp, fp, i32p, ctypes.POINTER(GrwTrie), ctypes.POINTER(GrwSelectOpts), i32, i32, i32,
                           i32p, i32p, fp, i32p, vp],
        "grw_trie_dense_build": [vp, vp, i32, i32, i32, vp, vp, ctypes.POINTER(i32)],
        "grw_plan_batches": [i32, vp, i32, i32, vp, ctypes.POINTER(i32)],
        "grw_backtrack": [vp, i32p, i32p, i32, i32p, vp],
        "grw_ws_error": [vp, vp, ctypes.POINTER(i32)],
        "grw_ws_splits": [vp, i32, ctypes.POINTER(i32)],
        "grw_ws_pool_size": [vp, i32, vp, ctypes.POINTER(ctypes.c_int64)],
        "grw_ws_set_wait_limit": [vp, i32],
        "beam_select_noalloc": [fp, fp, i32p, i32p, i32p, i32, i32, i32, i32, i32p, i32p, fp, i32p, i32p, vp],
        "grw_selftest_lanes": [vp, vp, ctypes.POINTER(i32)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.grw_status_str.argtypes = [ctypes.c_int]
    lib.grw_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != GRW_OK:
        raise GrwError(fn, status, load().grw_status_str(status).decode())
