"""Host-side checks of the C-ABI library (no GPU work): it loads, exports every entry point
the header declares, and rejects invalid limits before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grw.h")
LIB = os.path.join(ROOT, "generative_recommendation_wide_amd", "libgrw.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def clib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._build_module().build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("beam_attn_decode", "beam_select", "beam_select_gumbel", "beam_select_logits", "grw_ws_create",
              "grw_ws_destroy",
              "grw_ws_bind_batch", "grw_beams_init", "grw_backtrack", "grw_ws_error",
              "grw_ws_splits", "grw_ws_pool_size", "grw_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(clib):
    for n in declared_functions():
        assert hasattr(clib, n), n


def test_status_strings(clib):
    clib.grw_status_str.restype = ctypes.c_char_p
    assert clib.grw_status_str(0) == b"ok"
    assert b"invalid" in clib.grw_status_str(1)
    assert clib.grw_status_str(99) == b"unknown status"


def test_invalid_limits_rejected_on_host(clib):
    from generative_recommendation_wide_amd._lib import GrwLimits
    clib.grw_ws_create.argtypes = [ctypes.POINTER(GrwLimits), ctypes.POINTER(ctypes.c_void_p)]
    good = dict(max_requests=1, max_total_beams=8, max_W=8, max_K=8, max_C=64, max_S=3, max_P=128,
                Hq=16, Hkv=8, D=128, q_dtype=1, kv_dtype=1, max_splits=0)
    bad_cases = [
        dict(max_requests=0), dict(max_W=9), dict(max_K=0), dict(Hq=12), dict(q_dtype=2),
        dict(kv_dtype=7), dict(max_W=9000, max_total_beams=9000), dict(max_K=5000),
        dict(max_S=65), dict(max_splits=17), dict(Hq=24, Hkv=8), dict(D=96),
        dict(max_C=1 << 30, max_W=8),
    ]
    for bad in bad_cases:
        lim = GrwLimits(**{**good, **bad})
        h = ctypes.c_void_p()
        st = clib.grw_ws_create(ctypes.byref(lim), ctypes.byref(h))
        assert st in (1, 4), bad
        assert not h.value
    assert clib.grw_ws_create(None, None) == 1


def test_null_handles_rejected(clib):
    assert clib.grw_ws_destroy(None) == 1
    assert clib.grw_ws_bind_batch(None, 1, None, None, None, None) == 1
    assert clib.beam_attn_decode(None, None, None, None, None, None, None, None, None, 0, None, None) == 1
    assert clib.beam_attn_decode_overlap(None, None, None, None, None, None, None, None, None, 0, None, None,
                                         None) == 1
    assert clib.beam_select(None, *([None] * 5), 0, 1, 1, 1, None, None, None, None, None) == 1
    f = clib.beam_select_gumbel
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 4 + \
        [ctypes.c_void_p] * 5
    assert f(None, None, None, 1.0, None, None, None, None, 0, 1, 1, 1, None, None, None, None, None) == 1
    f = clib.beam_select_logits
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 4 + \
        [ctypes.c_void_p] * 5
    assert f(None, None, None, 0.0, None, None, None, None, 0, 1, 1, 1, None, None, None, None, None) == 1
    assert clib.grw_backtrack(None, None, None, 1, None, None) == 1
    assert clib.grw_ws_pool_size(None, 0, None, None) == 1
    clib.grw_selftest_lanes.argtypes = [ctypes.c_void_p] * 3
    assert clib.grw_selftest_lanes(None, None, None) == 1


def test_ceiling_probe_library_is_separate(clib):
    """The benchmark's MFMA ceiling probe lives in its own library: it loads and exports its
    launcher, and the decode library does not carry it."""
    path = os.path.join(ROOT, "generative_recommendation_wide_amd", "libgrw_ceiling.so")
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__._build_module().build()
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "grw_ceiling_mfma")
    lib.grw_ceiling_mfma_per_round.restype = ctypes.c_int
    assert lib.grw_ceiling_mfma_per_round() == 8
    # invalid arguments are rejected on the host, before any launch
    lib.grw_ceiling_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.grw_ceiling_mfma(0, 10, None, None, None) == -1
    assert not hasattr(clib, "grw_ceiling_mfma")
