"""Wide-beam decode step for generative recommendation on AMD Instinct MI355X (gfx950).

Python binding of the C-ABI library libgrw.so (include/grw.h).  The functions keep the C
names and only marshal arguments: torch tensors are passed as device pointers and the
current torch stream as the HIP stream.  Every step of the path runs in the library's
HIP kernels; if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (STAGE_MERGE, STAGE_SHARED, STAGE_UNSHARED,  # noqa: F401
                   FLAG_BAD_NODE, FLAG_BAD_PARENT, FLAG_CHILD_MISSING, FLAG_NAN_LOGPROB,  # noqa: F401
                   FLAG_BAD_NOISE, FLAG_POS_LOGPROB, GRW_BF16, GRW_F32, GRW_FP8_E4M3, GrwError,
                   GrwLimits)

_L = _lib.load()

DTYPES = {"f32": GRW_F32, "bf16": GRW_BF16, "fp8": GRW_FP8_E4M3}


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t, dtypes=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


_F32 = (torch.float32,)
_I32 = (torch.int32,)
_ANY_KV = (torch.float32, torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


class Workspace:
    """A grw_ws handle: the library's preallocated device state for one batch shape."""

    def __init__(self, *, max_requests, max_total_beams, max_W, max_K, max_C, max_S, max_P,
                 Hq, Hkv, D, q_dtype="bf16", kv_dtype="bf16", max_splits=0):
        lim = GrwLimits(max_requests, max_total_beams, max_W, max_K, max_C, max_S, max_P,
                        Hq, Hkv, D, DTYPES[q_dtype], DTYPES[kv_dtype], max_splits)
        h = ctypes.c_void_p()
        _lib.check("grw_ws_create", _L.grw_ws_create(ctypes.byref(lim), ctypes.byref(h)))
        self.handle = h
        self.limits = lim
        self.sumW = 0
        self.W = self.K = self.P = None

    def bind_batch(self, W, K, P, stream=None):
        n = len(W)
        arr = ctypes.c_int32 * n
        _lib.check("grw_ws_bind_batch", _L.grw_ws_bind_batch(
            self.handle, n, arr(*map(int, W)), arr(*map(int, K)), arr(*map(int, P)), _stream(stream)))
        self.W, self.K, self.P = [list(map(int, x)) for x in (W, K, P)]
        self.sumW = sum(self.W)

    def beams_init(self, beam_scores, beam_node, stream=None):
        _lib.check("grw_beams_init", _L.grw_beams_init(
            self.handle, _ptr(beam_scores, _F32, "beam_scores"), _ptr(beam_node, _I32, "beam_node"),
            _stream(stream)))

    def splits(self, r: int) -> int:
        v = ctypes.c_int32()
        _lib.check("grw_ws_splits", _L.grw_ws_splits(self.handle, r, ctypes.byref(v)))
        return v.value

    def pool_size(self, r: int, stream=None) -> int:
        """Candidate-pool entries of request r kept by the last beam_select (synchronises)."""
        v = ctypes.c_int64()
        _lib.check("grw_ws_pool_size", _L.grw_ws_pool_size(self.handle, r, _stream(stream), ctypes.byref(v)))
        return v.value

    def set_wait_limit(self, polls: int) -> None:
        """Polls a beam workgroup of the fused selection makes for its bound before it goes on
        without one (same result, slower); 0 forces that fallback."""
        _lib.check("grw_ws_set_wait_limit", _L.grw_ws_set_wait_limit(self.handle, int(polls)))

    def error_flags(self, stream=None) -> int:
        v = ctypes.c_int32()
        _lib.check("grw_ws_error", _L.grw_ws_error(self.handle, _stream(stream), ctypes.byref(v)))
        return v.value

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _L.grw_ws_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def beam_attn_decode(ws: Workspace, q, k_shared, v_shared, k_scale, v_scale, k_unshared, v_unshared,
                     parent_idx, step: int, out, stream=None):
    """Beam attention of one layer at decode depth ``step`` (see include/grw.h)."""
    _lib.check("beam_attn_decode", _L.beam_attn_decode(
        ws.handle, _ptr(q, (torch.float32, torch.bfloat16), "q"), _ptr(k_shared, _ANY_KV, "k_shared"),
        _ptr(v_shared, _ANY_KV, "v_shared"), _ptr(k_scale, _F32, "k_scale"), _ptr(v_scale, _F32, "v_scale"),
        _ptr(k_unshared, _ANY_KV, "k_unshared"), _ptr(v_unshared, _ANY_KV, "v_unshared"),
        _ptr(parent_idx, _I32, "parent_idx"), int(step), _ptr(out, _F32, "out"), _stream(stream)))


def beam_attn_decode_stages(ws: Workspace, q, k_shared, v_shared, k_scale, v_scale, k_unshared,
                            v_unshared, parent_idx, step: int, out, stages: int, stream=None):
    """beam_attn_decode restricted to the stages in the bit mask (1 shared, 2 unshared, 4 merge)."""
    _lib.check("beam_attn_decode_stages", _L.beam_attn_decode_stages(
        ws.handle, _ptr(q, (torch.float32, torch.bfloat16), "q"), _ptr(k_shared, _ANY_KV, "k_shared"),
        _ptr(v_shared, _ANY_KV, "v_shared"), _ptr(k_scale, _F32, "k_scale"), _ptr(v_scale, _F32, "v_scale"),
        _ptr(k_unshared, _ANY_KV, "k_unshared"), _ptr(v_unshared, _ANY_KV, "v_unshared"),
        _ptr(parent_idx, _I32, "parent_idx"), int(step), _ptr(out, _F32, "out"), int(stages),
        _stream(stream)))


def beam_attn_decode_overlap(ws: Workspace, q, k_shared, v_shared, k_scale, v_scale, k_unshared,
                             v_unshared, parent_idx, step: int, out, side_stream, stream=None):
    """beam_attn_decode with the unshared stage on side_stream (a torch.cuda.Stream other
    than ``stream``), overlapping the shared stage; the merge runs on ``stream``."""
    if side_stream is None:
        raise ValueError("beam_attn_decode_overlap needs a side stream")
    _lib.check("beam_attn_decode_overlap", _L.beam_attn_decode_overlap(
        ws.handle, _ptr(q, (torch.float32, torch.bfloat16), "q"), _ptr(k_shared, _ANY_KV, "k_shared"),
        _ptr(v_shared, _ANY_KV, "v_shared"), _ptr(k_scale, _F32, "k_scale"), _ptr(v_scale, _F32, "v_scale"),
        _ptr(k_unshared, _ANY_KV, "k_unshared"), _ptr(v_unshared, _ANY_KV, "v_unshared"),
        _ptr(parent_idx, _I32, "parent_idx"), int(step), _ptr(out, _F32, "out"), _stream(stream),
        side_stream.cuda_stream))


def beam_select(ws: Workspace, logprobs, beam_scores, beam_node, trie_row_ptr, trie_code,
                trie_n_internal: int, W: int, K: int, C: int, out_token, out_parent, out_score,
                out_node, stream=None):
    """One trie-constrained selection step of every bound request (see include/grw.h)."""
    _lib.check("beam_select", _L.beam_select(
        ws.handle, _ptr(logprobs, _F32, "logprobs"), _ptr(beam_scores, _F32, "beam_scores"),
        _ptr(beam_node, _I32, "beam_node"), _ptr(trie_row_ptr, _I32, "trie_row_ptr"),
        _ptr(trie_code, _I32, "trie_code"), int(trie_n_internal), int(W), int(K), int(C),
        _ptr(out_token, _I32, "out_token"), _ptr(out_parent, _I32, "out_parent"),
        _ptr(out_score, _F32, "out_score"), _ptr(out_node, _I32, "out_node"), _stream(stream)))


def beam_select_noalloc(logprobs, beam_scores, beam_node, trie_row_ptr, trie_code, trie_n_internal: int, W: int,
                        K: int, C: int, out_token, out_parent, out_score, out_node, device_flags=None, stream=None):
    """beam_select of one request without a workspace: its scratch is the library's static
    device array, so the call allocates nothing (see include/grw.h)."""
    _lib.check("beam_select_noalloc", _L.beam_select_noalloc(
        _ptr(logprobs, _F32, "logprobs"), _ptr(beam_scores, _F32, "beam_scores"),
        _ptr(beam_node, _I32, "beam_node"), _ptr(trie_row_ptr, _I32, "trie_row_ptr"),
        _ptr(trie_code, _I32, "trie_code"), int(trie_n_internal), int(W), int(K), int(C),
        _ptr(out_token, _I32, "out_token"), _ptr(out_parent, _I32, "out_parent"),
        _ptr(out_score, _F32, "out_score"), _ptr(out_node, _I32, "out_node"),
        _ptr(device_flags, _I32, "device_flags"), _stream(stream)))


def beam_select_gumbel(ws: Workspace, logprobs, noise, temperature: float, beam_scores, beam_node,
                       trie_row_ptr, trie_code, trie_n_internal: int, W: int, K: int, C: int,
                       out_token, out_parent, out_score, out_node, stream=None):
    """The sampled selection step: Gumbel top-k at temperature >= 0 (see include/grw.h)."""
    _lib.check("beam_select_gumbel", _L.beam_select_gumbel(
        ws.handle, _ptr(logprobs, _F32, "logprobs"), _ptr(noise, _F32, "noise"), float(temperature),
        _ptr(beam_scores, _F32, "beam_scores"), _ptr(beam_node, _I32, "beam_node"),
        _ptr(trie_row_ptr, _I32, "trie_row_ptr"), _ptr(trie_code, _I32, "trie_code"), int(trie_n_internal),
        int(W), int(K), int(C), _ptr(out_token, _I32, "out_token"), _ptr(out_parent, _I32, "out_parent"),
        _ptr(out_score, _F32, "out_score"), _ptr(out_node, _I32, "out_node"), _stream(stream)))


def beam_select_logits(ws: Workspace, logits, noise, temperature: float, beam_scores, beam_node,
                       trie_row_ptr, trie_code, trie_n_internal: int, W: int, K: int, C: int,
                       out_token, out_parent, out_score, out_node, stream=None):
    """The selection step from raw logits, log-softmax fused in; noise None for the
    deterministic selection (see include/grw.h)."""
    _lib.check("beam_select_logits", _L.beam_select_logits(
        ws.handle, _ptr(logits, _F32, "logits"), _ptr(noise, _F32, "noise"), float(temperature),
        _ptr(beam_scores, _F32, "beam_scores"), _ptr(beam_node, _I32, "beam_node"),
        _ptr(trie_row_ptr, _I32, "trie_row_ptr"), _ptr(trie_code, _I32, "trie_code"), int(trie_n_internal),
        int(W), int(K), int(C), _ptr(out_token, _I32, "out_token"), _ptr(out_parent, _I32, "out_parent"),
        _ptr(out_score, _F32, "out_score"), _ptr(out_node, _I32, "out_node"), _stream(stream)))


def beam_select_ex(ws: Workspace, input, beam_scores, beam_node, trie, W: int, K: int, C: int, out_token,
                   out_parent, out_score, out_node, noise=None, temperature: float = 0.0, raw_logits: bool = False,
                   stream=None, fanout: bool = False):
    """The selection step with every option (see include/grw.h).  trie: None, or a tuple
    (row_ptr, code, n_internal) or (row_ptr, code, n_internal, dense_slot, dense_mask) of
    device tensors (n_internal an int); fanout: the first-step fan-out."""
    t = None
    if trie is not None:
        row_ptr, code, n_int = trie[:3]
        dslot, dmask = (trie[3], trie[4]) if len(trie) > 3 else (None, None)
        t = _lib.GrwTrie(_ptr(row_ptr, _I32, "row_ptr"), _ptr(code, _I32, "code"), int(n_int),
                         _ptr(dslot, _I32, "dense_slot"), _ptr(dmask, (torch.int32, torch.uint32), "dense_mask"))
    o = _lib.GrwSelectOpts(_ptr(noise, _F32, "noise"), float(temperature), int(bool(raw_logits)), int(bool(fanout)))
    _lib.check("beam_select_ex", _L.beam_select_ex(
        ws.handle, _ptr(input, _F32, "input"), _ptr(beam_scores, _F32, "beam_scores"),
        _ptr(beam_node, _I32, "beam_node"), ctypes.byref(t) if t is not None else None, ctypes.byref(o),
        int(W), int(K), int(C), _ptr(out_token, _I32, "out_token"), _ptr(out_parent, _I32, "out_parent"),
        _ptr(out_score, _F32, "out_score"), _ptr(out_node, _I32, "out_node"), _stream(stream)))


def trie_dense_build(row_ptr, code, n_internal: int, C: int, min_fanout: int):
    """Host-side dense child masks (see grw_trie_dense_build): numpy int32 CSR arrays in,
    numpy (dense_slot int32 [n_internal], dense_mask uint32 [n_dense][(C + 31) // 32]) out."""
    import numpy as np
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    code = np.ascontiguousarray(code, dtype=np.int32)
    slot = np.empty(int(n_internal), np.int32)
    n = ctypes.c_int32(0)
    args = (row_ptr.ctypes.data, code.ctypes.data, int(n_internal), int(C), int(min_fanout), slot.ctypes.data)
    _lib.check("grw_trie_dense_build", _L.grw_trie_dense_build(*args, None, ctypes.byref(n)))
    masks = np.empty((n.value, (int(C) + 31) // 32), np.uint32)
    _lib.check("grw_trie_dense_build", _L.grw_trie_dense_build(*args, masks.ctypes.data if n.value else None,
                                                               ctypes.byref(n)))
    return slot, masks


def plan_batches(W, slot_budget: int, max_requests: int):
    """Host-side slot-budget batching (see grw_plan_batches): beam widths in queue order ->
    (batch_of int32 [n], n_batches), first fit in queue order."""
    import numpy as np
    W = np.ascontiguousarray(W, dtype=np.int32)
    batch_of = np.empty(W.size, np.int32)
    nb = ctypes.c_int32(0)
    _lib.check("grw_plan_batches", _L.grw_plan_batches(
        int(W.size), W.ctypes.data if W.size else None, int(slot_budget), int(max_requests),
        batch_of.ctypes.data if W.size else None, ctypes.byref(nb)))
    return batch_of, nb.value


def grw_backtrack(ws: Workspace, tokens, parents, S: int, sid_out, stream=None):
    """Semantic-ID tuples [sumW][S] of the final beams (see include/grw.h)."""
    _lib.check("grw_backtrack", _L.grw_backtrack(
        ws.handle, _ptr(tokens, _I32, "tokens"), _ptr(parents, _I32, "parents"), int(S),
        _ptr(sid_out, _I32, "sid_out"), _stream(stream)))


def selftest_lanes(device=None, stream=None) -> int:
    """(check, thread) pairs where the device's wave primitives disagree with the shuffle
    forms they replace; 0 = pass (see include/grw.h).  Synchronises the stream."""
    buf = torch.empty(_lib.SELFTEST_WORDS, dtype=torch.int32,
                      device=device if device is not None else torch.device("cuda", torch.cuda.current_device()))
    v = ctypes.c_int32()
    _lib.check("grw_selftest_lanes", _L.grw_selftest_lanes(buf.data_ptr(), _stream(stream), ctypes.byref(v)))
    return v.value


from .layout import pack_shared_kv, stored_tensor  # noqa: E402,F401
from .loop import DecodeLoop  # noqa: E402,F401
