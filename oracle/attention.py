"""Oracle beam attention: naive float64 softmax attention over the concatenated KV.

Source: xLLM generative-recommendation design doc, §4.2.1 (prompt KV from prefill is
stored once and shared by all beams; decode-token KV is kept per beam at token
granularity) and §4.2.2 (the shared stage, the unshared stage and the online-softmax
merge split one attention; this oracle computes that one attention without splitting).

Readings where the pages are silent:
* softmax scale 1/sqrt(D);
* grouped heads: query head h reads kv head h // (Hq / Hkv);
* a beam at depth d attends to all P prompt tokens and to its own d + 1 decode tokens
  (its ancestors at depths 0..d-1 and its own token at depth d), never to siblings;
* the ancestry is reached through parent pointers: j_d = b, j_{e-1} = parent[e][j_e];
* a slot whose parent pointer at depth d is negative is dead and its output is zero;
* fp8 KV values are code * scale, with one scale per kv head for K and one for V.
"""
from __future__ import annotations

import numpy as np

from .numformats import decode_stored


def attend_concat(q: np.ndarray, kcat: np.ndarray, vcat: np.ndarray) -> np.ndarray:
    """softmax(q kcat^T / sqrt(D)) vcat for one head, in float64.

    q [D], kcat [T, D], vcat [T, D]  ->  [D]
    """
    D = q.shape[-1]
    s = (kcat @ q) / np.sqrt(np.float64(D))
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ vcat


def ancestry(parents: np.ndarray, step: int, b: int):
    """Slots j_0..j_d of beam b at depth d, following parent pointers backwards."""
    js = [0] * (step + 1)
    j = b
    js[step] = j
    for e in range(step, 0, -1):
        j = int(parents[e][j])
        assert j >= 0, "a live beam has a dead ancestor"
        js[e - 1] = j
    return js


def oracle_attention(q, k_s, v_s, k_u, v_u, parents, step, *, q_dtype, kv_dtype,
                     k_scale=None, v_scale=None, beams=None, threads=1):
    """Attention output of one request at one layer and decode depth ``step``.

    q        [W][Hq][D]          stored (f32 / bf16 bits) — this request's slots
    k_s, v_s [Hkv][P][D]         stored prompt KV (f32 / bf16 bits / e4m3fn bits)
    k_u, v_u [S][W][Hkv][D]      stored decode-token KV of this request's slots
    parents  [S][W] int          request-local parent slot per depth (negative = dead)
    k_scale, v_scale [Hkv]       fp8 scales (kv_dtype == "fp8")
    beams    iterable of slots to evaluate (default: all)
    threads  beams evaluated at once (a thread pool; each beam's arithmetic is the same)

    Returns float64 [len(beams)][Hq][D].
    """
    W, Hq, D = q.shape[0], q.shape[1], q.shape[2]
    Hkv = k_s.shape[0]
    g = Hq // Hkv
    assert g * Hkv == Hq
    ksc = None if k_scale is None else np.asarray(k_scale, np.float64)
    vsc = None if v_scale is None else np.asarray(v_scale, np.float64)
    Ks = decode_stored(k_s, kv_dtype, None if ksc is None else ksc[:, None, None])
    Vs = decode_stored(v_s, kv_dtype, None if vsc is None else vsc[:, None, None])
    beams = list(range(W)) if beams is None else [int(b) for b in beams]
    out = np.zeros((len(beams), Hq, D), np.float64)

    def one(i):
        b = beams[i]
        if parents[step][b] < 0:
            return                                    # dead slot: zero output
        js = ancestry(parents, step, b)
        ku = np.stack([k_u[e][j] for e, j in enumerate(js)], axis=1)   # [Hkv][d+1][D]
        vu = np.stack([v_u[e][j] for e, j in enumerate(js)], axis=1)
        Ku = decode_stored(ku, kv_dtype, None if ksc is None else ksc[:, None, None])
        Vu = decode_stored(vu, kv_dtype, None if vsc is None else vsc[:, None, None])
        Kcat = np.concatenate([Ks, Ku], axis=1)       # [Hkv][P+d+1][D]
        Vcat = np.concatenate([Vs, Vu], axis=1)
        qb = decode_stored(q[b], q_dtype)             # [Hq][D]
        for h in range(Hq):
            out[i, h] = attend_concat(qb[h], Kcat[h // g], Vcat[h // g])

    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(len(beams))))
    else:
        for i in range(len(beams)):
            one(i)
    return out
