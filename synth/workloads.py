"""Seeded synthetic workloads shaped like the wide-beam generative-recommendation decode step.

The pages measure on real models and production traffic (OneRec-1.7B on RecIF-Bench and
SoHuRec traffic in the FlashRec announcement; Qwen3-0.6B at beam width 5000 in the SGLang
beam-search PR).  None of that data is available, so every input here is synthetic, drawn
with the shapes and value distributions of the five workloads below.

Random streams are random-access: every tensor is drawn from its own
``PCG64(SeedSequence([seed, workload_index, stream, *indices]))`` so that one layer or one
step can be generated without generating the others.

Nothing in this module computes attention or selects beams.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import numpy as np

# stream ids (fixed order, part of the recipe)
_S_CATALOG, _S_SHAPES, _S_Q, _S_KS, _S_VS, _S_KU, _S_VU, _S_LOGITS, _S_PARENTS, _S_GUMBEL = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_requests: int
    W: Optional[int]          # beam width (None: drawn per request)
    K: Optional[int]          # top_k (None: equal to the request's beam width)
    P: Optional[int]          # prompt length (None: drawn per request)
    Hq: int
    Hkv: int
    D: int
    S: int                    # decode steps == trie levels
    layers: int
    C: int                    # codes per SID level, or the vocabulary when unconstrained
    q_dtype: str              # "f32" | "bf16"
    kv_dtype: str             # "f32" | "bf16" | "fp8"
    logit_sigma: float
    catalog: Optional[tuple]  # ("uniform", N) | ("zipf", N, s) | None (unconstrained)


WORKLOADS = {
    # tiny fp32 reference case
    "tiny": Workload("tiny", 0, 1, 4, 4, 256, 4, 2, 64, 3, 1, 256, "f32", "f32", 2.0,
                     ("uniform", 1000)),
    # Qwen3-0.6B-shaped single layer, bf16
    "qwen06b": Workload("qwen06b", 1, 8, 50, 50, 2048, 16, 8, 128, 3, 1, 8192, "bf16", "bf16",
                        3.0, ("uniform", 1_000_000)),
    # wide-beam pool: W = K = 512, 4 requests, 28 layers, Zipf(1.1) catalog
    "wide512": Workload("wide512", 2, 4, 512, 512, 4096, 16, 8, 128, 3, 28, 8192, "bf16",
                        "bf16", 3.0, ("zipf", 4_000_000, 1.1)),
    # pool-saturating variant of wide512: unconstrained 8192-code levels
    "wide512u": Workload("wide512u", 5, 4, 512, 512, 4096, 16, 8, 128, 3, 28, 8192, "bf16",
                         "bf16", 3.0, None),
    # ultra-wide: W = 5000, K = 64, 16 steps over an unconstrained 151936-token vocabulary
    "ultra5000": Workload("ultra5000", 3, 1, 5000, 64, 1024, 16, 8, 128, 16, 28, 151936,
                          "bf16", "bf16", 4.0, None),
    # mixed ragged batch, fp8_e4m3 KV with per-head fp32 scales
    "mixed_fp8": Workload("mixed_fp8", 4, 101, None, None, None, 16, 8, 128, 4, 1, 8192,
                          "bf16", "fp8", 3.0, ("uniform", 2_000_000)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int, wl: Workload, stream: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.index, stream, *idx])))


# ----------------------------------------------------------------------------------------
# request shapes
# ----------------------------------------------------------------------------------------
def request_shapes(wl: Workload, seed: int = 0):
    """Per-request (W, K, P) as int32 arrays.

    mixed_fp8: 100 requests with W ~ U{2..100} plus one request of width 1000 (last),
    P ~ U{512..8192}, K = W.
    """
    R = wl.n_requests
    if wl.W is not None:
        W = np.full(R, wl.W, np.int32)
        K = np.full(R, wl.K, np.int32)
        P = np.full(R, wl.P, np.int32)
        return W, K, P
    g = _rng(seed, wl, _S_SHAPES)
    W = np.concatenate([g.integers(2, 101, size=R - 1), [1000]]).astype(np.int32)
    P = g.integers(512, 8193, size=R).astype(np.int32)
    K = W.copy()
    return W, K, P


# ----------------------------------------------------------------------------------------
# catalog of semantic-ID items and its prefix trie
# ----------------------------------------------------------------------------------------
def pack_prefix(codes: np.ndarray, C: int) -> np.ndarray:
    """Pack the rows of an integer array [..., l] into int64 (base-C digits, level 0 first)."""
    codes = np.asarray(codes, dtype=np.int64)
    out = np.zeros(codes.shape[:-1], dtype=np.int64)
    for i in range(codes.shape[-1]):
        out = out * C + codes[..., i]
    return out


def _unpack(packed: np.ndarray, C: int, L: int) -> np.ndarray:
    out = np.empty(packed.shape + (L,), dtype=np.int32)
    x = packed.copy()
    for i in range(L - 1, -1, -1):
        out[..., i] = x % C
        x //= C
    return out


def _first_distinct(draws: np.ndarray, n: int):
    """The first n distinct values of ``draws`` in draw order (or all distinct if fewer)."""
    uniq, first = np.unique(draws, return_index=True)
    order = np.sort(first)[:n]
    return draws[order]


@functools.lru_cache(maxsize=4)
def catalog_items(wl: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """Distinct items as an int32 array [N, S] of per-level codes, or None if unconstrained.

    uniform: N distinct S-tuples drawn uniformly without replacement from C^S.
    zipf:    each level's code drawn i.i.d. from a truncated Zipf(s) over ranks 1..C, mapped
             through a seeded per-level permutation of the codes; batches are drawn until N
             distinct tuples exist; the first N distinct in draw order are kept.
    """
    if wl.catalog is None:
        return None
    g = _rng(seed, wl, _S_CATALOG)
    kind, N = wl.catalog[0], wl.catalog[1]
    C, L = wl.C, wl.S
    assert C ** L < 2 ** 62
    if kind == "uniform":
        space = C ** L
        assert N <= space
        acc = np.empty(0, np.int64)
        while True:
            extra = max(1024, int((N - acc.size) * 1.1))
            acc = np.concatenate([acc, g.integers(0, space, size=extra, dtype=np.int64)])
            _, first = np.unique(acc, return_index=True)
            if first.size >= N:
                break
        packed = _first_distinct(acc, N)
        return _unpack(packed, C, L)
    if kind == "zipf":
        s = wl.catalog[2]
        ranks = np.arange(1, C + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** (-s))
        cdf /= cdf[-1]
        perms = [g.permutation(C) for _ in range(L)]
        acc = np.empty(0, np.int64)
        while True:
            extra = max(1024, int((N - np.unique(acc).size) * 1.3) + 1024)
            codes = np.empty((extra, L), np.int64)
            for lvl in range(L):
                r = np.minimum(np.searchsorted(cdf, g.random(extra), side="right"), C - 1)
                codes[:, lvl] = perms[lvl][r]
            acc = np.concatenate([acc, pack_prefix(codes, C)])
            if np.unique(acc).size >= N:
                break
        packed = _first_distinct(acc, N)
        return _unpack(packed, C, L)
    raise ValueError(kind)


def build_trie_csr(items: np.ndarray, C: int):
    """CSR layout of the prefix trie of ``items`` [N, L].

    Nodes are numbered breadth-first with the root as 0; within a depth, nodes follow the
    lexicographic order of their prefixes, which is the breadth-first order when children
    are visited in ascending code order.  Internal nodes (depth < L) own rows; row n holds
    the codes of n's children in ascending order in ``code[row_ptr[n]:row_ptr[n+1]]``, and
    the child reached through edge e is node e + 1.

    Returns a dict with row_ptr (int32 [n_internal+1]), code (int32 [n_edges]),
    n_internal, n_nodes, and node_depth / node_prefix (int64 packed prefix per node) used
    only to translate node ids back to prefixes in tests.
    """
    items = np.asarray(items, dtype=np.int64)
    N, L = items.shape
    level_prefixes = [np.zeros(1, np.int64)]           # depth 0: the root (empty prefix)
    for d in range(1, L + 1):
        level_prefixes.append(np.unique(pack_prefix(items[:, :d], C)))
    counts = [p.size for p in level_prefixes]
    n_nodes = int(sum(counts))
    n_internal = int(sum(counts[:L]))
    # children per internal node: a depth-(d+1) prefix's parent is prefix // C
    child_count = np.zeros(n_internal, np.int64)
    code_chunks = []
    base = 0
    for d in range(L):
        parents = level_prefixes[d]
        kids = level_prefixes[d + 1]
        parent_of_kid = np.searchsorted(parents, kids // C)   # kids are sorted, so are parents
        child_count[base:base + parents.size] = np.bincount(parent_of_kid, minlength=parents.size)
        code_chunks.append((kids % C).astype(np.int32))
        base += parents.size
    row_ptr = np.zeros(n_internal + 1, np.int64)
    np.cumsum(child_count, out=row_ptr[1:])
    code = np.concatenate(code_chunks) if code_chunks else np.zeros(0, np.int32)
    assert row_ptr[-1] == code.size == n_nodes - 1
    assert row_ptr[-1] < 2 ** 31
    node_depth = np.concatenate([np.full(c, d, np.int32) for d, c in enumerate(counts)])
    node_prefix = np.concatenate(level_prefixes)
    return dict(row_ptr=row_ptr.astype(np.int32), code=code.astype(np.int32),
                n_internal=n_internal, n_nodes=n_nodes, node_depth=node_depth,
                node_prefix=node_prefix)


# ----------------------------------------------------------------------------------------
# number formats of stored tensors (input preparation, not method arithmetic)
# ----------------------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """bfloat16 storage bits (uint16) of float32 values, rounded to nearest even (torch cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def e4m3fn_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """OCP fp8 E4M3 ("fn": max 448, no inf) storage bits (uint8); saturating, nearest even.

    Values are clipped to +-448 first, then converted by torch's float8_e4m3fn cast, which
    rounds to nearest even.
    """
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _store(x: np.ndarray, dtype: str, scale=None):
    """Convert a float32 array to the stored representation of ``dtype``."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "fp8":
        return e4m3fn_bits_from_f32(x / scale)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------
# attention inputs
# ----------------------------------------------------------------------------------------
def attention_layer(wl: Workload, layer: int, seed: int = 0, shapes=None, requests=None):
    """Synthetic attention inputs of one layer, in storage format.

    Values are N(0, 1).  Returns a dict:
      q       [S][sumW][Hq][D]    f32 array, or uint16 bf16 bits
      k_s,v_s list over requests of [Hkv][P_r][D]   (f32 / uint16 bf16 / uint8 e4m3fn bits)
      k_u,v_u [S][sumW][Hkv][D]   (same storage dtype as k_s)
      k_scale, v_scale  float32 [Hkv] (fp8 only, else None)
    fp8 scales are per (layer, kv head), separate for K and V, shared by every request and
    by both the prompt and the decode-token KV: scale = amax / 448.

    ``requests`` optionally restricts which requests' prompt KV is generated (others None).
    """
    W, K, P = shapes if shapes is not None else request_shapes(wl, seed)
    R = len(W)
    sumW = int(W.sum())
    S, Hq, Hkv, D = wl.S, wl.Hq, wl.Hkv, wl.D
    want = set(range(R)) if requests is None else set(requests)

    def normal(stream, *idx, shape):
        return _rng(seed, wl, stream, layer, *idx).standard_normal(shape, dtype=np.float32)

    q = normal(_S_Q, shape=(S, sumW, Hq, D))
    ks = [normal(_S_KS, r, shape=(Hkv, int(P[r]), D)) if r in want else None for r in range(R)]
    vs = [normal(_S_VS, r, shape=(Hkv, int(P[r]), D)) if r in want else None for r in range(R)]
    ku = normal(_S_KU, shape=(S, sumW, Hkv, D))
    vu = normal(_S_VU, shape=(S, sumW, Hkv, D))
    k_scale = v_scale = None
    if wl.kv_dtype == "fp8":
        # amax over every request of the layer (drawn even when not returned)
        def amax(stream, arrs, u):
            m = np.abs(u).max(axis=(0, 1, 3))
            for r in range(R):
                a = arrs[r] if arrs[r] is not None else normal(stream, r, shape=(Hkv, int(P[r]), D))
                m = np.maximum(m, np.abs(a).max(axis=(1, 2)))
            return m.astype(np.float32)
        k_scale = (amax(_S_KS, ks, ku) / np.float32(448.0)).astype(np.float32)
        v_scale = (amax(_S_VS, vs, vu) / np.float32(448.0)).astype(np.float32)
    qd = wl.q_dtype
    kd = wl.kv_dtype
    ksc = None if k_scale is None else k_scale[:, None, None]
    vsc = None if v_scale is None else v_scale[:, None, None]
    out = dict(
        q=_store(q, qd),
        k_s=[None if a is None else _store(a, kd, ksc) for a in ks],
        v_s=[None if a is None else _store(a, kd, vsc) for a in vs],
        k_u=_store(ku, kd, None if k_scale is None else k_scale[None, None, :, None]),
        v_u=_store(vu, kd, None if v_scale is None else v_scale[None, None, :, None]),
        k_scale=k_scale, v_scale=v_scale,
    )
    return out


def random_parents(wl: Workload, seed: int = 0, shapes=None, dead_frac: float = 0.0):
    """Parent pointers [S][sumW] int32 uniform in [0, W_r) per depth (request-local slot ids).

    Used by attention-only cases.  With ``dead_frac`` > 0 the last slots of each request
    are marked dead (-1) at every depth, like pad slots after a short pool.
    """
    W, K, P = shapes if shapes is not None else request_shapes(wl, seed)
    g = _rng(seed, wl, _S_PARENTS)
    sumW = int(W.sum())
    par = np.empty((wl.S, sumW), np.int32)
    off = 0
    for r, w in enumerate(W):
        w = int(w)
        n_live = w - int(round(dead_frac * w)) if dead_frac > 0 else w
        n_live = max(1, n_live)
        par[:, off:off + w] = g.integers(0, n_live, size=(wl.S, w))
        par[:, off + n_live:off + w] = -1
        off += w
    return par


# ----------------------------------------------------------------------------------------
# log-probabilities
# ----------------------------------------------------------------------------------------
def _log_softmax_f32(x: np.ndarray) -> np.ndarray:
    """Rows of x (float64) -> log_softmax in float64, rounded once to float32, clipped at 0."""
    m = x.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True))
    return np.minimum((x - lse).astype(np.float32), np.float32(0.0))


def _ultra_row(seed: int, wl: Workload, base: int, src: int) -> np.ndarray:
    """Row ``src`` of base matrix ``base`` of the ultra-wide workload (its own stream)."""
    g = _rng(seed, wl, _S_LOGITS, base, int(src))
    return _log_softmax_f32(g.standard_normal(wl.C) * wl.logit_sigma)


@functools.lru_cache(maxsize=2)
def _ultra_base(wl: Workload, seed: int, base: int, threads: int) -> np.ndarray:
    """Whole base matrix [W][C] of the ultra-wide workload, rows drawn by a thread pool (each
    row has its own generator, so the values do not depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    W = int(request_shapes(wl, seed)[0].sum())
    out = np.empty((W, wl.C), np.float32)

    def fill(lo):
        for i in range(lo, min(W, lo + 64)):
            out[i] = _ultra_row(seed, wl, base, i)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(0, W, 64)))
    return out


def logprob_rows(wl: Workload, step: int, seed: int = 0, shapes=None, rows=None, threads: int = 1):
    """Log-probabilities [sumW][C] float32 of one decode step.

    logits ~ N(0, sigma) per (step, slot) row (sigma is the standard deviation), then
    log_softmax in float64, rounded once to float32 (values are <= 0).

    The ultra-wide workload uses two base matrices; step d uses base d % 2 with its rows
    rotated by 7919 * d mod W (so 16 steps need only 2 x 2.8 GiB of host data).
    ``rows`` optionally selects a subset of slot rows.  For the ultra-wide workload without
    ``rows``, the step's base matrix is drawn once (by ``threads`` threads) and kept for the
    step of the same parity.
    """
    W, K, P = shapes if shapes is not None else request_shapes(wl, seed)
    sumW = int(W.sum())
    if wl.name == "ultra5000":
        base = step % 2
        shift = (7919 * step) % sumW
        idx = (np.arange(sumW) - shift) % sumW      # row i of step d = base row (i - shift)
        if rows is None:
            return _ultra_base(wl, seed, base, threads)[idx]
        idx = idx[np.asarray(rows)]
        out = np.empty((idx.size, wl.C), np.float32)
        # each base row has its own stream, so rows can be drawn independently
        for i, src in enumerate(idx):
            out[i] = _ultra_row(seed, wl, base, int(src))
        return out
    g = _rng(seed, wl, _S_LOGITS, step)
    x = g.standard_normal((sumW, wl.C)) * wl.logit_sigma
    lp = _log_softmax_f32(x)
    if rows is not None:
        lp = lp[np.asarray(rows)]
    return lp


def gumbel_rows(wl: Workload, step: int, seed: int = 0, shapes=None, rows=None):
    """Standard Gumbel draws [sumW][C] float32 for the sampled selection of one step.

    u is uniform on the open interval (0, 1) at 53-bit resolution ((k + 1/2) / 2^53 for an
    integer k), g = -log(-log(u)) in float64, rounded once to float32; every value is
    finite (about -3.6 .. 37.4).  The selection draws no random numbers itself: these
    rows are its noise input.  ``rows`` optionally selects a subset of slot rows.
    """
    if wl.name == "ultra5000":
        raise NotImplementedError("noise rows are not generated for the ultra-wide workload")
    W, K, P = shapes if shapes is not None else request_shapes(wl, seed)
    sumW = int(W.sum())
    g = _rng(seed, wl, _S_GUMBEL, step)
    k = g.integers(0, 1 << 53, size=(sumW, wl.C), dtype=np.int64)
    u = (k.astype(np.float64) + 0.5) / float(1 << 53)
    out = (-np.log(-np.log(u))).astype(np.float32)
    if rows is not None:
        out = out[np.asarray(rows)]
    return out


def logit_rows(wl: Workload, step: int, seed: int = 0, shapes=None, rows=None):
    """Raw logits [sumW][C] float32 of one decode step: the N(0, sigma) draws from which
    logprob_rows takes its log-softmax, rounded once to float32 (the input of the selection
    from raw logits)."""
    if wl.name == "ultra5000":
        raise NotImplementedError("raw logit rows are not generated for the ultra-wide workload")
    W, K, P = shapes if shapes is not None else request_shapes(wl, seed)
    sumW = int(W.sum())
    g = _rng(seed, wl, _S_LOGITS, step)
    x = (g.standard_normal((sumW, wl.C)) * wl.logit_sigma).astype(np.float32)
    if rows is not None:
        x = x[np.asarray(rows)]
    return x
