"""Pins of the oracle beam selection (CPU only).

S1  exhaustive pure-Python enumeration (struct-level float32 keys, counting-based
    per-beam top_k membership, tuple sort for the global beam_width) on many tiny cases
    with forced ties, -0.0 and -inf;
S2  K >= fan-out reduces to the textbook global top-W over all valid (beam, code);
S3  W = K = 1 is a constrained argmax with the lowest-code tie-break;
S4  with prefix-keyed log-probabilities and W >= |catalog|, the beam set after L steps is
    the whole catalog, ordered by the recursively defined tie rule;
S5  invariants on the synthetic workloads;
and the candidate-pool size the design doc prints for beam_width = top_k = 512.

Gumbel top-k (temperature T, noise g): G1 the enumeration above with perturbed ordering keys
float32(key + float32(T * g)); G2 T = 0 reduces exactly to the deterministic selection; G3
the Gumbel-max law: with one live beam and W = K = 1 the selected code is distributed as
softmax(lp / T) (chi-square over 20 000 draws); G4 the returned scores hold no noise and the
outputs are ordered by the perturbed key.

First-step fan-out: F1 at level 0 (one live prompt beam) the selection with top_k = W is the
textbook top-W of that beam's valid codes by (key descending, code ascending), pads after;
with top_k < W the plain first step keeps only top_k of them.

Selection from raw logits: L1 the row lse equals scipy's logsumexp rounded to float32, and
exp(lp) sums to 1; L2 with logits that already are log-probabilities rounded from a float64
log-softmax, the lse is ~0 and the selection matches the log-probability oracle up to the
rounding of that lse; L3 adding a power of two to a row's logits, when it keeps every logit's
bits exact, leaves that row's lp unchanged.
"""
import os
import struct

import numpy as np
import pytest

from oracle.select import catalog_prefix_sets, initial_beams, oracle_beam_search, oracle_select
from synth import build_trie_csr, catalog_items, logprob_rows, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG_INF = float("-inf")


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def enumerate_select(lp, scores, prefixes, level, K, W, C, items, noise=None, temperature=0.0):
    """Independent pure-Python selection by enumeration of the whole W x C grid.  With
    noise, candidates are ordered by float32(key + float32(T * g)) and keep their key as
    score.  (Each float32 operation is done in double and rounded once: for a sum or
    product of two float32 values that equals the float32 operation.)"""
    L = len(items[0]) if items else 0
    prefix_set = {tuple(it[:level + 1]) for it in items} if items is not None else None
    cands = []
    for b, s in enumerate(scores):
        if s == NEG_INF:
            continue
        for c in range(C):
            if prefix_set is not None and tuple(prefixes[b]) + (c,) not in prefix_set:
                continue
            key = f32(float(s) + float(lp[b][c]))         # fp32 + fp32, rounded once
            if key == NEG_INF:
                continue
            okey = key
            if noise is not None:
                okey = f32(key + f32(f32(temperature) * float(noise[b][c])))
                if okey == NEG_INF:
                    continue
            cands.append((okey, b, c, key))
    # per-beam top-K membership: fewer than K candidates of the same beam rank above it
    def better(x, y):   # x ranks strictly above y
        return x[0] > y[0] or (x[0] == y[0] and x[1] * C + x[2] < y[1] * C + y[2])
    pool = [x for x in cands if sum(1 for y in cands if y[1] == x[1] and better(y, x)) < K]
    pool.sort(key=lambda x: (-x[0], x[1] * C + x[2]))
    sel = pool[:W]
    tokens = [x[2] for x in sel] + [-1] * (W - len(sel))
    parents = [x[1] for x in sel] + [-1] * (W - len(sel))
    sc = [x[3] for x in sel] + [NEG_INF] * (W - len(sel))
    newp = [tuple(prefixes[x[1]]) + (x[2],) for x in sel] + [None] * (W - len(sel))
    return tokens, parents, sc, newp, len(pool)


def _unpack(p, C, L):
    out = []
    for _ in range(L):
        out.append(p % C)
        p //= C
    return tuple(reversed(out))


def _run_both(rng, W, K, C, L, n_items, tie_values, steps=None, sampled=False):
    items = None
    if n_items:
        space = C ** L
        n_items = min(n_items, space)
        packed = rng.choice(space, size=n_items, replace=False)
        items = [_unpack(int(p), C, L) for p in packed]
    psets = catalog_prefix_sets(np.array(items), C) if items is not None else None
    scores, prefixes = initial_beams(W)
    tprefixes = [() if p is not None else None for p in prefixes]
    for level in range(steps or L):
        if tie_values:
            lp = rng.choice(np.array([0.0, -0.0, -0.5, -1.0, -np.inf], np.float32), size=(W, C))
        else:
            lp = np.minimum(rng.standard_normal((W, C)).astype(np.float32), 0)
        noise, temp = None, 0.0
        if sampled:
            temp = float(rng.choice([0.0, 0.25, 1.0, 3.0]))
            if tie_values:      # few distinct values, so perturbed keys tie often
                noise = rng.choice(np.array([0.0, -0.0, 0.5, -1.0, 2.0], np.float32), size=(W, C))
            else:
                noise = (-np.log(-np.log(rng.uniform(1e-12, 1.0, size=(W, C))))).astype(np.float32)
        res = oracle_select(lp, scores, prefixes, level, K, W, C, psets, noise, temp)
        t2, p2, s2, np2, pool2 = enumerate_select(lp.tolist(), scores.tolist(), tprefixes, level, K, W, C, items,
                                                  noise.tolist() if noise is not None else None, temp)
        assert res["tokens"].tolist() == t2
        assert res["parents"].tolist() == p2
        assert [struct.pack("<f", x) for x in res["scores"].tolist()] == \
               [struct.pack("<f", x) for x in s2]
        assert res["pool_size"] == pool2
        got_prefixes = [None if p is None else _unpack(p, C, level + 1) for p in res["prefixes"]]
        assert got_prefixes == np2
        scores, prefixes, tprefixes = res["scores"], res["prefixes"], np2


@pytest.mark.parametrize("seed", range(4))
def test_exhaustive_enumeration_tiny_random(seed):
    rng = np.random.default_rng(100 + seed)
    n_cases = int(os.environ.get("GRW_S1_CASES", "2500"))
    for _ in range(n_cases):
        W = int(rng.integers(1, 9))
        K = int(rng.integers(1, 9))
        C = int(rng.integers(2, 17))
        L = int(rng.integers(1, 5))
        n_items = int(rng.integers(0, 41))       # 0 = unconstrained
        _run_both(rng, W, K, C, L, n_items, tie_values=bool(rng.integers(0, 2)))


def test_exhaustive_enumeration_tiny_workload_every_step():
    """The tiny fp32 workload at full size: every step against enumeration."""
    wl = workload("tiny")
    items = catalog_items(wl)
    psets = catalog_prefix_sets(items, wl.C)
    steps = oracle_beam_search(lambda d: logprob_rows(wl, d), wl.W, wl.K, wl.C, wl.S, psets)
    scores, prefixes = initial_beams(wl.W)
    tpre = [() if p is not None else None for p in prefixes]
    item_list = [tuple(int(v) for v in it) for it in items]
    for d, res in enumerate(steps):
        lp = logprob_rows(wl, d)
        t, p, s, npre, pool = enumerate_select(lp.tolist(), scores.tolist(), tpre, d, wl.K, wl.W,
                                               wl.C, item_list)
        assert res["tokens"].tolist() == t and res["parents"].tolist() == p
        assert res["scores"].tolist() == s and res["pool_size"] == pool
        scores, prefixes, tpre = res["scores"], res["prefixes"], npre


def test_k_at_least_fanout_is_global_topw():
    rng = np.random.default_rng(7)
    for _ in range(200):
        W, C, L = int(rng.integers(1, 12)), int(rng.integers(2, 30)), 3
        items = np.unique(rng.integers(0, C, size=(int(rng.integers(1, 200)), L)), axis=0)
        psets = catalog_prefix_sets(items, C)
        K = C                                   # at least every fan-out
        scores, prefixes = initial_beams(W)
        for level in range(L):
            lp = np.minimum(rng.standard_normal((W, C)).astype(np.float32), 0)
            res = oracle_select(lp, scores, prefixes, level, K, W, C, psets)
            # textbook: all valid (b, c), lexsort by (-key, flat)
            keys, flats = [], []
            for b in range(W):
                if scores[b] == -np.inf:
                    continue
                for c in range(C):
                    if prefixes[b] * C + c in set(psets[level + 1].tolist()):
                        keys.append(np.float32(scores[b]) + lp[b, c])
                        flats.append(b * C + c)
            keys, flats = np.array(keys, np.float32), np.array(flats)
            order = np.lexsort((flats, -keys))[:W]
            n = order.size
            assert np.array_equal(res["parents"][:n], flats[order] // C)
            assert np.array_equal(res["tokens"][:n], flats[order] % C)
            assert np.all(res["parents"][n:] == -1)
            scores, prefixes = res["scores"], res["prefixes"]


def test_first_step_fanout_is_top_w_of_the_prompt_row():
    rng = np.random.default_rng(17)
    for _ in range(300):
        W, C, L = int(rng.integers(1, 40)), int(rng.integers(2, 64)), 3
        items = np.unique(rng.integers(0, C, size=(int(rng.integers(1, 300)), L)), axis=0)
        psets = catalog_prefix_sets(items, C)
        scores, prefixes = initial_beams(W)
        lp = rng.choice(np.array([0.0, -0.5, -0.5, -1.0, -2.0, -np.inf], np.float32), size=(W, C))
        res = oracle_select(lp, scores, prefixes, 0, W, W, C, psets)
        valid = sorted(set(int(p) for p in psets[1].tolist()))
        keys = np.array([np.float32(0.0) + lp[0, c] for c in valid], np.float32)
        codes = np.array(valid)
        keep = keys != -np.inf
        keys, codes = keys[keep], codes[keep]
        order = np.lexsort((codes, -keys))[:W]
        n = order.size
        assert np.array_equal(res["tokens"][:n], codes[order])
        assert np.all(res["parents"][:n] == 0) and np.all(res["parents"][n:] == -1)
        assert np.all(res["tokens"][n:] == -1)
        K = max(1, W // 3)
        plain = oracle_select(lp, scores, prefixes, 0, K, W, C, psets)
        assert int((plain["parents"] >= 0).sum()) == min(K, n)
        assert np.array_equal(plain["tokens"][:min(K, n)], codes[order][:min(K, n)])


def test_width_one_is_constrained_argmax():
    rng = np.random.default_rng(8)
    for _ in range(300):
        C, L = int(rng.integers(2, 20)), 3
        items = np.unique(rng.integers(0, C, size=(int(rng.integers(1, 60)), L)), axis=0)
        psets = catalog_prefix_sets(items, C)
        scores, prefixes = initial_beams(1)
        path = ()
        for level in range(L):
            lp = rng.choice(np.array([0.0, -0.25, -1.0], np.float32), size=(1, C))
            res = oracle_select(lp, scores, prefixes, level, 1, 1, C, psets)
            valid = [c for c in range(C) if any(tuple(it[:level + 1]) == path + (c,) for it in items.tolist())]
            keys = [np.float32(scores[0]) + lp[0, c] for c in valid]
            best = valid[int(np.argmax(keys))]          # first maximum = lowest code
            assert res["tokens"][0] == best
            path = path + (best,)
            scores, prefixes = res["scores"], res["prefixes"]
        assert path in {tuple(it) for it in items.tolist()}


def test_full_catalog_closed_form():
    """W >= |catalog|, K >= max fan-out, prefix-keyed log-probs: after L steps the beams are
    exactly the catalog, ordered by path score with the recursive tie rule."""
    rng = np.random.default_rng(9)
    vals = np.array([0.0, -0.5, -1.0, -2.0, -0.125], np.float32)
    for trial in range(40):
        C, L = int(rng.integers(2, 7)), int(rng.integers(1, 4))
        items = np.unique(rng.integers(0, C, size=(int(rng.integers(1, 40)), L)), axis=0)
        N = len(items)
        W, K = N + int(rng.integers(0, 3)), C
        psets = catalog_prefix_sets(items, C)
        salt = int(rng.integers(0, 2 ** 31))

        def lp_of_prefix(prefix_tuple):
            h = np.random.default_rng([salt, len(prefix_tuple), *prefix_tuple])
            return h.choice(vals, size=C)

        # run the oracle, feeding each slot the row keyed by its prefix
        scores, prefixes = initial_beams(W)
        tuples = [() if p is not None else None for p in prefixes]
        for level in range(L):
            lp = np.zeros((W, C), np.float32)
            for b in range(W):
                if tuples[b] is not None:
                    lp[b] = lp_of_prefix(tuples[b])
            res = oracle_select(lp, scores, prefixes, level, K, W, C, psets)
            tuples = [None if p is None else tuples[pa] + (int(t),)
                      for p, pa, t in zip(res["prefixes"], res["parents"], res["tokens"])]
            scores, prefixes = res["scores"], res["prefixes"]
        # closed form: rank every prefix level by level
        ranked = [((), 0.0)]
        for level in range(L):
            nxt = []
            for slot, (pre, sc) in enumerate(ranked):
                for c in range(C):
                    t = pre + (c,)
                    if any(tuple(it[:level + 1]) == t for it in items.tolist()):
                        key = f32(sc + float(lp_of_prefix(pre)[c]))
                        nxt.append((key, slot * C + c, t))
            nxt.sort(key=lambda x: (-x[0], x[1]))
            ranked = [(t, k) for k, _, t in nxt]
        assert [t for t, _ in ranked] == tuples[:N]
        assert sorted(tuples[:N]) == sorted(tuple(int(v) for v in it) for it in items)
        assert all(t is None for t in tuples[N:])


def _check_invariants(res, lp, scores, prefixes, level, K, W, C, psets):
    n = int((res["parents"] >= 0).sum())
    assert np.all(res["parents"][:n] >= 0) and np.all(res["parents"][n:] == -1)
    assert n == min(W, res["pool_size"])
    par, tok, sc = res["parents"][:n], res["tokens"][:n], res["scores"][:n]
    assert np.all(np.isfinite(scores[par]))                       # parents are live
    recomputed = (scores[par] + lp[par, tok]).astype(np.float32)
    assert np.array_equal(recomputed.view(np.uint32) & 0x7FFFFFFF, sc.view(np.uint32) & 0x7FFFFFFF)
    flat = par.astype(np.int64) * C + tok
    assert np.unique(flat).size == n                              # no duplicates
    ok = (sc[:-1] > sc[1:]) | ((sc[:-1] == sc[1:]) & (flat[:-1] < flat[1:]))
    assert np.all(ok)                                             # sorted by the tie rule
    if psets is not None:
        newp = np.array([res["prefixes"][i] for i in range(n)], np.int64)
        assert np.all(np.isin(newp, psets[level + 1]))            # valid catalog prefixes


@pytest.mark.parametrize("name", ["tiny", "qwen06b"])
def test_invariants_on_workloads(name):
    wl = workload(name)
    items = catalog_items(wl)
    psets = catalog_prefix_sets(items, wl.C)
    W = wl.W
    for r in range(2 if name == "qwen06b" else 1):
        scores, prefixes = initial_beams(W)
        for d in range(wl.S):
            lp = logprob_rows(wl, d)[r * W:(r + 1) * W]
            res = oracle_select(lp, scores, prefixes, d, wl.K, W, wl.C, psets)
            _check_invariants(res, lp, scores, prefixes, d, wl.K, W, wl.C, psets)
            scores, prefixes = res["scores"], res["prefixes"]


def test_pool_size_printed_by_design_doc():
    """tests/golden/pool_size_w512_k512.txt: beam_width = top_k = 512 gives a 262144 pool."""
    with open(os.path.join(GOLDEN, "pool_size_w512_k512.txt")) as f:
        fields = dict(line.split("=", 1) for line in f.read().split("\n")
                      if "=" in line and not line.startswith("#"))
    W, K, pool = int(fields["beam_width"]), int(fields["top_k"]), int(fields["pool"])
    C = 1024
    rng = np.random.default_rng(10)
    lp = np.minimum(rng.standard_normal((W, C)).astype(np.float32), 0)
    scores = np.full(W, -1.0, np.float32)          # every slot live
    res = oracle_select(lp, scores, [0] * W, 1, K, W, C, None)
    assert res["pool_size"] == pool == W * K


def test_csr_trie_agrees_with_catalog_prefixes():
    """The CSR the GPU consumes encodes exactly the catalog prefix sets (layout check)."""
    rng = np.random.default_rng(11)
    C, L = 9, 3
    items = np.unique(rng.integers(0, C, size=(150, L)), axis=0)
    t = build_trie_csr(items, C)
    psets = catalog_prefix_sets(items, C)
    rp, code = t["row_ptr"], t["code"]
    # walk every edge: the child's prefix is the parent's prefix extended by the code
    for n in range(t["n_internal"]):
        for e in range(rp[n], rp[n + 1]):
            child = e + 1
            assert t["node_depth"][child] == t["node_depth"][n] + 1
            assert t["node_prefix"][child] == t["node_prefix"][n] * C + code[e]
        assert np.all(np.diff(code[rp[n]:rp[n + 1]]) > 0)
    for l in range(1, L + 1):
        assert np.array_equal(np.sort(t["node_prefix"][t["node_depth"] == l]), psets[l])


@pytest.mark.parametrize("seed", range(2))
def test_gumbel_exhaustive_enumeration_tiny_random(seed):
    """G1: the sampled selection against the enumeration with perturbed ordering keys."""
    rng = np.random.default_rng(300 + seed)
    n_cases = int(os.environ.get("GRW_G1_CASES", "1500"))
    for _ in range(n_cases):
        W = int(rng.integers(1, 9))
        K = int(rng.integers(1, 9))
        C = int(rng.integers(2, 17))
        L = int(rng.integers(1, 5))
        n_items = int(rng.integers(0, 41))
        _run_both(rng, W, K, C, L, n_items, tie_values=bool(rng.integers(0, 2)), sampled=True)


@pytest.mark.parametrize("name", ["tiny", "qwen06b"])
def test_gumbel_temperature_zero_is_deterministic(name):
    """G2: T = 0 gives exactly the deterministic selection, whatever the noise."""
    from synth import gumbel_rows, request_shapes
    wl = workload(name)
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    psets = catalog_prefix_sets(items, wl.C)
    w, k = int(W[0]), int(K[0])
    a = oracle_beam_search(lambda d: logprob_rows(wl, d)[:w], w, k, wl.C, wl.S, psets)
    b = oracle_beam_search(lambda d: logprob_rows(wl, d)[:w], w, k, wl.C, wl.S, psets,
                           noise_of_step=lambda d: gumbel_rows(wl, d)[:w], temperature=0.0)
    for ra, rb in zip(a, b):
        assert ra["tokens"].tolist() == rb["tokens"].tolist()
        assert ra["parents"].tolist() == rb["parents"].tolist()
        assert ra["scores"].view(np.uint32).tolist() == rb["scores"].view(np.uint32).tolist()


@pytest.mark.parametrize("temp", [0.5, 1.0, 2.0])
def test_gumbel_max_law(temp):
    """G3: one live beam, W = K = 1, unconstrained: the chosen code follows softmax(lp / T)."""
    from scipy.stats import chisquare
    rng = np.random.default_rng(7)
    C, n = 6, 20000
    logits = np.array([1.5, 0.2, -0.3, 0.9, -1.2, 0.0])
    lp = (logits - np.log(np.exp(logits).sum())).astype(np.float32)[None, :]
    scores, prefixes = initial_beams(1)
    counts = np.zeros(C)
    for _ in range(n):
        g = (-np.log(-np.log(rng.uniform(1e-15, 1.0, size=(1, C))))).astype(np.float32)
        res = oracle_select(lp, scores, prefixes, 0, 1, 1, C, None, g, temp)
        counts[res["tokens"][0]] += 1
    p = np.exp(lp[0].astype(np.float64) / temp)
    p /= p.sum()
    assert chisquare(counts, n * p).pvalue > 1e-4
    # noise added without the temperature would give another law
    q = np.exp(lp[0].astype(np.float64))
    q /= q.sum()
    if temp != 1.0:
        assert chisquare(counts, n * q).pvalue < 1e-6


def test_gumbel_scores_exclude_noise_and_order_by_perturbed_key():
    """G4 on the qwen06b-shaped workload (one request, all steps, T = 1)."""
    from synth import gumbel_rows, request_shapes
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    psets = catalog_prefix_sets(items, wl.C)
    w, k = int(W[0]), int(K[0])
    scores, prefixes = initial_beams(w)
    for d in range(wl.S):
        lp = logprob_rows(wl, d)[:w]
        g = gumbel_rows(wl, d)[:w]
        res = oracle_select(lp, scores, prefixes, d, k, w, wl.C, psets, g, 1.0)
        n = int((res["parents"] >= 0).sum())
        par, tok = res["parents"][:n], res["tokens"][:n]
        want = scores[par] + lp[par, tok]
        assert res["scores"][:n].view(np.uint32).tolist() == want.view(np.uint32).tolist()
        okey = want + np.float32(1.0) * g[par, tok]
        flat = par.astype(np.int64) * wl.C + tok
        assert all((okey[i] > okey[i + 1]) or (okey[i] == okey[i + 1] and flat[i] < flat[i + 1])
                   for i in range(n - 1))
        scores, prefixes = res["scores"], res["prefixes"]


def _logit_rows(seed, n, C, sigma=3.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, C)) * sigma).astype(np.float32)


def test_logits_lse_matches_library_logsumexp():
    """L1."""
    from scipy.special import logsumexp
    from oracle.select import oracle_log_softmax_rows
    for seed, (n, C) in enumerate([(64, 8192), (300, 257), (5, 3)]):
        x = _logit_rows(seed, n, C)
        x[0, : C // 2] = -np.inf                # masked logits
        lp, lse = oracle_log_softmax_rows(x)
        ref = logsumexp(x.astype(np.float64), axis=1)
        assert lse.tolist() == ref.astype(np.float32).tolist()
        s = np.exp(lp.astype(np.float64)).sum(axis=1)
        assert np.all(np.abs(s - 1.0) < 1e-5)
        assert (lp <= 0).all()


def test_logits_selection_equals_logprob_selection_for_normalised_rows():
    """L2: rows that are already log-softmax outputs have lse within float32 rounding of 0."""
    from oracle.select import oracle_select_logits
    wl = workload("qwen06b")
    from synth import request_shapes
    W, K, P = request_shapes(wl)
    w, k = int(W[0]), int(K[0])
    items = catalog_items(wl)
    psets = catalog_prefix_sets(items, wl.C)
    scores, prefixes = initial_beams(w)
    for d in range(wl.S):
        lp = logprob_rows(wl, d)[:w]
        a = oracle_select(lp, scores, prefixes, d, k, w, wl.C, psets)
        b = oracle_select_logits(lp, scores, prefixes, d, k, w, wl.C, psets)
        # the lse of a normalised row is 0 up to float64 rounding; where it rounds to 0 in
        # float32 the two selections are identical
        from oracle.select import oracle_log_softmax_rows
        live = scores != -np.inf
        lse = oracle_log_softmax_rows(lp[live])[1]
        assert np.all(np.abs(lse) < 1e-6)
        if np.all(lse == 0):
            assert a["tokens"].tolist() == b["tokens"].tolist()
            assert a["parents"].tolist() == b["parents"].tolist()
            assert a["scores"].view(np.uint32).tolist() == b["scores"].view(np.uint32).tolist()
        scores, prefixes = a["scores"], a["prefixes"]


def test_logits_shift_by_exact_power_of_two():
    """L3: rows whose lse lies in [16, 32) before and after adding 2 to every logit (exact in
    float32 for logits on a 1/64 grid): the float32 lse moves by exactly 2 and lp keeps its
    bits, as ln-sum-exp is shift-equivariant and both roundings see the same grid."""
    from oracle.select import oracle_log_softmax_rows
    rng = np.random.default_rng(9)
    x = (np.round(rng.standard_normal((64, 512)) * 64) / 64 + 16.0).astype(np.float32)
    y = (x + np.float32(2.0)).astype(np.float32)
    assert np.array_equal(y - np.float32(2.0), x)          # the shift is exact
    lp0, lse0 = oracle_log_softmax_rows(x)
    lp1, lse1 = oracle_log_softmax_rows(y)
    assert np.all((lse0 >= 16) & (lse1 < 32))
    assert np.array_equal(lse1, lse0 + np.float32(2.0))
    assert np.array_equal(lp0.view(np.uint32), lp1.view(np.uint32))
