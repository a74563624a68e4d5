"""Oracle beam selection: per-beam top_k over trie-valid candidates, then top beam_width.

Sources:
* xLLM generative-recommendation design doc, §4.1.1: every beam expands top_k candidates
  and the new beam set of size beam_width is chosen from the global beam_width x top_k
  pool; §4.3: invalid item paths are filtered during the search.
* FlashRec announcement (SGLang PR thread): with the semantic-ID trie, illegal IDs are
  never candidates.
* FlashRec deployment guide, request section: temperature 0 gives a deterministic top-k;
  a positive temperature gives a Gumbel top-k whose noise only orders the candidates, the
  returned sequence score holding none of it.

Readings where the pages are silent (each is the plainest one the rest supports):
* the ranking key of candidate (b, c) is the float32 sum score_b + lp[b, c] (one IEEE
  rounding); candidates whose key is -inf are not candidates;
* ties break by key descending, then flat index b * C + c ascending (within one beam this
  is code ascending); -0.0 and +0.0 compare equal;
* a beam whose score is -inf is dead and contributes nothing; a beam with fewer than
  top_k valid children contributes all of them; a pool smaller than beam_width leaves
  pad slots (token -1, parent -1, score -inf) after all real slots;
* at level 0 only slot 0 is live (score 0, empty prefix); the first-step fan-out variant (the
  prompt beam expanded to the full beam width, FlashRec deployment guide, wide-beam section)
  is this selection with top_k = beam_width at level 0;
* code c is valid for a beam with prefix p at level l iff p + (c,) is the length-(l+1)
  prefix of some catalog item (decided from the raw item list);
* selection from raw logits (the fused variant): lse_b = float32(ln sum_c exp(x_bc)) over
  the whole row of C codes, evaluated in float64 and rounded once, and lp = float32(x - lse_b)
  by one float32 subtraction; rounding the row's lse before the subtraction confines any
  difference between two float64 evaluations to that one rounding per row;
* Gumbel top-k at temperature T >= 0 with noise g (standard Gumbel draws, an input): the
  ordering key of (b, c) is float32(key + float32(T * g[b, c])), two IEEE roundings;
  every top_k / beam_width decision and tie rule above uses it in place of the key, and
  the returned score is the key itself.  Multiplying the noise by T keeps the key's units;
  for T > 0 the order equals that of key / T + g, the Gumbel-max form of sampling
  proportionally to exp(key / T).  A candidate whose ordering key is -inf is dropped.
"""
from __future__ import annotations

import numpy as np

NEG_INF = np.float32(-np.inf)


def catalog_prefix_sets(items: np.ndarray, C: int):
    """Sorted unique packed prefixes of every length 1..L, from the raw item list.

    Entry l (1-based length) holds the int64 base-C packing of items[:, :l].
    """
    items = np.asarray(items, dtype=np.int64)
    L = items.shape[1]
    sets = [None]
    packed = np.zeros(items.shape[0], np.int64)
    for l in range(1, L + 1):
        packed = packed * C + items[:, l - 1]
        sets.append(np.unique(packed))
    return sets


def _is_member(sorted_set: np.ndarray, keys: np.ndarray) -> np.ndarray:
    idx = np.searchsorted(sorted_set, keys)
    idx_c = np.minimum(idx, sorted_set.size - 1)
    return (idx < sorted_set.size) & (sorted_set[idx_c] == keys)


def oracle_select(lp, scores, prefixes, level, K, W, C, prefix_sets=None, noise=None, temperature=0.0,
                  threads=1):
    """One selection step of one request.

    lp        float32 [Wslots][C]   log-probabilities of this step
    scores    float32 [Wslots]      beam scores (-inf = dead slot)
    prefixes  list[int | None]      packed prefix of each slot (None for dead slots)
    level     number of codes already in each live prefix
    K, W      top_k and beam_width of the request
    prefix_sets  output of catalog_prefix_sets, or None when unconstrained
    noise     float32 [Wslots][C] Gumbel draws of the sampled selection, or None
    temperature  T >= 0 of the sampled selection (T = 0 orders by the key alone)
    threads   beams whose per-beam sort runs at once (a thread pool: numpy releases the
              interpreter lock inside its sorts); every beam's arithmetic is the same

    Returns a dict: tokens int32 [W], parents int32 [W], scores float32 [W],
    prefixes (list of packed prefixes, None for pad slots) and pool_size (the number of
    candidates that survived the per-beam top_k).
    """
    lp = np.asarray(lp, dtype=np.float32)
    scores = np.asarray(scores, dtype=np.float32)
    assert not np.isnan(scores).any()
    t = np.float32(temperature)
    assert np.isfinite(t) and t >= 0
    if noise is not None:
        noise = np.asarray(noise, dtype=np.float32)
        assert np.isfinite(noise).all()
    all_codes = np.arange(C, dtype=np.int64)

    def beam_top_k(b):
        """Beam b's top_k candidates (keys, ordering keys, flat indices), or None."""
        s = scores[b]
        if s == NEG_INF:
            return None
        codes = all_codes
        if prefix_sets is not None:
            codes = all_codes[_is_member(prefix_sets[level + 1], prefixes[b] * C + all_codes)]
        keys = s + lp[b, codes]                       # float32 + float32 -> float32
        assert keys.dtype == np.float32
        assert not np.isnan(keys).any(), "NaN log-probability"
        okeys = keys if noise is None else keys + t * noise[b, codes]   # two float32 roundings
        assert okeys.dtype == np.float32
        live = (keys != NEG_INF) & (okeys != NEG_INF)
        codes, keys, okeys = codes[live], keys[live], okeys[live]
        order = np.lexsort((codes, -okeys))[:K]       # full stable sort, keep top_k
        return keys[order], okeys[order], b * C + codes[order]

    beams = range(scores.shape[0])
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(beam_top_k, beams))
    else:
        parts = [beam_top_k(b) for b in beams]
    parts = [x for x in parts if x is not None]
    pool_key = [x[0] for x in parts]
    pool_okey = [x[1] for x in parts]
    pool_flat = [x[2] for x in parts]
    tokens = np.full(W, -1, np.int32)
    parents = np.full(W, -1, np.int32)
    out_scores = np.full(W, NEG_INF, np.float32)
    new_prefixes = [None] * W
    if pool_key:
        key = np.concatenate(pool_key)
        okey = np.concatenate(pool_okey)
        flat = np.concatenate(pool_flat)
        order = np.lexsort((flat, -okey))[:W]
        n = order.size
        tokens[:n] = flat[order] % C
        parents[:n] = flat[order] // C
        out_scores[:n] = key[order]
        for i in range(n):
            new_prefixes[i] = int(prefixes[parents[i]]) * C + int(tokens[i])
    pool_size = int(sum(k.size for k in pool_key))
    return dict(tokens=tokens, parents=parents, scores=out_scores, prefixes=new_prefixes,
                pool_size=pool_size)


def oracle_log_softmax_rows(logits):
    """Log-softmax of raw logit rows as the fused selection defines it.

    lse_b = float32(ln sum_c exp(x_bc)), evaluated in float64 as m + ln(sum exp(x - m)) with
    m the row max and rounded once to float32; lp_bc = float32(x_bc - lse_b), one float32
    subtraction.  Logits are finite or -inf, at least one finite per row.
    Returns (lp float32 [n][C], lse float32 [n]).
    """
    x32 = np.asarray(logits, dtype=np.float32)
    assert not np.isnan(x32).any() and not np.isposinf(x32).any()
    x = x32.astype(np.float64)
    m = x.max(axis=1)
    assert np.isfinite(m).all(), "a row without a finite logit"
    lse = (m + np.log(np.exp(x - m[:, None]).sum(axis=1))).astype(np.float32)
    lp = x32 - lse[:, None]                      # float32 - float32
    assert lp.dtype == np.float32
    return lp, lse


def oracle_select_logits(logits, scores, prefixes, level, K, W, C, prefix_sets=None, noise=None,
                         temperature=0.0):
    """The selection step from raw logits: log-softmax of every live row over all C codes
    (oracle_log_softmax_rows), then oracle_select on the result."""
    scores = np.asarray(scores, dtype=np.float32)
    lp = np.zeros(np.shape(logits), np.float32)
    live = scores != NEG_INF
    if live.any():
        lp[live] = oracle_log_softmax_rows(np.asarray(logits, np.float32)[live])[0]
    return oracle_select(lp, scores, prefixes, level, K, W, C, prefix_sets, noise, temperature)


def initial_beams(W):
    """Level-0 beam state: slot 0 live with score 0 and the empty prefix."""
    scores = np.full(W, NEG_INF, np.float32)
    scores[0] = 0.0
    prefixes = [None] * W
    prefixes[0] = 0
    return scores, prefixes


def oracle_beam_search(lp_of_step, W, K, C, S, prefix_sets=None, noise_of_step=None, temperature=0.0):
    """S selection steps of one request.  ``lp_of_step(d)`` returns float32 [W][C], and
    ``noise_of_step(d)`` the step's Gumbel draws for the sampled selection.

    Returns the list of per-step results of oracle_select.
    """
    scores, prefixes = initial_beams(W)
    steps = []
    for d in range(S):
        noise = noise_of_step(d) if noise_of_step is not None else None
        res = oracle_select(lp_of_step(d), scores, prefixes, d, K, W, C, prefix_sets, noise, temperature)
        steps.append(res)
        scores, prefixes = res["scores"], res["prefixes"]
    return steps
