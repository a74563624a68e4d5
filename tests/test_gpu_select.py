"""GPU parity of beam_select against the oracle: bit-exact tokens, parents, score bits, order
and trie nodes, on the synthetic workloads and on edge cases."""
import numpy as np
import pytest
import torch

from synth import catalog_items, logprob_rows, request_shapes, workload
from tests.gpu_util import oracle_threads, say, select_loop_vs_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "qwen06b"])
def test_workload_every_step(lib, name):
    wl = workload(name)
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say(f"[select] {name}: R={len(W)} W={W[0]} K={K[0]} C={wl.C}")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, label=name)


def test_wide512_zipf_trie(lib):
    wl = workload("wide512")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say(f"[select] wide512: {len(items)} items")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items,
                          check=[0, 3], label="wide512")


def test_wide512_unconstrained_full_pool(lib):
    wl = workload("wide512u")
    W, K, P = request_shapes(wl)
    say("[select] wide512u")
    loop, ws = select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), None,
                                     check=[1], label="wide512u")
    # with every beam live, the pilot bound keeps a small part of the 262144-entry pool
    assert loop.pool_sizes[1][-1] < int(W[1]) * int(K[1]) // 8, loop.pool_sizes


def test_wide_requests_beyond_the_fused_limit(lib):
    """W > 1024: pilot, per-beam and the 1024-thread global select kernels."""
    rng = np.random.default_rng(7)
    W, K, C, S = [1200, 1500], [16, 3], 500, 3
    lps = [rng.normal(0.0, 2.0, size=(sum(W), C)) for _ in range(S)]
    lps = [(x - np.log(np.exp(x).sum(axis=1, keepdims=True))).astype(np.float32) for x in lps]
    lps = [np.minimum(x, 0.0) for x in lps]
    say("[select] W > 1024")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="wide-multi")


def test_maximum_width(lib):
    """The largest beam width the library takes (8192): the first step fans the prompt beam
    out to 4096 children, the next fills all 8192 slots from the 4096 x 2 pool."""
    rng = np.random.default_rng(8)
    W, K, C, S = [8192], [2], 4096, 2
    lps = [rng.normal(0.0, 2.0, size=(sum(W), C)) for _ in range(S)]
    lps = [np.minimum((x - np.log(np.exp(x).sum(axis=1, keepdims=True))).astype(np.float32), 0.0) for x in lps]
    say("[select] W = 8192")
    loop, ws = select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="w8192", fanout=True)
    assert int((loop.parents[1] >= 0).sum().item()) == 8192


def test_mixed_ragged_batch(lib):
    wl = workload("mixed_fp8")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    rng = np.random.default_rng(0)
    check = sorted(set(rng.choice(len(W) - 1, size=12, replace=False).tolist()) | {len(W) - 1})
    say(f"[select] mixed: R={len(W)} sumW={W.sum()} checking {check}")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, check=check,
                          label="mixed")


def _tie_lp(rng, n, C, values):
    return rng.choice(np.array(values, np.float32), size=(n, C))


@pytest.mark.parametrize("seed", range(3))
def test_random_small_batches_with_ties(lib, seed):
    """Many small requests in one ragged batch: ties, -0.0, -inf, K > fan-out, pools
    smaller than W (pads), W = 1 and K = 1."""
    rng = np.random.default_rng(1000 + seed)
    C = int(rng.integers(2, 40))
    L = 3
    items = np.unique(rng.integers(0, C, size=(int(rng.integers(5, 300)), L)), axis=0)
    R = 40
    Ws = rng.integers(1, 12, size=R)
    Ks = rng.integers(1, 12, size=R)
    sumW = int(Ws.sum())
    tie = seed % 2 == 0

    def lp(d):
        g = np.random.default_rng([seed, d])
        if tie:
            return _tie_lp(g, sumW, C, [0.0, -0.0, -0.5, -1.0, -np.inf])
        return np.minimum(g.standard_normal((sumW, C)).astype(np.float32), 0)

    select_loop_vs_oracle(lib, Ws, Ks, C, L, lp, items, label=f"random{seed}")
    select_loop_vs_oracle(lib, Ws, Ks, C, L, lp, None, label=f"random{seed}u")


def test_long_rows_stream_through_buffer(lib):
    """Unconstrained rows longer than the LDS buffer, C not a multiple of the chunk:
    exercises compaction rounds and the admission threshold."""
    C = 30011
    Ws, Ks = [7, 33, 5], [3, 64, 200]
    rng = np.random.default_rng(5)
    lps = [np.minimum(rng.standard_normal((sum(Ws), C)).astype(np.float32) * 2, 0) for _ in range(3)]
    select_loop_vs_oracle(lib, Ws, Ks, C, 3, lambda d: lps[d], None, label="long")


def test_early_exit_bound_keeps_result(lib):
    """W = K = 512 over an unconstrained 2048-code level: beams publish lower bounds of the
    512-th best key and later beams exit early; the result must not change."""
    C = 2048
    rng = np.random.default_rng(6)
    lps = [np.minimum(rng.standard_normal((512, C)).astype(np.float32) * 3 - 6, 0) for _ in range(3)]
    select_loop_vs_oracle(lib, [512], [512], C, 3, lambda d: lps[d], None, label="bound")


def test_wide_tie_plateau(lib):
    """Many equal keys at the cut: every candidate key equal, so the tie-break alone decides."""
    C = 700
    lps = [np.full((300, C), -1.0, np.float32) for _ in range(2)]
    select_loop_vs_oracle(lib, [300], [250], C, 2, lambda d: lps[d], None, label="plateau")


@pytest.mark.parametrize("case", ["trie", "unconstrained", "gumbel", "logits"])
def test_bound_wait_fallback_keeps_result(lib, case):
    """Beam workgroups of the fused pilot + per-beam kernel that stop waiting for their
    request's bound at once (wait limit 0) admit every candidate; rows with more than top_k of
    them go to the W-of-pool stage's overflow path.  The selection is unchanged: bit-exact
    against the oracle on every step."""
    rng = np.random.default_rng(21)
    S = 3
    if case == "trie":
        wl = workload("tiny")
        W, K, P = request_shapes(wl)
        items = catalog_items(wl)
        say("[select] wait limit 0: tiny trie")
        select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items,
                              label="wait0-trie", wait_limit=0)
        return
    W, K, C = [48, 64, 17], [48, 8, 17], 512
    x = [rng.normal(0.0, 3.0, size=(sum(W), C)) for _ in range(S)]
    lps = [np.minimum((v - np.log(np.exp(v).sum(axis=1, keepdims=True))).astype(np.float32), 0.0) for v in x]
    say(f"[select] wait limit 0: {case}")
    if case == "unconstrained":
        select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="wait0", wait_limit=0)
    elif case == "gumbel":
        g = [rng.gumbel(size=(sum(W), C)).astype(np.float32) for _ in range(S)]
        select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="wait0-gumbel", wait_limit=0,
                              noise_of_step=lambda d: g[d], temperature=1.0)
    else:
        raw = [v.astype(np.float32) for v in x]
        select_loop_vs_oracle(lib, W, K, C, S, lambda d: raw[d], None, label="wait0-logits", wait_limit=0,
                              raw_logits=True)


def test_wide_request_long_rows_with_pilot_bound(lib):
    """A request wider than the register-resident path's pilot capacity on the general
    kernels (W = 4500, top_k = 32, rows of 9000 codes): its own pilot set gives a bound, the
    rows stream through the LDS buffer in prefetched rounds, and the selection stays
    bit-exact; the bound keeps the pool far below W * top_k."""
    W, K, C, S = [4500], [32], 9000, 2
    rng = np.random.default_rng(31)
    lps = [np.minimum(rng.standard_normal((W[0], C)).astype(np.float32) * 3 - 9, 0) for _ in range(S)]
    say("[select] W = 4500, K = 32, C = 9000 (general kernels, fan-out first step)")
    loop, ws = select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="wide-long", fanout=True)
    assert int((loop.parents[1] >= 0).sum().item()) == W[0]
    assert loop.pool_sizes[0][-1] < W[0] * K[0] // 8, loop.pool_sizes


def test_ultra5000_select_at_its_shape(lib):
    """The ultra-wide workload's selection at its real shape: one request, W = 5000, top_k =
    64, unconstrained rows of 151936 codes (the general kernels: rows longer than 8192 codes,
    W > 1024, the wide pilot set).  Steps 0-3 take the live beams 1 -> 64 -> 4096 -> 5000 ->
    5000; every step is bit-exact against the oracle fed the checked state."""
    import synth.workloads as sw
    wl = workload("ultra5000")
    W, K, P = request_shapes(wl)
    th = oracle_threads()
    say(f"[select] ultra5000 shape: W={W[0]} K={K[0]} C={wl.C}, 4 steps, oracle on {th} threads")
    try:
        loop, ws = select_loop_vs_oracle(lib, W, K, wl.C, 4, lambda d: logprob_rows(wl, d, threads=th), None,
                                         label="ultra5000", threads=th)
    finally:
        sw._ultra_base.cache_clear()
    live = [int((loop.parents[d] >= 0).sum().item()) for d in range(4)]
    assert live == [64, 4096, 5000, 5000], live
