"""GPU parity of the first-step fan-out (beam_select_ex with first_step_fanout): the prompt
beam of each request expands to its best W_r children at the first step, the later steps
keep top_k.  The oracle is the selection with top_k = W_r at level 0.  Bit-exact tokens,
parents, score bits, order and trie nodes on ragged trie batches, the fused kernels (a row
of 8192 codes cut to 1024), the general kernels (W = 2048, rows longer than 8192 codes),
with Gumbel noise and from raw logits; wider than 2048 (the whole row through the pool);
refused when the row does not fit the pool."""
import numpy as np
import pytest
import torch

from synth import catalog_items, request_shapes, workload
from tests.gpu_util import make_ws, say, select_loop_vs_oracle

pytestmark = pytest.mark.gpu


def _lp(rng, n, C, sigma=2.0):
    x = rng.normal(0.0, sigma, size=(n, C))
    return np.minimum((x - np.log(np.exp(x).sum(axis=1, keepdims=True))).astype(np.float32), 0)


def _gumbel(rng, shape):
    u = rng.uniform(1e-12, 1.0, size=shape)
    return (-np.log(-np.log(u))).astype(np.float32)


def test_ragged_trie_batch(lib):
    wl = workload("qwen06b")
    items = catalog_items(wl)
    W, K = [64, 7, 200, 33], [8, 3, 16, 33]
    rng = np.random.default_rng(21)
    lps = [_lp(rng, sum(W), wl.C) for _ in range(wl.S)]
    say("[fanout] ragged trie batch")
    loop, ws = select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: lps[d], items, label="fanout-trie",
                                     fanout=True)
    # at the first step each prompt beam kept W_r candidates (its root has more children)
    assert [loop.pool_sizes[r][0] for r in range(len(W))] == W


def test_fused_path_unconstrained(lib):
    """W = 1024 of a row of 8192 codes: the row overflows and is cut to W by a radix select."""
    rng = np.random.default_rng(22)
    W, K, C, S = [1024], [4], 8192, 3
    lps = [_lp(rng, sum(W), C) for _ in range(S)]
    say("[fanout] fused W=1024")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="fanout-fused", fanout=True)


def test_general_kernels(lib):
    rng = np.random.default_rng(23)
    W, K, C, S = [2048], [2], 500, 3
    lps = [_lp(rng, sum(W), C) for _ in range(S)]
    say("[fanout] general W=2048")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="fanout-w2048", fanout=True)
    W, K, C = [256, 40], [4, 2], 20011
    lps = [_lp(rng, sum(W), C) for _ in range(S)]
    say("[fanout] long rows")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="fanout-long", fanout=True)


def test_gumbel_and_raw_logits(lib):
    wl = workload("qwen06b")
    items = catalog_items(wl)
    rng = np.random.default_rng(24)
    W, K = [100, 50], [10, 5]
    lps = [_lp(rng, sum(W), wl.C) for _ in range(wl.S)]
    gs = [_gumbel(rng, (sum(W), wl.C)) for _ in range(wl.S)]
    say("[fanout] gumbel")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: lps[d], items, label="fanout-g",
                          noise_of_step=lambda d: gs[d], temperature=1.0, fanout=True)
    xs = [rng.normal(0.0, 3.0, size=(sum(W), wl.C)).astype(np.float32) for _ in range(wl.S)]
    say("[fanout] raw logits")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: xs[d], items, label="fanout-x", raw_logits=True,
                          fanout=True)


def test_wider_than_the_per_beam_limit(lib):
    """W > 2048: the prompt beam keeps its whole row in the request's pool region and the
    W-of-pool stage cuts it to W (rows longer than 8192 codes, and shorter ones)."""
    rng = np.random.default_rng(25)
    for W, K, C in (([3000], [64], 20011), ([2500, 40], [4, 4], 6000)):
        lps = [_lp(rng, sum(W), C) for _ in range(2)]
        say(f"[fanout] W={W} K={K} C={C}")
        loop, ws = select_loop_vs_oracle(lib, W, K, C, 2, lambda d: lps[d], None, label=f"fanout-wide-{C}",
                                         fanout=True)
        assert loop.pool_sizes[0][0] == C


def test_width_above_limit_is_refused(lib):
    """A fan-out wider than 2048 whose row does not fit W * K pool entries is refused."""
    W, K, C = [3000], [2], 8000
    ws = make_ws(lib, W, K, [64], C=C, S=2)
    loop = lib.DecodeLoop(ws, 2, C, None, fanout=True)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    lp = torch.zeros(sum(W), C, device="cuda")
    with pytest.raises(lib.GrwError):
        loop.select_step(0, lp)
    loop.fanout = False
    loop.select_step(0, lp)          # the same step keeping top_k runs
    torch.cuda.synchronize()
    assert ws.error_flags() == 0
