"""GPU parity of beam_select_logits (the selection from raw logits with the row log-softmax
fused in) against the oracle: bit-exact tokens, parents, score bits, order and trie nodes,
on the synthetic workloads, the general kernels (W > 1024, rows longer than the one-pass
length), masked logits, the sampled variant, and a precondition flag."""
import numpy as np
import pytest
import torch

from synth import catalog_items, gumbel_rows, logit_rows, request_shapes, workload
from tests.gpu_util import make_ws, say, select_loop_vs_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "qwen06b"])
def test_workload_every_step(lib, name):
    wl = workload(name)
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say(f"[logits] {name}")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logit_rows(wl, d), items, label=f"{name}-x",
                          raw_logits=True)


def test_wide512_unconstrained_and_trie(lib):
    wl = workload("wide512u")
    W, K, P = request_shapes(wl)
    say("[logits] wide512u")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logit_rows(wl, d), None, check=[0], label="wide512u-x",
                          raw_logits=True)
    wl = workload("wide512")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say("[logits] wide512")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logit_rows(wl, d), items, check=[3], label="wide512-x",
                          raw_logits=True)


def test_sampled_from_logits(lib):
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say("[logits] qwen06b sampled")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logit_rows(wl, d), items, label="qwen06b-xg",
                          noise_of_step=lambda d: gumbel_rows(wl, d), temperature=1.0, raw_logits=True)


def test_general_kernels_and_masked_logits(lib):
    """W > 1024 and rows longer than 8192 codes take the lse kernel, then the general
    kernels; some logits are -inf (masked codes)."""
    rng = np.random.default_rng(21)
    W, K, C, S = [1100, 1300], [16, 5], 600, 3
    xs = []
    for _ in range(S):
        x = (rng.standard_normal((sum(W), C)) * 3).astype(np.float32)
        x[rng.random(x.shape) < 0.2] = -np.inf
        x[:, 0] = 0.0                           # every row keeps a finite logit
        xs.append(x)
    say("[logits] W > 1024")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: xs[d], None, label="wide-multi-x", raw_logits=True)
    C = 20011
    Ws, Ks = [9, 40], [4, 100]
    xs = [(rng.standard_normal((sum(Ws), C)) * 2).astype(np.float32) for _ in range(3)]
    say("[logits] long rows")
    select_loop_vs_oracle(lib, Ws, Ks, C, 3, lambda d: xs[d], None, label="long-x", raw_logits=True)


def test_random_small_batches(lib):
    """Ragged batches of small requests with trie constraints; logits on a coarse grid so
    that log-probabilities tie."""
    rng = np.random.default_rng(3000)
    C, L = 23, 3
    items = np.unique(rng.integers(0, C, size=(200, L)), axis=0)
    Ws = rng.integers(1, 12, size=40)
    Ks = rng.integers(1, 12, size=40)
    sumW = int(Ws.sum())

    def x(d):
        g = np.random.default_rng([d, 5])
        return g.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.5, -np.inf], np.float32), size=(sumW, C))

    select_loop_vs_oracle(lib, Ws, Ks, C, L, x, items, label="small-x", raw_logits=True)
    select_loop_vs_oracle(lib, Ws, Ks, C, L, x, None, label="small-xu", raw_logits=True)


def test_nan_logit_flagged(lib):
    wl = workload("tiny")
    W, K, P = request_shapes(wl)
    ws = make_ws(lib, W, K, P, C=wl.C, S=wl.S)
    loop = lib.DecodeLoop(ws, wl.S, wl.C, None)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    x = torch.from_numpy(logit_rows(wl, 0)).cuda()
    x[0, 5] = float("nan")
    loop.select_step(0, x, raw_logits=True)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_NAN_LOGPROB
