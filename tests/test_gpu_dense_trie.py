"""GPU parity of the selection with a dense-or-CSR trie (beam_select_ex with dense child masks
for the nodes of large fan-out) against the oracle, which decides validity from the raw item
list: bit-exact tokens, parents, score bits, order and trie nodes, for several fan-out
thresholds, with log-probabilities, raw logits and Gumbel noise."""
import numpy as np
import pytest

from synth import catalog_items, gumbel_rows, logit_rows, logprob_rows, request_shapes, workload
from tests.gpu_util import say, select_loop_vs_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,min_fanout", [("tiny", 1), ("tiny", 5), ("qwen06b", 100), ("qwen06b", 1)])
def test_workload_every_step(lib, name, min_fanout):
    wl = workload(name)
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say(f"[dense] {name} min_fanout={min_fanout}")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, label=f"{name}-dense",
                          dense_min_fanout=min_fanout)


def test_wide512_zipf(lib):
    wl = workload("wide512")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say("[dense] wide512 min_fanout=1024")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, check=[0, 2],
                          label="wide512-dense", dense_min_fanout=1024)


def test_logits_and_noise_with_dense_rows(lib):
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say("[dense] qwen06b logits + noise")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logit_rows(wl, d), items, label="qwen06b-dense-x",
                          raw_logits=True, dense_min_fanout=50)
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, label="qwen06b-dense-g",
                          noise_of_step=lambda d: gumbel_rows(wl, d), temperature=1.0, dense_min_fanout=50)


@pytest.mark.parametrize("seed", range(2))
def test_random_small_batches_with_ties(lib, seed):
    rng = np.random.default_rng(4000 + seed)
    C, L = int(rng.integers(33, 80)), 3
    items = np.unique(rng.integers(0, C, size=(int(rng.integers(50, 400)), L)), axis=0)
    Ws = rng.integers(1, 12, size=40)
    Ks = rng.integers(1, 12, size=40)
    sumW = int(Ws.sum())

    def lp(d):
        g = np.random.default_rng([seed, d, 9])
        return g.choice(np.array([0.0, -0.0, -0.5, -1.0, -np.inf], np.float32), size=(sumW, C))

    select_loop_vs_oracle(lib, Ws, Ks, C, L, lp, items, label=f"dense-ties{seed}", dense_min_fanout=3)
