"""GPU parity of beam_select_gumbel (the Gumbel top-k selection at a positive temperature)
against the oracle: bit-exact tokens, parents, score bits, order and trie nodes, on the
synthetic workloads, the general kernels (W > 1024, rows longer than the one-pass length)
and tie-heavy batches; temperature 0 equals beam_select; non-finite noise is flagged."""
import numpy as np
import pytest
import torch

from synth import catalog_items, gumbel_rows, logprob_rows, request_shapes, workload
from tests.gpu_util import make_ws, say, select_loop_vs_oracle, trie_device

pytestmark = pytest.mark.gpu


def _gumbel(rng, shape):
    u = rng.uniform(1e-12, 1.0, size=shape)
    return (-np.log(-np.log(u))).astype(np.float32)


@pytest.mark.parametrize("name,temp", [("tiny", 1.0), ("qwen06b", 1.0), ("qwen06b", 0.3)])
def test_workload_every_step(lib, name, temp):
    wl = workload(name)
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say(f"[gumbel] {name} T={temp}")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, label=f"{name}-g",
                          noise_of_step=lambda d: gumbel_rows(wl, d), temperature=temp)


def test_wide512_unconstrained(lib):
    wl = workload("wide512u")
    W, K, P = request_shapes(wl)
    say("[gumbel] wide512u")
    loop, ws = select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), None, check=[2],
                                     label="wide512u-g", noise_of_step=lambda d: gumbel_rows(wl, d),
                                     temperature=1.0)
    assert loop.pool_sizes[2][-1] < int(W[2]) * int(K[2]) // 4, loop.pool_sizes


def test_wide512_zipf_trie(lib):
    wl = workload("wide512")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    say("[gumbel] wide512")
    select_loop_vs_oracle(lib, W, K, wl.C, wl.S, lambda d: logprob_rows(wl, d), items, check=[1],
                          label="wide512-g", noise_of_step=lambda d: gumbel_rows(wl, d), temperature=0.7)


def test_general_kernels(lib):
    """W > 1024 (pilot, per-beam and global kernels) and rows longer than 8192 codes
    (streamed through the LDS buffer), with noise."""
    rng = np.random.default_rng(11)
    W, K, C, S = [1200, 1100], [16, 3], 500, 3
    lps = [rng.normal(0.0, 2.0, size=(sum(W), C)) for _ in range(S)]
    lps = [np.minimum((x - np.log(np.exp(x).sum(axis=1, keepdims=True))).astype(np.float32), 0) for x in lps]
    gs = [_gumbel(rng, (sum(W), C)) for _ in range(S)]
    say("[gumbel] W > 1024")
    select_loop_vs_oracle(lib, W, K, C, S, lambda d: lps[d], None, label="wide-multi-g",
                          noise_of_step=lambda d: gs[d], temperature=1.5)
    C = 20011
    Ws, Ks = [7, 33], [3, 64]
    lps = [np.minimum(rng.standard_normal((sum(Ws), C)).astype(np.float32) * 2, 0) for _ in range(3)]
    gs = [_gumbel(rng, (sum(Ws), C)) for _ in range(3)]
    say("[gumbel] long rows")
    select_loop_vs_oracle(lib, Ws, Ks, C, 3, lambda d: lps[d], None, label="long-g",
                          noise_of_step=lambda d: gs[d], temperature=0.5)


@pytest.mark.parametrize("seed", range(2))
def test_random_small_batches_with_ties(lib, seed):
    """Ragged batches of small requests; log-probabilities and noise from small value sets so
    that perturbed keys tie often; -0.0 and -inf included."""
    rng = np.random.default_rng(2000 + seed)
    C = int(rng.integers(2, 40))
    L = 3
    items = np.unique(rng.integers(0, C, size=(int(rng.integers(5, 300)), L)), axis=0)
    R = 40
    Ws = rng.integers(1, 12, size=R)
    Ks = rng.integers(1, 12, size=R)
    sumW = int(Ws.sum())

    def lp(d):
        g = np.random.default_rng([seed, d, 1])
        return g.choice(np.array([0.0, -0.0, -0.5, -1.0, -np.inf], np.float32), size=(sumW, C))

    def noise(d):
        g = np.random.default_rng([seed, d, 2])
        return g.choice(np.array([0.0, -0.0, 0.5, -1.0, 2.0], np.float32), size=(sumW, C))

    select_loop_vs_oracle(lib, Ws, Ks, C, L, lp, items, label=f"ties{seed}", noise_of_step=noise, temperature=0.5)
    select_loop_vs_oracle(lib, Ws, Ks, C, L, lp, None, label=f"ties{seed}u", noise_of_step=noise, temperature=1.0)


def test_temperature_zero_equals_beam_select(lib):
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    trie = trie_device(__import__("synth").build_trie_csr(catalog_items(wl), wl.C))
    outs = []
    for sampled in (False, True):
        ws = make_ws(lib, W, K, P, C=wl.C, S=wl.S)
        loop = lib.DecodeLoop(ws, wl.S, wl.C, trie)
        ws.beams_init(loop.scores[0], loop.nodes[0])
        for d in range(wl.S):
            lp = torch.from_numpy(logprob_rows(wl, d)).cuda()
            g = torch.from_numpy(gumbel_rows(wl, d)).cuda() if sampled else None
            loop.select_step(d, lp, noise=g, temperature=0.0)
        torch.cuda.synchronize()
        outs.append([loop.tokens.clone(), loop.parents.clone(), loop.final_scores().view(torch.int32).clone(),
                     loop.final_nodes().clone()])
        assert ws.error_flags() == 0
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_bad_noise_is_flagged_and_bad_temperature_rejected(lib):
    wl = workload("tiny")
    W, K, P = request_shapes(wl)
    ws = make_ws(lib, W, K, P, C=wl.C, S=wl.S)
    loop = lib.DecodeLoop(ws, wl.S, wl.C, None)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    lp = torch.from_numpy(logprob_rows(wl, 0)).cuda()
    g = torch.from_numpy(gumbel_rows(wl, 0)).cuda()
    with pytest.raises(lib.GrwError):
        loop.select_step(0, lp, noise=g, temperature=-1.0)
    with pytest.raises(lib.GrwError):
        loop.select_step(0, lp, noise=g, temperature=float("inf"))
    g[0, 3] = float("nan")
    loop.select_step(0, lp, noise=g, temperature=1.0)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_BAD_NOISE
