"""Slot-budget batching on the GPU: a queue of mixed-width requests packed by
grw_plan_batches (first fit in queue order under a beam-row budget) runs batch by batch
through ONE workspace, rebound per batch.  Every request's selection steps equal the
oracle's bit for bit, and its attention matches the oracle's within the fp8 tolerance,
whatever batch it lands in and whoever shares it.  Inputs are drawn once for the whole
queue and sliced per batch, so a request sees the same inputs in any packing."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle.attention import oracle_attention
from oracle.select import catalog_prefix_sets, initial_beams, oracle_select
from synth import attention_layer, build_trie_csr, catalog_items, logprob_rows, workload
from tests.gpu_util import say, trie_device, upload_layer

pytestmark = pytest.mark.gpu

BUDGET, MAX_REQ = 128, 5
TOL = 2e-2


def queue():
    rng = np.random.default_rng(2024)
    W = np.concatenate([rng.integers(2, 41, size=13), [100]]).astype(np.int32)
    rng.shuffle(W)
    P = rng.integers(64, 1200, size=W.size).astype(np.int32)
    return W, W.copy(), P


def test_packed_queue_matches_oracle_per_request(lib):
    W, K, P = queue()
    wl = dataclasses.replace(workload("mixed_fp8"), name="batching", index=61, n_requests=W.size, S=3,
                             C=512, catalog=("uniform", 30000))
    batch_of, nb = lib.plan_batches(W, BUDGET, MAX_REQ)
    say(f"[batching] {W.size} requests, sum W {int(W.sum())}, budget {BUDGET}: {nb} batches {batch_of.tolist()}")
    assert nb >= 3
    shapes = (W, K, P)
    layer = attention_layer(wl, 0, shapes=shapes)
    lps = [logprob_rows(wl, d, shapes=shapes) for d in range(wl.S)]
    items = catalog_items(wl)
    trie = build_trie_csr(items, wl.C)
    psets = catalog_prefix_sets(items, wl.C)
    boff_all = np.concatenate([[0], np.cumsum(W)[:-1]]).astype(int)
    ws = lib.Workspace(max_requests=MAX_REQ, max_total_beams=BUDGET, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=wl.C, max_S=wl.S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    rng = np.random.default_rng(5)
    worst = 0.0
    for b in range(nb):
        ids = np.flatnonzero(batch_of == b)
        Wb, Kb, Pb = W[ids], K[ids], P[ids]
        assert int(Wb.sum()) <= BUDGET and ids.size <= MAX_REQ
        slots = np.concatenate([np.arange(boff_all[i], boff_all[i] + W[i]) for i in ids])
        lb = dict(q=layer["q"][:, slots], k_s=[layer["k_s"][i] for i in ids], v_s=[layer["v_s"][i] for i in ids],
                  k_u=layer["k_u"][:, slots], v_u=layer["v_u"][:, slots], k_scale=layer["k_scale"],
                  v_scale=layer["v_scale"])
        ws.bind_batch(Wb, Kb, Pb)
        dev = upload_layer(lb, wl.q_dtype, wl.kv_dtype)
        loop = lib.DecodeLoop(ws, wl.S, wl.C, trie_device(trie))
        ws.beams_init(loop.scores[0], loop.nodes[0])
        out = torch.empty(int(Wb.sum()), wl.Hq, wl.D, dtype=torch.float32, device="cuda")
        boff = np.concatenate([[0], np.cumsum(Wb)[:-1]]).astype(int)
        state = {j: initial_beams(int(Wb[j])) for j in range(ids.size)}
        for d in range(wl.S):
            lp = np.ascontiguousarray(lps[d][slots])
            loop.select_step(d, torch.from_numpy(lp).cuda())
            lib.beam_attn_decode(ws, dev["q"][d], dev["k_s"], dev["v_s"], dev["k_scale"], dev["v_scale"],
                                 dev["k_u"], dev["v_u"], loop.parents, d, out)
            torch.cuda.synchronize()
            tok, par = loop.tokens[d].cpu().numpy(), loop.parents[: d + 1].cpu().numpy()
            sc = loop.scores[(d + 1) % 2].cpu().numpy()
            o = out.cpu().numpy()
            for j, i in enumerate(ids):
                a, w = boff[j], int(Wb[j])
                res = oracle_select(lp[a:a + w], *state[j], d, int(Kb[j]), w, wl.C, psets)
                where = f"batch {b} request {i} step {d}"
                np.testing.assert_array_equal(tok[a:a + w], res["tokens"], err_msg=where)
                np.testing.assert_array_equal(par[d, a:a + w], res["parents"], err_msg=where)
                np.testing.assert_array_equal(sc[a:a + w].view(np.uint32), res["scores"].view(np.uint32),
                                              err_msg=where)
                state[j] = (res["scores"], res["prefixes"])
                live = np.flatnonzero(res["parents"] >= 0)
                assert np.all(o[a + np.setdiff1d(np.arange(w), live)] == 0.0), where
                beams = live if live.size <= 6 else rng.choice(live, size=6, replace=False)
                if beams.size == 0:
                    continue
                parents = np.zeros((wl.S, w), np.int32)
                parents[: d + 1] = par[:, a:a + w]
                ref = oracle_attention(lb["q"][d][a:a + w], lb["k_s"][j], lb["v_s"][j], lb["k_u"][:, a:a + w],
                                       lb["v_u"][:, a:a + w], parents, d, q_dtype=wl.q_dtype,
                                       kv_dtype=wl.kv_dtype, k_scale=lb["k_scale"], v_scale=lb["v_scale"],
                                       beams=list(beams))
                err = float(np.max(np.abs(o[a + beams].astype(np.float64) - ref)))
                worst = max(worst, err)
                assert err <= TOL, f"{where}: attention max abs error {err}"
        assert ws.error_flags() == 0
    say(f"[batching] every request matches the oracle; worst attention error {worst:.3e}")
