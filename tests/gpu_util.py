"""Helpers shared by the GPU parity tests: upload synthetic inputs, drive the library
through its binding, and compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from oracle.attention import oracle_attention
from oracle.select import catalog_prefix_sets, initial_beams, oracle_select, oracle_select_logits
from synth import build_trie_csr


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_threads() -> int:
    """Threads for the oracle's per-beam loops: the host cores this process may use, at most
    16 (the share of one GPU's host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_ws(lib, Ws, Ks, Ps, *, C, S, Hq=16, Hkv=8, D=128, q_dtype="bf16", kv_dtype="bf16",
            max_splits=0):
    ws = lib.Workspace(max_requests=len(Ws), max_total_beams=int(sum(Ws)), max_W=int(max(Ws)),
                       max_K=int(max(Ks)), max_C=int(C), max_S=int(S), max_P=int(max(Ps)), Hq=Hq,
                       Hkv=Hkv, D=D, q_dtype=q_dtype, kv_dtype=kv_dtype, max_splits=max_splits)
    ws.bind_batch(Ws, Ks, Ps)
    return ws


def trie_device(trie, lib=None, C=None, dense_min_fanout=None):
    """Device CSR trie tuple; with dense_min_fanout also the dense child masks of the nodes
    with at least that many children (five-tuple)."""
    if trie is None:
        return None
    t = (torch.from_numpy(trie["row_ptr"]).cuda(), torch.from_numpy(trie["code"]).cuda(),
         int(trie["n_internal"]))
    if dense_min_fanout is None:
        return t
    slot, masks = lib.trie_dense_build(trie["row_ptr"], trie["code"], trie["n_internal"], C, dense_min_fanout)
    masks = masks if masks.size else np.zeros((1, (C + 31) // 32), np.uint32)
    return t + (torch.from_numpy(slot).cuda(), torch.from_numpy(masks.view(np.int32)).cuda())


def select_loop_vs_oracle(lib, Ws, Ks, C, S, lp_of_step, items=None, check=None, label="",
                          noise_of_step=None, temperature=0.0, raw_logits=False, dense_min_fanout=None,
                          fanout=False, wait_limit=None, threads=1):
    """Run S beam_select steps on the GPU (its own outputs feeding the next step) and compare
    every checked request bit-exactly with oracle_select at every step.  With noise_of_step,
    the steps are the Gumbel-sampled selection at the given temperature; with raw_logits,
    lp_of_step returns raw logits and the steps fuse their log-softmax; with fanout, the first
    step is the first-step fan-out, whose oracle is the selection with top_k = W; with
    wait_limit, the workspace's bound-wait limit; threads: the oracle's per-beam thread pool.
    Returns the loop."""
    Ws, Ks = list(map(int, Ws)), list(map(int, Ks))
    R = len(Ws)
    boff = np.concatenate([[0], np.cumsum(Ws)[:-1]]).astype(int)
    trie = build_trie_csr(items, C) if items is not None else None
    psets = catalog_prefix_sets(items, C) if items is not None else None
    ws = make_ws(lib, Ws, Ks, [64] * R, C=C, S=S)
    if wait_limit is not None:
        ws.set_wait_limit(wait_limit)
    loop = lib.DecodeLoop(ws, S, C, trie_device(trie, lib, C, dense_min_fanout), fanout=fanout)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    check = list(range(R)) if check is None else list(check)
    state = {r: initial_beams(Ws[r]) for r in check}
    pools = {}
    for d in range(S):
        lp = lp_of_step(d)
        g = noise_of_step(d) if noise_of_step is not None else None
        loop.select_step(d, torch.from_numpy(np.ascontiguousarray(lp)).cuda(),
                         noise=None if g is None else torch.from_numpy(np.ascontiguousarray(g)).cuda(),
                         temperature=temperature, raw_logits=raw_logits)
        torch.cuda.synchronize()
        tok = loop.tokens[d].cpu().numpy()
        par = loop.parents[d].cpu().numpy()
        sc = loop.scores[(d + 1) % 2].cpu().numpy()
        nd = loop.nodes[(d + 1) % 2].cpu().numpy()
        for r in check:
            a, W = boff[r], Ws[r]
            scores, prefixes = state[r]
            sel = oracle_select_logits if raw_logits else oracle_select
            res = sel(lp[a:a + W], scores, prefixes, d, W if fanout and d == 0 else Ks[r], W, C, psets,
                      None if g is None else g[a:a + W], temperature, **({"threads": threads} if not raw_logits else {}))
            where = f"{label} step {d} request {r}"
            np.testing.assert_array_equal(tok[a:a + W], res["tokens"], err_msg=where + " tokens")
            np.testing.assert_array_equal(par[a:a + W], res["parents"], err_msg=where + " parents")
            np.testing.assert_array_equal(sc[a:a + W].view(np.uint32), res["scores"].view(np.uint32),
                                          err_msg=where + " score bits")
            n = int((res["parents"] >= 0).sum())
            if trie is not None:
                got = trie["node_prefix"][nd[a:a + n]]
                want = np.array(res["prefixes"][:n], np.int64)
                np.testing.assert_array_equal(got, want, err_msg=where + " node prefixes")
                assert np.all(trie["node_depth"][nd[a:a + n]] == d + 1), where
            else:
                assert np.all(nd[a:a + W] == -1), where
            assert np.all(nd[a + n:a + W] == -1), where
            # the kept pool holds every winner and at most W * K entries
            pool = ws.pool_size(r)
            assert n <= pool <= W * (W if fanout and d == 0 else Ks[r]), f"{where}: pool {pool} for {n} winners"
            pools.setdefault(r, []).append(pool)
            state[r] = (res["scores"], res["prefixes"])
    flags = ws.error_flags()
    assert flags == 0, f"device flags {flags}"
    loop.pool_sizes = pools
    return loop, ws


def upload_layer(layer, wl_dtype_q, wl_dtype_kv, device="cuda", pad=0):
    """Synthetic layer (synth.attention_layer output) -> device tensors in library layout;
    ``pad`` fills the prompt storage padding."""
    lib_layout = sys.modules["generative_recommendation_wide_amd"]
    k_s, v_s = lib_layout.pack_shared_kv(layer["k_s"], layer["v_s"], wl_dtype_kv, device, pad=pad)
    out = dict(q=lib_layout.stored_tensor(layer["q"], wl_dtype_q, device),
               k_s=k_s, v_s=v_s,
               k_u=lib_layout.stored_tensor(layer["k_u"], wl_dtype_kv, device),
               v_u=lib_layout.stored_tensor(layer["v_u"], wl_dtype_kv, device),
               k_scale=None if layer["k_scale"] is None else torch.from_numpy(layer["k_scale"]).to(device),
               v_scale=None if layer["v_scale"] is None else torch.from_numpy(layer["v_scale"]).to(device))
    return out


def attention_vs_oracle(out_gpu, layer, parents, step, Ws, q_dtype, kv_dtype, samples, tol, label="", threads=1):
    """Compare sampled slots of the GPU output [sumW][Hq][D] with oracle_attention."""
    boff = np.concatenate([[0], np.cumsum(Ws)[:-1]]).astype(int)
    worst = 0.0
    for r, beams in samples.items():
        a, W = boff[r], Ws[r]
        beams = list(beams)
        if not beams:
            continue
        ref = oracle_attention(layer["q"][step][a:a + W], layer["k_s"][r], layer["v_s"][r],
                               layer["k_u"][:, a:a + W], layer["v_u"][:, a:a + W], parents[:, a:a + W],
                               step, q_dtype=q_dtype, kv_dtype=kv_dtype, k_scale=layer["k_scale"],
                               v_scale=layer["v_scale"], beams=beams, threads=threads)
        got = out_gpu[a + np.array(beams)].astype(np.float64)
        err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
        worst = max(worst, err)
        assert err <= tol, f"{label} request {r}: max abs error {err} > {tol}"
    return worst
