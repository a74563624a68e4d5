"""Pins of the oracle beam attention (CPU only).

Each test ties oracle_attention to something other than itself:
closed forms, a library routine (torch scaled_dot_product_attention in float64), the
log-sum-exp merge identity of split attention, and a materialised reorder of the beam
caches (what a cache_select copy would produce) instead of the parent-pointer walk.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attend_concat, oracle_attention
from oracle.numformats import decode_stored


def _case(rng, W=5, Hq=4, Hkv=2, D=16, P=12, S=4, dead=()):
    q = rng.standard_normal((W, Hq, D)).astype(np.float32)
    ks = rng.standard_normal((Hkv, P, D)).astype(np.float32)
    vs = rng.standard_normal((Hkv, P, D)).astype(np.float32)
    ku = rng.standard_normal((S, W, Hkv, D)).astype(np.float32)
    vu = rng.standard_normal((S, W, Hkv, D)).astype(np.float32)
    par = rng.integers(0, W, size=(S, W)).astype(np.int32)
    for b in dead:
        par[:, b] = -1
    # live beams must have live ancestors
    live = [b for b in range(W) if b not in dead]
    for e in range(S):
        for b in range(W):
            if par[e, b] >= 0:
                par[e, b] = live[par[e, b] % len(live)]
    return q, ks, vs, ku, vu, par


def test_zero_keys_give_mean_of_values():
    rng = np.random.default_rng(0)
    q, ks, vs, ku, vu, par = _case(rng)
    ks[:] = 0
    ku[:] = 0
    step = 3
    out = oracle_attention(q, ks, vs, ku, vu, par, step, q_dtype="f32", kv_dtype="f32")
    g = 2
    for b in range(q.shape[0]):
        js = [0] * (step + 1)
        js[step] = b
        for e in range(step, 0, -1):
            js[e - 1] = par[e][js[e]]
        for h in range(q.shape[1]):
            rows = [vs[h // g, t] for t in range(vs.shape[1])] + [vu[e, js[e], h // g] for e in range(step + 1)]
            mean = np.mean(np.asarray(rows, np.float64), axis=0)
            np.testing.assert_allclose(out[b, h], mean, rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value_exactly():
    rng = np.random.default_rng(1)
    q, ks, vs, ku, vu, par = _case(rng, W=3, Hq=2, Hkv=1, D=8, P=6, S=2)
    q[:] = 1.0
    ks[:] = 0.0
    ku[:] = 0.0
    ks[0, 4, :] = 1000.0                # score 8000/sqrt(8) ~ 2828 above every other key
    out = oracle_attention(q, ks, vs, ku, vu, par, 1, q_dtype="f32", kv_dtype="f32")
    for b in range(3):
        for h in range(2):
            assert np.array_equal(out[b, h], vs[0, 4].astype(np.float64))


def test_two_point_softmax_closed_form():
    # P = 1, depth 0: two keys (the prompt token and the beam's own token)
    rng = np.random.default_rng(2)
    for _ in range(20):
        q, ks, vs, ku, vu, par = _case(rng, W=2, Hq=2, Hkv=2, D=4, P=1, S=1)
        out = oracle_attention(q, ks, vs, ku, vu, par, 0, q_dtype="f32", kv_dtype="f32")
        for b in range(2):
            for h in range(2):
                s1 = float(np.dot(q[b, h].astype(np.float64), ks[h, 0])) / 2.0
                s2 = float(np.dot(q[b, h].astype(np.float64), ku[0, b, h])) / 2.0
                sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
                ref = sig * vs[h, 0].astype(np.float64) + (1 - sig) * vu[0, b, h].astype(np.float64)
                np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-14)


def test_matches_torch_sdpa_float64_with_grouped_heads():
    rng = np.random.default_rng(3)
    for g in (1, 2, 4):
        Hkv = 2
        q, ks, vs, ku, vu, par = _case(rng, W=6, Hq=Hkv * g, Hkv=Hkv, D=32, P=40, S=3, dead=(5,))
        step = 2
        out = oracle_attention(q, ks, vs, ku, vu, par, step, q_dtype="f32", kv_dtype="f32")
        for b in range(5):
            js = [0] * (step + 1)
            js[step] = b
            for e in range(step, 0, -1):
                js[e - 1] = par[e][js[e]]
            kc = np.concatenate([ks, np.stack([ku[e, js[e]] for e in range(step + 1)], 1)], 1)
            vc = np.concatenate([vs, np.stack([vu[e, js[e]] for e in range(step + 1)], 1)], 1)
            K = torch.from_numpy(kc.astype(np.float64)).repeat_interleave(g, dim=0)
            V = torch.from_numpy(vc.astype(np.float64)).repeat_interleave(g, dim=0)
            Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, 0, :].numpy()
            np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
        assert np.all(out[5] == 0.0)        # dead slot


def _partial(qv, Kp, Vp):
    """(normalised output, natural-log sum-exp) of one head over a KV chunk, float64."""
    s = (Kp @ qv) / np.sqrt(np.float64(qv.size))
    m = s.max()
    p = np.exp(s - m)
    return (p @ Vp) / p.sum(), m + np.log(p.sum())


def _merge(parts):
    lses = np.array([l for _, l in parts])
    M = lses.max()
    w = np.exp(lses - M)
    return sum(wi * o for wi, (o, _) in zip(w, parts)) / w.sum()


def test_merge_of_split_attention_equals_unsplit():
    rng = np.random.default_rng(4)
    q, ks, vs, ku, vu, par = _case(rng, W=4, Hq=4, Hkv=2, D=16, P=50, S=4)
    step = 3
    out = oracle_attention(q, ks, vs, ku, vu, par, step, q_dtype="f32", kv_dtype="f32")
    for b in range(4):
        js = [0] * (step + 1)
        js[step] = b
        for e in range(step, 0, -1):
            js[e - 1] = par[e][js[e]]
        for h in range(4):
            kv = h // 2
            qv = q[b, h].astype(np.float64)
            Ku = np.stack([ku[e, js[e], kv] for e in range(step + 1)]).astype(np.float64)
            Vu = np.stack([vu[e, js[e], kv] for e in range(step + 1)]).astype(np.float64)
            # prompt split at random cut points, plus the ancestry part
            cuts = np.sort(rng.choice(np.arange(1, 50), size=rng.integers(0, 5), replace=False))
            bounds = [0, *cuts.tolist(), 50]
            parts = [_partial(qv, ks[kv, a:z].astype(np.float64), vs[kv, a:z].astype(np.float64))
                     for a, z in zip(bounds[:-1], bounds[1:])]
            parts.append(_partial(qv, Ku, Vu))
            np.testing.assert_allclose(_merge(parts), out[b, h], rtol=0, atol=1e-12)


def test_parent_walk_equals_materialised_reorder():
    """Gather through parent pointers == attention over per-beam copies built step by step
    the way a cache-select reorder would build them."""
    rng = np.random.default_rng(5)
    W, S = 7, 5
    q, ks, vs, ku, vu, par = _case(rng, W=W, Hq=2, Hkv=1, D=8, P=9, S=S)
    caches_k = [[] for _ in range(W)]
    caches_v = [[] for _ in range(W)]
    for step in range(S):
        # reorder: the new slot b inherits the cache of its parent, then appends its token
        if step > 0:
            caches_k = [list(caches_k[par[step, b]]) for b in range(W)]
            caches_v = [list(caches_v[par[step, b]]) for b in range(W)]
        for b in range(W):
            caches_k[b].append(ku[step, b])
            caches_v[b].append(vu[step, b])
        out = oracle_attention(q, ks, vs, ku, vu, par, step, q_dtype="f32", kv_dtype="f32")
        for b in range(W):
            kc = np.concatenate([ks[0], np.stack(caches_k[b])[:, 0]]).astype(np.float64)
            vc = np.concatenate([vs[0], np.stack(caches_v[b])[:, 0]]).astype(np.float64)
            for h in range(2):
                assert np.array_equal(attend_concat(q[b, h].astype(np.float64), kc, vc), out[b, h])


def test_fp8_and_bf16_inputs_decode_through_scales():
    rng = np.random.default_rng(6)
    W, Hq, Hkv, D, P, S = 3, 4, 2, 16, 20, 2
    q = torch.randn(W, Hq, D).to(torch.bfloat16)
    kv = [torch.randn(Hkv, P, D) for _ in range(2)] + [torch.randn(S, W, Hkv, D) for _ in range(2)]
    ksc = np.array([0.01, 0.02], np.float32)
    vsc = np.array([0.03, 0.005], np.float32)
    k8 = (kv[0] / torch.from_numpy(ksc)[:, None, None]).to(torch.float8_e4m3fn)
    v8 = (kv[1] / torch.from_numpy(vsc)[:, None, None]).to(torch.float8_e4m3fn)
    ku8 = (kv[2] / torch.from_numpy(ksc)[None, None, :, None]).to(torch.float8_e4m3fn)
    vu8 = (kv[3] / torch.from_numpy(vsc)[None, None, :, None]).to(torch.float8_e4m3fn)
    par = np.zeros((S, W), np.int32)
    par[1] = [2, 0, 1]
    as_u8 = lambda t: t.view(torch.uint8).numpy()
    out = oracle_attention(q.view(torch.int16).numpy().view(np.uint16), as_u8(k8), as_u8(v8),
                           as_u8(ku8), as_u8(vu8), par, 1, q_dtype="bf16", kv_dtype="fp8",
                           k_scale=ksc, v_scale=vsc)
    # same attention with every tensor decoded by torch and scaled in float64
    Kd = k8.to(torch.float64) * torch.from_numpy(ksc.astype(np.float64))[:, None, None]
    Vd = v8.to(torch.float64) * torch.from_numpy(vsc.astype(np.float64))[:, None, None]
    Kud = ku8.to(torch.float64) * torch.from_numpy(ksc.astype(np.float64))[None, None, :, None]
    Vud = vu8.to(torch.float64) * torch.from_numpy(vsc.astype(np.float64))[None, None, :, None]
    for b in range(W):
        js = [par[1][b], b]
        Kc = torch.cat([Kd, torch.stack([Kud[e, js[e]] for e in range(2)], 1)], 1)
        Vc = torch.cat([Vd, torch.stack([Vud[e, js[e]] for e in range(2)], 1)], 1)
        Q = q[b].to(torch.float64)[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, Kc.repeat_interleave(2, 0), Vc.repeat_interleave(2, 0))[:, 0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name,P,index,step", [("wide512", 64, 60, 2), ("ultra5000", 64, 61, 15)])
def test_short_prompt_cases_see_the_decode_tokens(name, P, index, step):
    """The GPU parity cases with a 64-token prompt (tests/test_gpu_attention.py) can tell a
    right answer from the mistakes the unshared stage and the merge could make: on the same
    inputs, a wrong ancestor at one depth, or the decode-token partial left out of the merge,
    moves the oracle's output by more than five times the 2e-2 tolerance on every sampled slot.
    (At the full 4096-token prompt the same mistakes stay below the tolerance.)"""
    import dataclasses

    from synth import attention_layer, random_parents, request_shapes, workload
    wl = dataclasses.replace(workload(name), P=P, layers=1, index=index)
    W, K, Ps = request_shapes(wl)
    shapes = (W, K, Ps)
    layer = attention_layer(wl, 0, shapes=shapes, requests=[0])
    par = random_parents(wl, shapes=shapes, dead_frac=0.05 if name == "wide512" else 0.0)
    Wr = int(W[0])
    rng = np.random.default_rng(9)
    beams = [int(b) for b in rng.choice(np.nonzero(par[step, :Wr] >= 0)[0], size=12, replace=False)]
    args = (layer["q"][step][:Wr], layer["k_s"][0], layer["v_s"][0], layer["k_u"][:, :Wr], layer["v_u"][:, :Wr])
    right = oracle_attention(*args, par[:, :Wr], step, q_dtype="bf16", kv_dtype="bf16", beams=beams)
    # a wrong ancestor: every parent pointer at depth `step` moved to another live slot
    wrong = par[:, :Wr].copy()
    live = np.nonzero(par[step - 1, :Wr] >= 0)[0] if step > 1 else np.arange(Wr)
    for b in beams:
        wrong[step, b] = int(live[(np.searchsorted(live, wrong[step, b]) + 1) % live.size])
    moved = oracle_attention(*args, wrong, step, q_dtype="bf16", kv_dtype="bf16", beams=beams)
    # the decode tokens left out: attention over the prompt alone
    prompt_only = np.stack([
        np.stack([attend_concat(decode_stored(args[0][b][h], "bf16"),
                                decode_stored(args[1][h // 2], "bf16"), decode_stored(args[2][h // 2], "bf16"))
                  for h in range(wl.Hq)]) for b in beams])
    d_anc = np.abs(moved - right).max(axis=(1, 2))
    d_merge = np.abs(prompt_only - right).max(axis=(1, 2))
    assert np.all(d_anc > 0.1), d_anc
    assert np.all(d_merge > 0.1), d_merge
