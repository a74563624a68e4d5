#!/usr/bin/env python3
"""Throughput of the wide-beam decode step on one MI355X.

One bench step = one pass of the whole hot path over one batch: the device-resident
S-step decode loop (per decode step: beam_select for every request, then
beam_attn_decode for every layer), ending with the semantic-ID backtrack.  The reported
value is beam decode steps per second (S decode steps per bench step).

Default workload "wide512": 4 requests, beam_width = top_k = 512 (262144-candidate pools),
prompt 4096, 16 query / 8 kv heads, head dim 128, 28 layers, bf16 KV, 3 decode steps over
8192-code levels constrained by a 4M-item Zipf(1.1) catalog trie.  Inputs are synthetic
(seeded), generated on the device in the library's storage layout before timing.

Usage:  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wide512]
        python bench.py --summarize DIR   (rocprofv3 output -> profiles/*.md summaries)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
N_SIMDS = 1024                # 256 CUs x 4 SIMDs
N_XCDS = 8                    # GRBM_GUI_ACTIVE comes back summed over the XCDs
DOMINANT = "attn_shared_split_kernel"
_CSRC = "generative_recommendation_wide_amd/csrc/"
KERNEL_SOURCES = [_CSRC + "attn_shared.hip", _CSRC + "device_common.h", _CSRC + "grw_internal.h"]
SELECT_SOURCES = [_CSRC + "select.hip", _CSRC + "device_common.h", _CSRC + "grw_internal.h"]
# counter records: (kernels whose dispatches are summed, sources whose hash the record carries)
TRAFFIC = {
    "shared": (os.path.join(ROOT, "profiles", "attn_shared_split_wide512_traffic.txt"), [DOMINANT], KERNEL_SOURCES,
               "wide512: one layer, 4 requests, W=K=512, P=4096",
               "--steps 1 --warmup 1 --stage-reps 0"),
    "select": (os.path.join(ROOT, "profiles", "beam_select_wide512u_traffic.txt"),
               ["select_pilot_beam_kernel", "select_final_kernel"], SELECT_SOURCES,
               "wide512u: one beam_select call, 4 requests, W=K=512, 8192 codes, every beam live, rows not in cache",
               "--select-only --stage-reps 1"),
}
TRAFFIC_FILE = TRAFFIC["shared"][0]
MFMA_FILE = os.path.join(ROOT, "profiles", "attn_shared_split_wide512_mfma.txt")
N_COLD_SETS = 8               # select inputs rotated per call: 8 x 64 MiB > the 256 MB last-level cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------------------
# workload setup (device-side synthetic inputs in the library's storage layout)
# ----------------------------------------------------------------------------------------
def setup(wl, seed, dev):
    import numpy as np
    import torch

    import generative_recommendation_wide_amd as grw
    from synth import build_trie_csr, catalog_items, request_shapes

    W, K, P = request_shapes(wl, seed)
    sumW, S, C = int(W.sum()), wl.S, wl.C
    Pp = ((P + 63) // 64) * 64
    kv_elems = int(wl.Hkv * wl.D * Pp.sum())
    g = torch.Generator(device=dev).manual_seed(seed)

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32)

    def kv_store(x, scale=None):
        if wl.kv_dtype == "bf16":
            return x.to(torch.bfloat16)
        if wl.kv_dtype == "fp8":
            return (x / scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        return x

    layers = []
    for _ in range(wl.layers):
        q = randn(S, sumW, wl.Hq, wl.D).to(torch.bfloat16 if wl.q_dtype == "bf16" else torch.float32)
        ks, vs = randn(kv_elems), randn(kv_elems)
        ku, vu = randn(S, sumW, wl.Hkv, wl.D), randn(S, sumW, wl.Hkv, wl.D)
        k_scale = v_scale = None
        if wl.kv_dtype == "fp8":
            # per kv head scales (amax / 448) over this layer's prompt and decode KV
            def head_amax(flat, u):
                m = u.abs().amax(dim=(0, 1, 3))
                off = 0
                for p in Pp.tolist():
                    blk = flat[off:off + wl.Hkv * p * wl.D].view(wl.Hkv, -1).abs().amax(dim=1)
                    m = torch.maximum(m, blk)
                    off += wl.Hkv * p * wl.D
                return m
            k_scale = (head_amax(ks, ku) / 448.0).float()
            v_scale = (head_amax(vs, vu) / 448.0).float()
            # broadcast scale over the packed layout: [Hkv][...] blocks per request
            def scale_flat(x, sc):
                out, off = [], 0
                for p in Pp.tolist():
                    n = wl.Hkv * p * wl.D
                    out.append(kv_store(x[off:off + n].view(wl.Hkv, -1), sc[:, None]).reshape(-1))
                    off += n
                return torch.cat(out)
            ks_s, vs_s = scale_flat(ks, k_scale), scale_flat(vs, v_scale)
            ku_s = kv_store(ku, k_scale[None, None, :, None])
            vu_s = kv_store(vu, v_scale[None, None, :, None])
        else:
            ks_s, vs_s, ku_s, vu_s = kv_store(ks), kv_store(vs), kv_store(ku), kv_store(vu)
        layers.append(dict(q=q, k_s=ks_s, v_s=vs_s, k_u=ku_s, v_u=vu_s, k_scale=k_scale, v_scale=v_scale))
        del ks, vs, ku, vu
    lps = []
    for _ in range(S):
        x = torch.randn(sumW, C, generator=g, device=dev, dtype=torch.float64) * wl.logit_sigma
        lps.append(torch.log_softmax(x, dim=-1).to(torch.float32).clamp_max_(0.0))
        del x
    trie = t = None
    items = catalog_items(wl, seed)
    if items is not None:
        t = build_trie_csr(items, C)
        trie = (torch.from_numpy(t["row_ptr"]).to(dev), torch.from_numpy(t["code"]).to(dev), t["n_internal"])
    ws = grw.Workspace(max_requests=len(W), max_total_beams=sumW, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=C, max_S=S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    ws.bind_batch(W, K, P)
    loop = grw.DecodeLoop(ws, S, C, trie, device=dev)
    out = torch.empty(sumW, wl.Hq, wl.D, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    return dict(W=W, K=K, P=P, ws=ws, loop=loop, layers=layers, lps=lps, out=out, trie=trie, trie_host=t)


def shared_stage_work(wl, st):
    """Algorithmic flops and bytes of one shared-stage launch (one layer, all requests)."""
    W, P = st["W"], st["P"]
    ws = st["ws"]
    esz = {"bf16": 2, "fp8": 1, "f32": 4}[wl.kv_dtype]
    qsz = 2 if wl.q_dtype == "bf16" else 4
    flops = sum(4.0 * int(W[r]) * wl.Hq * int(P[r]) * wl.D for r in range(len(W)))
    bytes_ = sum(2.0 * wl.Hkv * int(P[r]) * wl.D * esz            # K and V prompt tiles, once
                 + int(W[r]) * wl.Hq * wl.D * qsz                 # queries
                 + ws.splits(r) * int(W[r]) * wl.Hq * (wl.D + 1) * 4   # partial o + lse
                 for r in range(len(W)))
    return flops, bytes_


def time_stage(fn, n_launch, stream):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()                                   # warm
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_launch):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_launch   # ms per call


def time_graph(fn, n_launch, stream, replays=3):
    """Device time per call of fn: a HIP graph of n_launch calls (no host work between the
    kernels), replayed `replays` times between HIP events on the launch stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n_launch):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (replays * n_launch)


def stage_timings(wl, st, reps):
    """Per-call device time of each stage at the last depth, every layer in turn: HIP graphs of
    the stage's launches replayed between HIP events on the launch stream (so host launch
    gaps between short kernels do not count)."""
    import torch

    import generative_recommendation_wide_amd as grw
    stream = torch.cuda.current_stream()
    loop, layers, out, ws = st["loop"], st["layers"], st["out"], st["ws"]
    d = wl.S - 1
    res = {}
    for name, mask in (("shared", grw.STAGE_SHARED),
                       ("unshared_merge_fused", grw.STAGE_UNSHARED | grw.STAGE_MERGE),
                       ("unshared", grw.STAGE_UNSHARED), ("merge", grw.STAGE_MERGE)):
        def fn(mask=mask):
            for L in layers:
                grw.beam_attn_decode_stages(ws, L["q"][d], L["k_s"], L["v_s"], L["k_scale"], L["v_scale"],
                                            L["k_u"], L["v_u"], loop.parents, d, out, mask)
        res[name] = time_graph(fn, reps, stream) / len(layers)

    def sel_all():
        ws.beams_init(loop.scores[0], loop.nodes[0])
        for dd in range(wl.S):
            loop.select_step(dd, st["lps"][dd])
    res["select_loop_3steps"] = time_graph(sel_all, reps, stream)
    return res


def dense_sweep(seed, dev, reps=10):
    """The wide512 3-step select loop (Zipf trie) with a CSR-only trie and with dense child
    masks for the nodes of at least `threshold` children: device time per loop (HIP graph of
    `reps` loops, best of 5 replays), and whether the outputs equal the CSR-only ones."""
    import numpy as np
    import torch

    import generative_recommendation_wide_amd as grw
    from synth import build_trie_csr, catalog_items, request_shapes, workload
    wl = workload("wide512")
    W, K, P = request_shapes(wl, seed)
    sumW, C, S = int(W.sum()), wl.C, wl.S
    g = torch.Generator(device=dev).manual_seed(seed)
    lps = []
    for _ in range(S):
        x = torch.randn(sumW, C, generator=g, device=dev, dtype=torch.float64) * wl.logit_sigma
        lps.append(torch.log_softmax(x, dim=-1).to(torch.float32).clamp_max_(0.0))
        del x
    t = build_trie_csr(catalog_items(wl, seed), C)
    base = (torch.from_numpy(t["row_ptr"]).to(dev), torch.from_numpy(t["code"]).to(dev), t["n_internal"])
    fan = np.diff(t["row_ptr"][: t["n_internal"] + 1])
    ws = grw.Workspace(max_requests=len(W), max_total_beams=sumW, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=C, max_S=S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    ws.bind_batch(W, K, P)
    rows, ref = [], None
    for thr in (None, 4096, 1024, 256):
        trie = base
        if thr is not None:
            slot, masks = grw.trie_dense_build(t["row_ptr"], t["code"], t["n_internal"], C, thr)
            trie = base + (torch.from_numpy(slot).to(dev), torch.from_numpy(masks.view(np.int32)).to(dev))
        loop = grw.DecodeLoop(ws, S, C, trie, device=dev)

        def run():
            ws.beams_init(loop.scores[0], loop.nodes[0])
            for d in range(S):
                loop.select_step(d, lps[d])
        run()
        torch.cuda.synchronize()
        out = (loop.tokens.clone(), loop.parents.clone(), loop.final_scores().view(torch.int32).clone())
        ref = out if ref is None else ref
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(5):
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        del graph
        rows.append({"min_fanout": thr, "dense_nodes": int((fan >= thr).sum()) if thr else 0,
                     "us_per_3step_loop": round(min(ts) * 1e3, 1),
                     "equal_to_csr": bool(all(torch.equal(a, b) for a, b in zip(out, ref)))})
    flags = ws.error_flags()
    ws.close()
    return {"workload": "wide512", "select_loops": rows, "device_flags": flags}


def overlap_timings(wl, st, steps):
    """The two-stream attention (unshared stage on a side stream beside the shared stage,
    merge after both) against the default path (shared stage, then the unshared stage with
    the merge fused in): per-layer attention at the last depth (HIP graph of every layer,
    4 times, best of 5 replays) and the whole decode loop as a replayed graph."""
    import torch

    import generative_recommendation_wide_amd as grw
    ws, loop, layers, out, lps = st["ws"], st["loop"], st["layers"], st["out"], st["lps"]
    loop2 = grw.DecodeLoop(ws, wl.S, wl.C, st["trie"], device=out.device, overlap=True)
    loop2.run(lps, layers, out)
    torch.cuda.synchronize()
    d = wl.S - 1
    res = {}
    for name, lp in (("fused", loop), ("overlap", loop2)):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(4):
                for L in layers:
                    lp.attn_step(d, L, out)
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / (4 * len(layers)))
        res[f"{name}_attention_us_per_layer"] = round(min(ts), 2)
        del graph
    graph = loop2.capture(lps, layers, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    res["overlap_graph_replay_value"] = round(wl.S * steps / (time.perf_counter() - t0), 2)
    del graph, loop2
    return res


def fanout_bench(seed, dev, steps=3, reps=10):
    """First-step fan-out on the ultra-wide shape (W = 5000, top_k = 64, 151936-token rows,
    no trie): the first step expanding the prompt beam to its best 5000 children against
    the plain first step (top_k = 64).  Device time of the first step and of the first
    `steps` steps (HIP graphs, best of 5 replays of `reps` loops), and the live beams after
    each step."""
    import torch

    import generative_recommendation_wide_amd as grw
    from synth import request_shapes, workload
    wl = workload("ultra5000")
    W, K, P = request_shapes(wl, seed)
    sumW, C = int(W.sum()), wl.C
    g = torch.Generator(device=dev).manual_seed(seed)
    lps = []
    for _ in range(steps):
        x = torch.randn(sumW, C, generator=g, device=dev, dtype=torch.float32) * wl.logit_sigma
        lps.append(torch.log_softmax(x.double(), dim=-1).to(torch.float32).clamp_max_(0.0))
        del x
    ws = grw.Workspace(max_requests=len(W), max_total_beams=sumW, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=C, max_S=wl.S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    ws.bind_batch(W, K, P)
    rows = []
    for fan in (False, True):
        loop = grw.DecodeLoop(ws, wl.S, C, None, device=dev, fanout=fan)
        res = {"first_step": "fan-out to W" if fan else "top_k"}
        for n in (1, steps):
            def run(n=n):
                ws.beams_init(loop.scores[0], loop.nodes[0])
                for d in range(n):
                    loop.select_step(d, lps[d])
            run()
            torch.cuda.synchronize()
            if n == steps:
                res["live_beams_after_each_step"] = [int((loop.parents[d] >= 0).sum().item()) for d in range(steps)]
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    run()
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / reps)
            res[f"us_first_{n}_steps"] = round(min(ts), 1)
            del graph
        rows.append(res)
        del loop
    flags = ws.error_flags()
    ws.close()
    return {"workload": "ultra5000 (select only)", "beam_width": int(W.max()), "top_k": int(K.max()),
            "codes": C, "variants": rows, "device_flags": flags}


def batching_bench(seed, dev, budget=4096, max_requests=128):
    """The ragged fp8 workload's queue (101 requests: widths 2..100 and one of 1000, top_k =
    width, prompts 512..8192, 4 steps, one layer, 4-level trie of 2M items) run batch by batch
    through one workspace, rebound per batch: packed by grw_plan_batches (first fit in queue
    order under a beam-row slot budget) against one request per batch.  Per batch, the S-step
    loop (select, then attention) is timed by HIP events; binds are host work outside them.
    The rate is beam-row steps per second of device time; both packings must give every
    request the same tokens, parents and scores."""
    import numpy as np
    import torch

    import generative_recommendation_wide_amd as grw
    from synth import build_trie_csr, catalog_items, request_shapes, workload
    wl = workload("mixed_fp8")
    W, K, P = request_shapes(wl, seed)
    n, S, C = len(W), wl.S, wl.C
    Pp = ((P + 63) // 64) * 64
    g = torch.Generator(device=dev).manual_seed(seed)

    def fp8(*shape):
        x = torch.randn(*shape, generator=g, device=dev) * 64.0
        return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)

    q = [torch.randn(S, int(w), wl.Hq, wl.D, generator=g, device=dev).to(torch.bfloat16) for w in W]
    ku = [fp8(S, int(w), wl.Hkv, wl.D) for w in W]
    vu = [fp8(S, int(w), wl.Hkv, wl.D) for w in W]
    ks = [fp8(wl.Hkv * int(p) * wl.D) for p in Pp]
    vs = [fp8(wl.Hkv * int(p) * wl.D) for p in Pp]
    lps = []
    for w in W:
        x = torch.randn(S, int(w), C, generator=g, device=dev, dtype=torch.float64) * wl.logit_sigma
        lps.append(torch.log_softmax(x, dim=-1).to(torch.float32).clamp_max_(0.0))
    k_scale = torch.full((wl.Hkv,), 1.0 / 64.0, device=dev)
    v_scale = torch.full((wl.Hkv,), 1.0 / 64.0, device=dev)
    t = build_trie_csr(catalog_items(wl, seed), C)
    trie = (torch.from_numpy(t["row_ptr"]).to(dev), torch.from_numpy(t["code"]).to(dev), t["n_internal"])
    ws = grw.Workspace(max_requests=max_requests, max_total_beams=budget, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=C, max_S=S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    rows, results = [], []
    for name, mr in ((f"first fit, {budget} slots", max_requests), ("one request per batch", 1)):
        batch_of, nb = grw.plan_batches(W, budget, mr)
        dev_ms, per_req = 0.0, {}
        t_wall = time.perf_counter()
        for b in range(nb):
            ids = np.flatnonzero(batch_of == b).tolist()
            ws.bind_batch(W[ids], K[ids], P[ids])
            qb = torch.cat([q[i] for i in ids], dim=1)
            kub, vub = torch.cat([ku[i] for i in ids], dim=1), torch.cat([vu[i] for i in ids], dim=1)
            ksb, vsb = torch.cat([ks[i] for i in ids]), torch.cat([vs[i] for i in ids])
            lpb = [torch.cat([lps[i][d] for i in ids]) for d in range(S)]
            out = torch.empty(qb.shape[1], wl.Hq, wl.D, dtype=torch.float32, device=dev)
            loop = grw.DecodeLoop(ws, S, C, trie, device=dev)
            layer = dict(q=qb, k_s=ksb, v_s=vsb, k_u=kub, v_u=vub, k_scale=k_scale, v_scale=v_scale)
            ms = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                loop.run(lpb, [layer], out)
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            dev_ms += min(ms[1:])
            tok, par = loop.tokens.cpu(), loop.parents.cpu()
            sc = loop.final_scores().view(torch.int32).cpu()
            off = 0
            for i in ids:
                w = int(W[i])
                per_req[i] = (tok[:, off:off + w].clone(), par[:, off:off + w].clone(), sc[off:off + w].clone())
                off += w
            del qb, kub, vub, ksb, vsb, lpb, out, loop
        wall = time.perf_counter() - t_wall
        rows.append({"policy": name, "batches": int(nb), "device_ms": round(dev_ms, 3),
                     "wall_ms_incl_binds": round(wall * 1e3, 1),
                     "beam_row_steps_per_s": round(float(W.sum()) * S / (dev_ms / 1e3), 1)})
        results.append(per_req)
    same = all(all(torch.equal(a, b) for a, b in zip(results[0][i], results[1][i])) for i in range(n))
    flags = ws.error_flags()
    ws.close()
    return {"workload": "mixed_fp8 queue", "requests": n, "sum_W": int(W.sum()), "slot_budget": budget,
            "max_requests": max_requests, "policies": rows,
            "speedup_packed_vs_one_per_batch": round(rows[1]["device_ms"] / rows[0]["device_ms"], 2),
            "same_results_both_packings": bool(same), "device_flags": flags}


def select_roofline(seed, dev, reps, temperature=None, raw_logits=False, warm=True):
    """beam_select on the unconstrained wide-pool workload (4 requests, W = K = 512, 8192 codes,
    262144-entry pools): device time of one call with every beam live (the third decode step,
    beams from two real selections), against the HBM time of its algorithmic bytes: every
    beam's log-probability row, the beam scores, and the four output arrays.  Timed cold:
    a HIP graph of `reps` calls that rotate over N_COLD_SETS distinct row sets (512 MiB in
    all, more than the 256 MB last-level cache, so every call reads its rows from HBM); and
    warm: the same number of calls on one 64 MiB set.  With a temperature, beam_select_gumbel
    with standard Gumbel noise rows (one more row per beam in the algorithmic bytes).  With
    raw_logits, beam_select_logits on the raw logit rows (the log-softmax fused in; the same
    algorithmic bytes), and beside it the time of torch's float32 log_softmax followed by
    beam_select.  warm=False (counter runs) makes only cold calls."""
    import torch

    import generative_recommendation_wide_amd as grw
    from synth import request_shapes, workload
    wl = workload("wide512u")
    W, K, P = request_shapes(wl, seed)
    sumW, C = int(W.sum()), wl.C
    g = torch.Generator(device=dev).manual_seed(seed + 1)

    def rows():
        x = torch.randn(sumW, C, generator=g, device=dev, dtype=torch.float64) * wl.logit_sigma
        return x.to(torch.float32) if raw_logits else torch.log_softmax(x, dim=-1).to(torch.float32).clamp_max_(0.0)

    def gumbel():
        if temperature is None:
            return None
        u = torch.rand(sumW, C, generator=g, device=dev, dtype=torch.float64).clamp_(1e-300, 1.0 - 1e-16)
        return (-torch.log(-torch.log(u))).to(torch.float32)

    lps = [rows() for _ in range(2)]
    noise = [gumbel() for _ in range(2)]
    ws = grw.Workspace(max_requests=len(W), max_total_beams=sumW, max_W=int(W.max()), max_K=int(K.max()),
                       max_C=C, max_S=wl.S, max_P=int(P.max()), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype)
    ws.bind_batch(W, K, P)
    loop = grw.DecodeLoop(ws, wl.S, C, None, device=dev)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    loop.select_step(0, lps[0], noise=noise[0], temperature=temperature or 0.0, raw_logits=raw_logits)
    loop.select_step(1, lps[1], noise=noise[1], temperature=temperature or 0.0, raw_logits=raw_logits)
    sc, nd = loop.scores[0].clone(), loop.nodes[0].clone()     # step-2 input beams
    del lps, noise
    sets = [(rows(), gumbel()) for _ in range(N_COLD_SETS)]    # the step-2 rows: N_COLD_SETS draws
    live = int((sc > float("-inf")).sum())
    tok, par = torch.empty(sumW, dtype=torch.int32, device=dev), torch.empty(sumW, dtype=torch.int32, device=dev)
    osc, ond = torch.empty(sumW, dtype=torch.float32, device=dev), torch.empty(sumW, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    Wm, Km = int(W.max()), int(K.max())

    def call(i):
        x, gn = sets[i % N_COLD_SETS]
        if raw_logits:
            grw.beam_select_logits(ws, x, gn, temperature or 0.0, sc, nd, None, None, 0, Wm, Km, C, tok, par, osc, ond)
        elif temperature is None:
            grw.beam_select(ws, x, sc, nd, None, None, 0, Wm, Km, C, tok, par, osc, ond)
        else:
            grw.beam_select_gumbel(ws, x, gn, temperature, sc, nd, None, None, 0, Wm, Km, C, tok, par, osc, ond)

    ms_eager = time_stage(lambda: call(0), reps, stream) if warm else float("nan")
    refs = []
    for i in range(N_COLD_SETS):
        call(i)
        torch.cuda.synchronize()
        refs.append((tok.clone(), par.clone(), osc.clone()))
    pools = [ws.pool_size(r) for r in range(len(W))]   # after the last set's call

    def graph_ms(which):
        """Device time per call of a captured graph of `reps` calls on sets which(i) (the select
        kernels record no memset nodes), and whether its last call's outputs equal the eager
        ones."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                call(which(i))
        graph.replay()
        torch.cuda.synchronize()
        tok.fill_(-7)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ref = refs[which(reps - 1) % N_COLD_SETS]
        same = bool(torch.equal(tok, ref[0]) and torch.equal(par, ref[1]) and
                    torch.equal(osc.view(torch.int32), ref[2].view(torch.int32)))
        del graph
        return e0.elapsed_time(e1) / (3 * reps), same

    ms_cold, same_cold = graph_ms(lambda i: i)
    ms_warm, same_warm = graph_ms(lambda i: 0) if warm else (float("nan"), True)
    unfused = None
    if raw_logits and temperature is None:
        lp_buf = torch.empty_like(sets[0][0])

        def fn2():
            torch.log_softmax(sets[0][0], dim=-1, out=lp_buf)
            grw.beam_select(ws, lp_buf, sc, nd, None, None, 0, Wm, Km, C, tok, par, osc, ond)
        unfused = time_stage(fn2, reps, stream) * 1e3
    bytes_ = sumW * C * 4.0 * (1 if temperature is None else 2) + sumW * 4.0 + sumW * 16.0
    t = ms_cold / 1e3
    achieved = bytes_ / t / 1e9
    traffic = read_traffic("select") if temperature is None and not raw_logits else None
    ws.close()
    del sets
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "workload": "wide512u",
            "live_beams": live, "bytes_per_call": bytes_, "avg_call_us": round(t * 1e6, 2),
            "warm_call_us": round(ms_warm * 1e3, 2), "warm_frac": round(bytes_ / (ms_warm / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "eager_call_us": round(ms_eager * 1e3, 2), "graph_matches_eager": same_cold and same_warm,
            "pool_after_pruning": pools, "pool_unpruned": int(W[0]) * int(K[0]),
            "timing": (f"HIP graph of {reps} calls replayed 3 times; cold: the calls rotate over {N_COLD_SETS} "
                       f"distinct 64 MiB row sets ({N_COLD_SETS * 64} MiB); warm: one set"),
            "kernels": "select_pilot_beam_kernel + select_final_kernel",
            "entry_point": ("beam_select_logits" if raw_logits else "beam_select_gumbel" if temperature is not None
                            else "beam_select") + ("" if temperature is None else f" (temperature {temperature})"),
            "unfused_log_softmax_then_select_us": None if unfused is None else round(unfused, 2)}


def measured_ceilings(dev):
    """Achievable ceilings measured on this GPU beside the spec peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and a hipBLASLt bf16 GEMM of 8192^3 through
    torch.matmul (a plain library GEMM, measurement only)."""
    import torch
    n = (1 << 30) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * 4 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    z = torch.matmul(x, y)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        z = torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * m ** 3 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e12
    del x, y, z
    res = {"hbm_copy_GBs": round(copy_gbs, 1), "hbm_copy_frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
           "bf16_gemm_TFLOPs": round(gemm_tf, 1), "bf16_gemm_frac_of_peak": round(gemm_tf / PEAK_BF16_TFLOPS, 4),
           "how": "1 GiB torch copy_ (2 x bytes / time), 10 reps; torch.matmul bf16 8192^3 (hipBLASLt), 10 reps"}
    res.update(mfma_ceiling(dev))
    return res


def mfma_ceiling(dev, launches=8, iters=20000):
    """Dense bf16 MFMA rate of the whole chip under sustained load, from the probe in
    libgrw_ceiling.so: one 4-wave workgroup per CU, 8 independent 32x32x16 accumulations per
    wave, `launches` back-to-back launches (about 20 ms; the clock ramps up over the first
    ones, so the rate is the last launch's).  Also that launch's shader clock (s_memtime
    cycles over s_memrealtime 100 MHz ticks, median over workgroups) and the dense peak at that
    clock (1024 flops per SIMD and cycle, 1024 SIMDs).  With every matrix pipe busy the chip
    clocks down well below the 2.4 GHz of the spec peak; a kernel that keeps the pipes busy
    part of the time runs at a higher clock, so its MFMA busy fraction (counters) is the
    cycle-level measure."""
    import ctypes

    import numpy as np
    import torch
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "generative_recommendation_wide_amd",
                        "libgrw_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP libraries first")
    lib = ctypes.CDLL(path)
    lib.grw_ceiling_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.grw_ceiling_mfma_per_round.restype = ctypes.c_int
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    ts = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    if lib.grw_ceiling_mfma(blocks, iters, out.data_ptr(), ts.data_ptr(), sp) != 0:
        raise RuntimeError("grw_ceiling_mfma failed")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    ev[0].record(stream)
    for j in range(launches):
        if lib.grw_ceiling_mfma(blocks, iters, out.data_ptr(), ts.data_ptr(), sp) != 0:
            raise RuntimeError("grw_ceiling_mfma failed")
        ev[j + 1].record(stream)
    torch.cuda.synchronize()
    per_round = lib.grw_ceiling_mfma_per_round()
    mfmas_per_wave = per_round * iters
    flops = 32768.0 * mfmas_per_wave * 4 * blocks
    # the clock ramps up under sustained load: everything is taken from the last launch.  The
    # rate is over the workgroups' own span (first loop start to last loop end, 100 MHz
    # s_memrealtime): the launch as HIP events see it is about 1 ms longer whatever its length
    # (a fixed per-launch cost outside the loops), which is no property of the MFMA pipes.
    t = ts.cpu().numpy().reshape(blocks, 4).astype(np.float64)
    span_us = float(t[:, 3].max() - t[:, 2].min()) / 100.0
    tf = flops / (span_us / 1e6) / 1e12
    ghz = float(np.median(t[:, 0] / (t[:, 1] * 10.0)))
    cyc = float(np.median(t[:, 0] / mfmas_per_wave))
    dur_us = t[:, 1] / 100.0
    peak_at_clock = 1024.0 * 1024 * ghz * 1e9 / 1e12
    return {"mfma_bf16_TFLOPs": round(tf, 1), "mfma_bf16_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "mfma_cycles_per_32x32x16": round(cyc, 2), "shader_clock_GHz_under_mfma_load": round(ghz, 3),
            "workgroup_loop_us_min_median_max": [round(float(dur_us.min()), 1), round(float(np.median(dur_us)), 1),
                                                 round(float(dur_us.max()), 1)],
            "first_start_to_last_end_us": round(span_us, 1),
            "launch_us_hip_events": round(ev[launches - 1].elapsed_time(ev[launches]) * 1e3, 1),
            "dense_bf16_peak_at_that_clock_TFLOPs": round(peak_at_clock, 1),
            "mfma_how": (f"libgrw_ceiling.so probe: {blocks} workgroups x 4 waves, {per_round} independent "
                         f"32x32x16 bf16 accumulations per wave, {iters} rounds, {launches} launches back to back; "
                         "rate over the last launch's workgroup span (s_memrealtime, 100 MHz), clock = s_memtime "
                         "cycles / s_memrealtime ticks of its loops")}


def unshared_roofline(wl, st, t_ms):
    """The fused unshared + merge kernel at the last depth against HBM: algorithmic bytes from
    the loop's actual parent pointers (queries of live slots, the distinct decode-token rows
    reachable from them, the parent pointers on the walks, the shared partials, the outputs)
    over the kernel's measured time per launch."""
    import numpy as np
    par = st["loop"].parents.cpu().numpy()
    W, ws = st["W"], st["ws"]
    d = wl.S - 1
    kvb = {"bf16": 2, "fp8": 1, "f32": 4}[wl.kv_dtype]
    qb = 2 if wl.q_dtype == "bf16" else 4
    boff = np.concatenate([[0], np.cumsum(W)[:-1]]).astype(int)
    live = nodes = walk_ptrs = 0
    part = 0.0
    for r, w in enumerate(W):
        p = par[:, boff[r]:boff[r] + int(w)]
        cur = np.nonzero(p[d] >= 0)[0]
        live += cur.size
        part += ws.splits(r) * cur.size * wl.Hq * (wl.D + 1) * 4.0
        for e in range(d, -1, -1):
            cur = np.unique(cur)
            nodes += cur.size
            if e > 0:
                walk_ptrs += cur.size
                cur = p[e][cur]
                cur = cur[cur >= 0]
    sumW = int(W.sum())
    bytes_ = (live * wl.Hq * wl.D * qb + nodes * 2.0 * wl.Hkv * wl.D * kvb + (sumW + walk_ptrs) * 4.0 + part
              + sumW * wl.Hq * wl.D * 4.0)
    t = t_ms / 1e3
    return {"bound": "hbm", "achieved": round(bytes_ / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(bytes_ / t / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
            "kernel": "attn_unshared_kernel (merge fused)", "depth": d, "live_slots": live,
            "distinct_decode_rows": nodes, "bytes_per_launch": bytes_, "avg_launch_us": round(t * 1e6, 2)}


def select_loop_roofline(wl, st, t_ms):
    """The decode loop's selections (every step, every request, on the catalog trie) against
    HBM: algorithmic bytes are the 128-byte lines of each live beam's log-probability row that
    hold its trie children (all lines when unconstrained), the CSR codes of those rows, the
    beam state and the outputs; over the measured time of the S-step selection loop."""
    import numpy as np
    import torch
    loop, ws, lps = st["loop"], st["ws"], st["lps"]
    trie = st.get("trie_host")
    sumW = int(st["W"].sum())
    ws.beams_init(loop.scores[0], loop.nodes[0])
    lines = codes = 0
    for d in range(wl.S):
        sc = loop.scores[d % 2].cpu().numpy()
        nd = loop.nodes[d % 2].cpu().numpy()
        for b in np.nonzero(np.isfinite(sc))[0]:
            if trie is None:
                lines += (wl.C * 4 + 127) // 128
            else:
                row = trie["code"][trie["row_ptr"][nd[b]]:trie["row_ptr"][nd[b] + 1]]
                lines += np.unique(row // 32).size
                codes += row.size
        loop.select_step(d, lps[d])
    torch.cuda.synchronize()
    bytes_ = lines * 128.0 + codes * 4.0 + wl.S * sumW * (8.0 + 16.0)
    t = t_ms / 1e3
    return {"bound": "hbm", "achieved": round(bytes_ / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(bytes_ / t / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
            "what": f"{wl.S}-step selection loop of the decode loop ({wl.name}, catalog trie)",
            "lines_128B": int(lines), "csr_codes": int(codes), "bytes_per_loop": bytes_,
            "loop_us": round(t * 1e6, 2)}


# ----------------------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample of the same workload
# ----------------------------------------------------------------------------------------
def oracle_cores() -> int:
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, seed):
    """The oracle on this host's cores (BLAS at one thread; the oracle's per-beam loops on a
    thread pool of one thread per core) on a bounded sample of the workload: every request's
    selection over all S steps, and the attention of request 0's slots at the last depth on one
    layer; scaled to every request, beam and layer of a decode step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.attention import oracle_attention
    from oracle.select import catalog_prefix_sets, initial_beams, oracle_select
    from synth import attention_layer, catalog_items, logprob_rows, random_parents, request_shapes

    n = oracle_cores()
    W, K, P = request_shapes(wl, seed)
    R = len(W)
    items = catalog_items(wl, seed)
    psets = catalog_prefix_sets(items, wl.C) if items is not None else None
    boff = np.concatenate([[0], np.cumsum(W)[:-1]]).astype(int)
    with threadpool_limits(limits=1):
        t_sel = 0.0
        lps = [logprob_rows(wl, d, seed) for d in range(wl.S)]
        for r in range(R):
            scores, prefixes = initial_beams(int(W[r]))
            for d in range(wl.S):
                lp = lps[d][boff[r]:boff[r] + int(W[r])]
                t0 = time.perf_counter()
                res = oracle_select(lp, scores, prefixes, d, int(K[r]), int(W[r]), wl.C, psets, threads=n)
                t_sel += time.perf_counter() - t0
                scores, prefixes = res["scores"], res["prefixes"]
        del lps
        layer = attention_layer(wl, 0, seed, requests=[0])
        par = random_parents(wl, seed)
        W0 = int(W[0])
        nb = min(W0, 512)
        d = wl.S - 1
        t0 = time.perf_counter()
        oracle_attention(layer["q"][d][:W0], layer["k_s"][0], layer["v_s"][0], layer["k_u"][:, :W0],
                         layer["v_u"][:, :W0], par[:, :W0], d, q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype,
                         k_scale=layer["k_scale"], v_scale=layer["v_scale"], beams=range(nb), threads=n)
        t_attn_beam = (time.perf_counter() - t0) / nb
    sumW = int(W.sum())
    t_step = t_sel / wl.S + sumW * wl.layers * t_attn_beam
    return {"value": 1.0 / t_step, "unit": "beam decode steps/s", "cores": n, "kind": "oracle",
            "sample": (f"oracle_select on all {R} requests over all {wl.S} steps ({t_sel:.2f} s) and "
                       f"oracle_attention on {nb} slots of request 0, layer 0, depth {d} "
                       f"({t_attn_beam * 1e3:.2f} ms per slot); scaled to {sumW} slots x {wl.layers} layers per "
                       f"decode step; {n} threads (per-beam thread pool), BLAS at 1 thread")}


def cpu_full(name, seed):
    """The oracle on a whole small workload, in full: every request, every decode step (the
    selection, then every layer's attention of every slot at that depth with the parents the
    selection chose), on this host's cores.  Returns decode steps per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.attention import oracle_attention
    from oracle.select import catalog_prefix_sets, initial_beams, oracle_select
    from synth import attention_layer, catalog_items, logprob_rows, request_shapes, workload

    wl = workload(name)
    n = oracle_cores()
    W, K, P = request_shapes(wl, seed)
    items = catalog_items(wl, seed)
    psets = catalog_prefix_sets(items, wl.C) if items is not None else None
    boff = np.concatenate([[0], np.cumsum(W)[:-1]]).astype(int)
    lps = [logprob_rows(wl, d, seed) for d in range(wl.S)]
    layers = [attention_layer(wl, li, seed) for li in range(wl.layers)]
    total = 0.0
    with threadpool_limits(limits=1):
        for r in range(len(W)):
            a, w = boff[r], int(W[r])
            scores, prefixes = initial_beams(w)
            par = np.full((wl.S, w), -1, np.int32)
            for d in range(wl.S):
                t0 = time.perf_counter()
                res = oracle_select(lps[d][a:a + w], scores, prefixes, d, int(K[r]), w, wl.C, psets, threads=n)
                scores, prefixes = res["scores"], res["prefixes"]
                par[d] = res["parents"]
                for L in layers:
                    oracle_attention(L["q"][d][a:a + w], L["k_s"][r], L["v_s"][r], L["k_u"][:, a:a + w],
                                     L["v_u"][:, a:a + w], par, d, q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype,
                                     k_scale=L["k_scale"], v_scale=L["v_scale"], threads=n)
                total += time.perf_counter() - t0
    return {"workload": name, "value": round(wl.S / total, 4), "unit": "beam decode steps/s", "cores": n,
            "seconds": round(total, 2), "requests": len(W), "slots": int(W.sum()), "steps": wl.S,
            "layers": wl.layers}


def _read_record(path, sources):
    """key = value lines of a counter record, or None when it is missing or was taken from
    other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != kernel_source_sha(sources):
        return None
    return kv


def read_traffic(target="shared"):
    path, _, sources, _, _ = TRAFFIC[target]
    kv = _read_record(path, sources)
    try:
        return None if kv is None else float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma():
    kv = _read_record(MFMA_FILE, KERNEL_SOURCES)
    if kv is None:
        return None
    try:
        return {k: float(kv[k]) for k in ("mfma_busy", "coexec_of_mfma_busy", "valu_per_mfma", "lds_bank_conflict_cycles",
                                          "mfma_insts")}
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------------------
# rocprofv3 summaries
# ----------------------------------------------------------------------------------------
def _short_kernel_name(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:                      # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def summarize(args):
    """Turn rocprofv3 CSV output into short text summaries under profiles/."""
    import csv
    d = args.summarize
    out_lines = []
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        out_lines.append(f"## kernel stats ({os.path.relpath(f, d)})\n")
        out_lines.append("| kernel | calls | total ms | avg us | min us | max us | % |")
        out_lines.append("|---|---|---|---|---|---|---|")
        for r in rows:
            short = _short_kernel_name(r.get("Name", ""))
            out_lines.append(f"| {short[:80]} | {r.get('Calls')} | {float(r.get('TotalDurationNs', 0)) / 1e6:.3f} | "
                             f"{float(r.get('AverageNs', 0)) / 1e3:.2f} | {float(r.get('MinNs', 0)) / 1e3:.2f} | "
                             f"{float(r.get('MaxNs', 0)) / 1e3:.2f} | {float(r.get('Percentage', 0)):.2f} |")
    counters = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    agg = {}
    for f in counters:
        for r in csv.DictReader(open(f)):
            name = _short_kernel_name(r.get("Kernel_Name", ""))
            key = (name, r.get("Counter_Name"))
            a = agg.setdefault(key, [0.0, 0])
            a[0] += float(r.get("Counter_Value", 0))
            a[1] += 1
    if agg:
        out_lines.append("\n## counters (per dispatch average)\n")
        out_lines.append("| kernel | counter | dispatches | avg value |")
        out_lines.append("|---|---|---|---|")
        for (k, c), (s, n) in sorted(agg.items()):
            out_lines.append(f"| {k[:80]} | {c} | {n} | {s / n:.1f} |")
    text = "\n".join(out_lines) + "\n"
    if args.summary_out:
        with open(args.summary_out, "w") as f:
            f.write(args.summary_header.replace("\\n", "\n") + "\n" + text if args.summary_header else text)
    print(text)


def _counter_rows(d):
    import csv
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(f[0])))


def write_traffic(args):
    """HBM bytes per launch (per call for the selection: its kernels' dispatches summed) from
    two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the calibration copy (the largest copyBuffer dispatch, of
    --calib-copy-mib MiB)."""
    fetch_dir, write_dir = args.traffic
    path, kernels, sources, what, flags = TRAFFIC[args.traffic_target]
    calib_kib = args.calib_copy_mib * 1024.0

    def per_dispatch(d, counter):
        per_k = {k: [] for k in kernels}
        copies = []
        for r in _counter_rows(d):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            for k in kernels:
                if k in r["Kernel_Name"]:
                    per_k[k].append(v)
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(v)
        # the median dispatch: the selection's first step (one live beam per request) and any
        # other odd dispatch do not move it
        return {k: sorted(v)[len(v) // 2] for k, v in per_k.items()}, max(copies)

    fk, fcal = per_dispatch(fetch_dir, "FETCH_SIZE")
    wk, wcal = per_dispatch(write_dir, "WRITE_SIZE")
    ff, wf = calib_kib / fcal, calib_kib / wcal
    total = (sum(fk.values()) * ff + sum(wk.values()) * wf) * 1024.0
    lines = [
        f"# HBM traffic of {' + '.join(kernels)} per launch ({what})",
        "# Commands (repo root on the GPU box, TMPDIR=/tmp), one counter per run:",
        "#   rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv -- "
        f"python3 bench.py {flags} --no-cpu-baseline --counter-run --calib-copy-mib {args.calib_copy_mib}",
        "#   (same with --pmc WRITE_SIZE -d gpurun_out/pmc_write)",
        f"#   python bench.py --traffic gpurun_out/pmc_fetch gpurun_out/pmc_write --traffic-target {args.traffic_target} "
        f"--calib-copy-mib {args.calib_copy_mib}",
        f"# calibration: a {args.calib_copy_mib} MiB device copy reads FETCH_SIZE={fcal:.1f} KiB and WRITE_SIZE={wcal:.1f} KiB,",
        f"# so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {wf:.4f}.",
    ]
    for k in kernels:
        lines.append(f"# {k}: FETCH_SIZE {fk[k]:.1f} KiB, WRITE_SIZE {wk[k]:.1f} KiB per dispatch (raw, median)")
    lines += [
        f"fetch_kib_raw={sum(fk.values()):.1f}",
        f"write_kib_raw={sum(wk.values()):.1f}",
        f"fetch_scale={ff:.4f}",
        f"write_scale={wf:.4f}",
        f"hbm_bytes_per_launch={total:.0f}",
        f"source_sha={kernel_source_sha(sources)}",
    ]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_mfma(args):
    """MFMA utilisation of the dominant kernel from two rocprofv3 --pmc runs (per dispatch):
    run 1 SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE,
    run 2 SQ_INSTS_VALU SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES GRBM_GUI_ACTIVE.  MFMA busy = busy
    cycles (counted per SIMD, summed over the chip's SIMDs) / (SIMDs x active GPU cycles of one
    XCD; GRBM_GUI_ACTIVE is reported summed over the 8 XCDs)."""
    vals = {}
    for d in args.mfma:
        acc = {}
        for r in _counter_rows(d):
            if DOMINANT not in r["Kernel_Name"]:
                continue
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, v in acc.items():
            vals.setdefault(k, []).extend(v)
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    xcd_cycles = avg["GRBM_GUI_ACTIVE"] / N_XCDS
    busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMDS * xcd_cycles)
    lines = [
        f"# MFMA counters of {DOMINANT} per dispatch (wide512: one layer, 4 requests, W=K=512, P=4096)",
        "# Commands (repo root on the GPU box, TMPDIR=/tmp):",
        "#   rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE "
        "-d gpurun_out/pmc_mfma1 -o run --output-format csv -- python3 bench.py --steps 1 --warmup 1 --stage-reps 0 "
        "--no-cpu-baseline --counter-run",
        "#   rocprofv3 --pmc SQ_INSTS_VALU SQ_LDS_BANK_CONFLICT SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -d gpurun_out/pmc_mfma2 ...",
        "#   python bench.py --mfma gpurun_out/pmc_mfma1 gpurun_out/pmc_mfma2",
        "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); coexec_of_mfma_busy =",
        "# SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA",
    ]
    for k in sorted(avg):
        lines.append(f"# {k}: {avg[k]:.1f}")
    lines += [
        f"# active cycles per XCD: {xcd_cycles:.0f} ({xcd_cycles / 2.4e3:.1f} us at 2.4 GHz)",
        f"mfma_insts={avg['SQ_INSTS_MFMA']:.0f}",
        f"mfma_busy={busy:.4f}",
        f"coexec_of_mfma_busy={avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.4f}",
        f"valu_per_mfma={avg.get('SQ_INSTS_VALU', float('nan')) / avg['SQ_INSTS_MFMA']:.3f}",
        f"lds_bank_conflict_cycles={avg.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f}",
        f"source_sha={kernel_source_sha(KERNEL_SOURCES)}",
    ]
    with open(MFMA_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def calib_copy(args, dev):
    """One device copy of --calib-copy-mib MiB (the counters' calibration dispatch)."""
    if not args.calib_copy_mib:
        return
    import torch
    n = args.calib_copy_mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


# ----------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wide512")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=3)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--select-only", action="store_true",
                    help="only the beam_select measurement on the unconstrained wide pool (for kernel traces)")
    ap.add_argument("--select-temperature", type=float, default=None,
                    help="with --select-only: time beam_select_gumbel at this temperature")
    ap.add_argument("--select-logits", action="store_true",
                    help="with --select-only: time beam_select_logits on raw logits")
    ap.add_argument("--dense-sweep", action="store_true",
                    help="time the wide512 select loop with dense child masks at several fan-out thresholds")
    ap.add_argument("--batching", action="store_true",
                    help="run the ragged fp8 queue packed under a slot budget and one request per batch")
    ap.add_argument("--fanout", action="store_true",
                    help="time the first-step fan-out against the plain first step on the ultra-wide shape")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--traffic", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--traffic-target", default="shared", choices=sorted(TRAFFIC))
    ap.add_argument("--mfma", nargs="+", default=None, metavar="PMC_DIR",
                    help="write the dominant kernel's MFMA counter record from rocprofv3 --pmc output")
    ap.add_argument("--counter-run", action="store_true",
                    help="short run for rocprofv3 counters: no graph replays, no two-stream timing, cold selection "
                         "calls only")
    ap.add_argument("--no-cpu-full", action="store_true",
                    help="skip the oracle's full runs of the two small workloads")
    ap.add_argument("--summary-out", default=None)
    ap.add_argument("--summary-header", default="")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return 0
    if args.traffic:
        write_traffic(args)
        return 0
    if args.mfma:
        write_mfma(args)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode step shards by request, with no exchange, and multi-GPU runs are not "
              "part of this build", file=sys.stderr)
        return 2

    import torch

    from synth import workload
    wl = workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dense_sweep:
        print(json.dumps(dense_sweep(args.seed, dev)), flush=True)
        return 0
    if args.fanout:
        print(json.dumps(fanout_bench(args.seed, dev)), flush=True)
        return 0
    if args.batching:
        print(json.dumps(batching_bench(args.seed, dev)), flush=True)
        return 0
    if args.select_only:
        print(json.dumps(select_roofline(args.seed, dev, 16 * max(1, args.stage_reps),
                                         temperature=args.select_temperature, raw_logits=args.select_logits,
                                         warm=not args.counter_run)),
              flush=True)
        calib_copy(args, dev)
        return 0
    log(f"[bench] setting up {wl.name} ...")
    t_setup = time.perf_counter()
    st = setup(wl, args.seed, dev)
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; warmup {args.warmup}, timed {args.steps}")
    loop, layers, out, lps = st["loop"], st["layers"], st["out"], st["lps"]
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        loop.run(lps, layers, out)
    torch.cuda.synchronize()
    flags = st["ws"].error_flags()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        loop.run(lps, layers, out)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = e0.elapsed_time(e1) / 1000.0
    log(f"[bench] timed {args.steps} steps: wall {wall * 1e3:.2f} ms, events {ev * 1e3:.2f} ms")
    decode_steps = wl.S * args.steps
    value = decode_steps / wall
    graph_value = overlap = None
    if not args.counter_run:
        # the same loop captured as one HIP graph and replayed (no host work between kernels)
        graph = loop.capture(lps, layers, out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        del graph
        graph_value = round(decode_steps / graph_wall, 2)
        log(f"[bench] graph replay of {args.steps} steps: wall {graph_wall * 1e3:.2f} ms")
        overlap = overlap_timings(wl, st, args.steps)
        log(f"[bench] two-stream attention: {overlap}")
    if args.stage_reps > 0:
        stages = stage_timings(wl, st, args.stage_reps)
    else:
        stages = {"shared": float("nan"), "unshared_merge_fused": float("nan"), "unshared": float("nan"),
                  "merge": float("nan"), "select_loop_3steps": float("nan")}
    log(f"[bench] stage ms/call: {stages}")
    flops, bytes_ = shared_stage_work(wl, st)
    t_shared = stages["shared"] / 1e3
    achieved = flops / t_shared / 1e12
    traffic = read_traffic()
    mfma = read_mfma()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "mfma_busy": None if mfma is None else mfma["mfma_busy"],
                "kernel": DOMINANT, "flops_per_launch": flops, "avg_launch_us": round(t_shared * 1e6, 2),
                "algorithmic_bytes_per_launch": bytes_,
                "algorithmic_hbm_GBs": round(bytes_ / t_shared / 1e9, 1),
                "counters": mfma}
    sel_roof = sel_gumbel = sel_logits = uns_roof = sel_loop_roof = ceilings = None
    if args.stage_reps > 0:
        uns_roof = unshared_roofline(wl, st, stages["unshared_merge_fused"])
        log(f"[bench] unshared + merge: {uns_roof}")
        sel_loop_roof = select_loop_roofline(wl, st, stages["select_loop_3steps"])
        log(f"[bench] select loop: {sel_loop_roof}")
        ceilings = measured_ceilings(dev)
        log(f"[bench] measured ceilings: {ceilings}")
        if ceilings:
            roofline["frac_of_measured_gemm"] = round(achieved / ceilings["bf16_gemm_TFLOPs"], 4)
            roofline["frac_of_measured_mfma_rate"] = round(achieved / ceilings["mfma_bf16_TFLOPs"], 4)
        sel_roof = select_roofline(args.seed, dev, 16 * args.stage_reps)
        log(f"[bench] select on wide512u: {sel_roof}")
        sel_gumbel = select_roofline(args.seed, dev, 16 * args.stage_reps, temperature=1.0)
        log(f"[bench] Gumbel select on wide512u: {sel_gumbel}")
        sel_logits = select_roofline(args.seed, dev, 16 * args.stage_reps, raw_logits=True)
        log(f"[bench] select from raw logits on wide512u: {sel_logits}")
    calib_copy(args, dev)

    cpu = cpu_small = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on a bounded sample ({oracle_cores()} cores) ...")
        cpu = cpu_baseline(wl, args.seed)
        log(f"[bench] oracle: {cpu}")
        if not args.no_cpu_full:
            cpu_small = []
            for name in ("tiny", "qwen06b"):
                log(f"[bench] the oracle on all of {name} ...")
                cpu_small.append(cpu_full(name, args.seed))
                log(f"[bench] {cpu_small[-1]}")
    res = {
        "metric": "beam decode steps/s (attn+select) at W=K=512; achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "beam decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.kv_dtype == "bf16" else wl.kv_dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": len(st["W"]), "beam_width": int(st["W"].max()),
                   "top_k": int(st["K"].max()), "prompt": int(st["P"].max()), "layers": wl.layers,
                   "heads": f"{wl.Hq}/{wl.Hkv}x{wl.D}", "codes_per_level": wl.C,
                   "decode_steps_per_bench_step": wl.S,
                   "trie": None if wl.catalog is None else f"{wl.catalog[0]} {wl.catalog[1]} items",
                   "device_flags": flags},
        "graph_replay_value": graph_value,
        "two_stream_attention": overlap,
        "stages_ms_per_call": {k: round(v, 4) for k, v in stages.items()},
        "roofline": roofline,
        "measured_ceilings": ceilings,
        "unshared_roofline": uns_roof,
        "select_loop_roofline": sel_loop_roof,
        "select_roofline": sel_roof,
        "select_gumbel_roofline": sel_gumbel,
        "select_logits_roofline": sel_logits,
        "cpu_baseline": cpu,
        "cpu_oracle_full_small_workloads": cpu_small,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
