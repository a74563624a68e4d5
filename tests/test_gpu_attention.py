"""GPU parity of beam_attn_decode against the oracle's float64 concatenated-KV attention.

Tolerance (max abs error): 1e-4 for float32 inputs, 2e-2 for bf16 / fp8 KV with float32
accumulation.  Parent pointers are uniform in [0, W_r) per depth, with dead slots."""
import numpy as np
import pytest
import torch

from synth import attention_layer, random_parents, request_shapes, workload
from tests.gpu_util import attention_vs_oracle, make_ws, oracle_threads, say, upload_layer

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 2e-2}


def run_attention(lib, wl, layer, parents, Ws, Ks, Ps, steps, samples_of_step, max_splits=0,
                  Hq=None, Hkv=None, D=None, pad=0):
    Hq, Hkv, D = Hq or wl.Hq, Hkv or wl.Hkv, D or wl.D
    ws = make_ws(lib, Ws, Ks, Ps, C=16, S=wl.S, Hq=Hq, Hkv=Hkv, D=D, q_dtype=wl.q_dtype,
                 kv_dtype=wl.kv_dtype, max_splits=max_splits)
    dev = upload_layer(layer, wl.q_dtype, wl.kv_dtype, pad=pad)
    par = torch.from_numpy(parents).cuda()
    out = torch.empty(int(sum(Ws)), Hq, D, dtype=torch.float32, device="cuda")
    worst = 0.0
    for d in steps:
        out.fill_(float("nan"))
        lib.beam_attn_decode(ws, dev["q"][d], dev["k_s"], dev["v_s"], dev["k_scale"], dev["v_scale"],
                             dev["k_u"], dev["v_u"], par, d, out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        # dead slots are exactly zero
        dead = np.nonzero(parents[d] < 0)[0]
        assert np.all(o[dead] == 0.0)
        say(f"[attn] {wl.name} d={d}: comparing with the oracle")
        worst = max(worst, attention_vs_oracle(o, layer, parents, d, list(Ws), wl.q_dtype, wl.kv_dtype,
                                               samples_of_step(d), TOL[wl.kv_dtype], label=f"{wl.name} d={d}",
                                               threads=oracle_threads()))
    assert ws.error_flags() == 0
    say(f"[attn] {wl.name}: worst max-abs error {worst:.3e}")
    return ws


def all_slots(Ws):
    return lambda d: {r: range(int(w)) for r, w in enumerate(Ws)}


def test_tiny_fp32_every_slot(lib):
    wl = workload("tiny")
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl, dead_frac=0.25)
    run_attention(lib, wl, layer, par, W, K, P, range(wl.S), all_slots(W))


def test_qwen06b_bf16_every_slot(lib):
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl, dead_frac=0.1)
    ws = run_attention(lib, wl, layer, par, W, K, P, [0, 2], all_slots(W))
    assert ws.splits(0) > 1          # the prompt is split across workgroups and merged


def test_wide512_sampled(lib):
    wl = workload("wide512")
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl)
    rng = np.random.default_rng(1)
    samples = lambda d: {r: rng.choice(512, size=24, replace=False) for r in range(len(W))}
    run_attention(lib, wl, layer, par, W, K, P, range(wl.S), samples)


def short_prompt_case(name, P, index):
    """A workload's attention shape with a short prompt, so that the decode tokens carry a
    large share of the softmax mass (a wrong ancestor or merge weight then moves the output far
    beyond the tolerance; tests/test_oracle_attention.py checks that on these inputs)."""
    import dataclasses
    wl = dataclasses.replace(workload(name), P=P, layers=1, index=index)
    W, K, Ps = request_shapes(wl)
    return wl, (W, K, Ps)


def test_wide512_short_prompt_every_slot(lib):
    """The headline attention shape (4 requests x W = 512, 16/8/128 bf16: two waves per slot in
    the unshared stage, slots up to 2047) with a 64-token prompt: every slot at depths 0-2
    against the oracle."""
    wl, shapes = short_prompt_case("wide512", 64, 60)
    W, K, P = shapes
    layer = attention_layer(wl, 0, shapes=shapes)
    par = random_parents(wl, shapes=shapes, dead_frac=0.05)
    run_attention(lib, wl, layer, par, W, K, P, range(wl.S), all_slots(W))


def test_ultra5000_short_prompt_deep_every_slot(lib):
    """The ultra-wide attention shape (W = 5000) with a 64-token prompt: every slot walks 15
    parent pointers at depth 15 (and 3 at depth 3) and every slot is compared."""
    wl, shapes = short_prompt_case("ultra5000", 64, 61)
    W, K, P = shapes
    layer = attention_layer(wl, 0, shapes=shapes)
    par = random_parents(wl, shapes=shapes)
    run_attention(lib, wl, layer, par, W, K, P, [3, 15], all_slots(W))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_nan_padding_is_ignored(lib, kv):
    """Prompt storage padding (rows P_r .. Pp_r - 1 of K, columns of V^T) filled with NaN bit
    patterns (bf16 0x7FC0, e4m3 0x7F): the outputs are finite and match the oracle, on the
    8-wave wide kernel (bf16 W = 300, split prompt), the 4-wave kernel (narrow bf16 and every
    fp8 request) and prompts whose last tile is partial."""
    import dataclasses
    wl = dataclasses.replace(workload("mixed_fp8" if kv == "fp8" else "qwen06b"), n_requests=3, W=None, K=None,
                             P=None, S=3, index=70 + (kv == "fp8"))
    Ws = np.array([300, 20, 129], np.int32)
    Ps = np.array([1000, 77, 130], np.int32)
    Ks = Ws.copy()
    layer = attention_layer(wl, 0, shapes=(Ws, Ks, Ps))
    par = random_parents(wl, shapes=(Ws, Ks, Ps), dead_frac=0.1)
    pad = 0x7FC0 if kv == "bf16" else 0x7F
    run_attention(lib, wl, layer, par, Ws, Ks, Ps, [0, 2], all_slots(Ws), max_splits=4, pad=pad)


def test_mixed_fp8_ragged(lib):
    wl = workload("mixed_fp8")
    W, K, P = request_shapes(wl)
    rng = np.random.default_rng(2)
    check = sorted(set(rng.choice(len(W) - 1, size=10, replace=False).tolist()) | {len(W) - 1})
    layer = attention_layer(wl, 0, requests=check)
    # prompt KV of unchecked requests still has to exist on the device: zeros of the right shape
    for r in range(len(W)):
        if layer["k_s"][r] is None:
            layer["k_s"][r] = np.zeros((wl.Hkv, int(P[r]), wl.D), np.uint8)
            layer["v_s"][r] = np.zeros((wl.Hkv, int(P[r]), wl.D), np.uint8)
    par = random_parents(wl, dead_frac=0.1)
    samples = lambda d: {r: (range(int(W[r])) if W[r] <= 8 else rng.choice(int(W[r]), size=8, replace=False))
                         for r in check}
    run_attention(lib, wl, layer, par, W, K, P, [0, 3], samples)


def test_ultra5000_deep_ancestry(lib):
    wl = workload("ultra5000")
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl)
    rng = np.random.default_rng(3)
    samples = lambda d: {0: rng.choice(5000, size=24, replace=False)}
    run_attention(lib, wl, layer, par, W, K, P, [0, 7, 15], samples)


def test_deepest_ancestry(lib):
    """The deepest decode step the library takes (step 63 of 64): every slot walks 63 parent
    pointers; bf16 (8-wave kernel for the wide request) and the narrow request."""
    import dataclasses
    wl = dataclasses.replace(workload("qwen06b"), n_requests=2, W=None, K=None, P=None, S=64, index=98)
    Ws = np.array([80, 6], np.int32)
    Ps = np.array([200, 64], np.int32)
    Ks = Ws.copy()
    layer = attention_layer(wl, 0, shapes=(Ws, Ks, Ps))
    par = random_parents(wl, shapes=(Ws, Ks, Ps), dead_frac=0.1)
    run_attention(lib, wl, layer, par, Ws, Ks, Ps, [63, 31], all_slots(Ws))


@pytest.mark.parametrize("P", [1, 63, 65, 1000, 4097])
def test_ragged_prompt_lengths_and_rows(lib, P):
    """Prompt lengths off the 64-key tile, row counts off the 128-row tile, split prompts."""
    import dataclasses
    wl = dataclasses.replace(workload("qwen06b"), n_requests=3, W=None, K=None, P=None, S=3, index=90 + P)
    Ws = np.array([1, 37, 70], np.int32)
    Ps = np.array([P, max(1, P // 2), P + 3], np.int32)
    Ks = Ws.copy()
    layer = attention_layer(wl, 0, shapes=(Ws, Ks, Ps))
    par = random_parents(wl, shapes=(Ws, Ks, Ps), dead_frac=0.2)
    run_attention(lib, wl, layer, par, Ws, Ks, Ps, [0, 2], all_slots(Ws), max_splits=4)


def test_bf16_generic_head_dim_path(lib):
    """Head dim 64 with bf16 KV takes the generic VALU shared stage."""
    import dataclasses
    wl = dataclasses.replace(workload("qwen06b"), n_requests=2, W=9, K=9, P=300, D=64, S=2, index=80)
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl)
    run_attention(lib, wl, layer, par, W, K, P, [0, 1], all_slots(W))


def test_stage_by_stage_equals_fused_path(lib):
    """Shared, unshared and merge launched one stage at a time (merge as its own kernel over
    workspace partials) give the same output as the default path (merge fused into the
    unshared epilogue), and both match the oracle."""
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    layer = attention_layer(wl, 0)
    par = random_parents(wl, dead_frac=0.1)
    ws = make_ws(lib, W, K, P, C=16, S=wl.S)
    dev = upload_layer(layer, wl.q_dtype, wl.kv_dtype)
    parents = torch.from_numpy(par).cuda()
    out_a = torch.full((int(W.sum()), wl.Hq, wl.D), float("nan"), device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    d = 2
    args = (dev["q"][d], dev["k_s"], dev["v_s"], None, None, dev["k_u"], dev["v_u"], parents, d)
    lib.beam_attn_decode(ws, *args, out_a)
    for mask in (lib.STAGE_SHARED, lib.STAGE_UNSHARED, lib.STAGE_MERGE):
        lib.beam_attn_decode_stages(ws, *args, out_b, mask)
    torch.cuda.synchronize()
    a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    assert np.max(np.abs(a - b)) <= 1e-5
    attention_vs_oracle(b, layer, par, d, list(W), wl.q_dtype, wl.kv_dtype,
                        {0: range(int(W[0])), 7: range(int(W[7]))}, TOL["bf16"], label="stagewise")
    with pytest.raises(lib.GrwError):
        lib.beam_attn_decode_stages(ws, *args, out_b, 0)


def test_wide_and_narrow_requests_equal_stagewise(lib):
    """Wide bf16 requests (the 8-wave shared-stage kernel) next to a narrow one (the 4-wave
    kernel), with split and unsplit prompts, deep ancestry and dead slots: the default path
    equals the stage-by-stage path, matches the oracle, and repeats bit for bit over calls
    at other depths and over graph replays."""
    import dataclasses
    wl = dataclasses.replace(workload("qwen06b"), n_requests=3, W=None, K=None, P=None, S=4, index=97)
    Ws = np.array([300, 40, 129], np.int32)
    Ps = np.array([3000, 200, 64], np.int32)
    Ks = Ws.copy()
    layer = attention_layer(wl, 0, shapes=(Ws, Ks, Ps))
    par = random_parents(wl, shapes=(Ws, Ks, Ps), dead_frac=0.15)
    ws = make_ws(lib, Ws, Ks, Ps, C=16, S=wl.S)
    assert ws.splits(0) > 1 and ws.splits(2) == 1
    dev = upload_layer(layer, wl.q_dtype, wl.kv_dtype)
    parents = torch.from_numpy(par).cuda()
    rng = np.random.default_rng(6)
    outs = {}
    for d in (3, 0, 2):
        out_a = torch.full((int(Ws.sum()), wl.Hq, wl.D), float("nan"), device="cuda")
        out_b = torch.full_like(out_a, float("nan"))
        args = (dev["q"][d], dev["k_s"], dev["v_s"], None, None, dev["k_u"], dev["v_u"], parents, d)
        lib.beam_attn_decode(ws, *args, out_a)
        for mask in (lib.STAGE_SHARED, lib.STAGE_UNSHARED, lib.STAGE_MERGE):
            lib.beam_attn_decode_stages(ws, *args, out_b, mask)
        torch.cuda.synchronize()
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.all(np.isfinite(a))
        assert np.max(np.abs(a - b)) <= 1e-5, f"d={d}: {np.max(np.abs(a - b))}"
        samples = {r: rng.choice(int(Ws[r]), size=min(24, int(Ws[r])), replace=False) for r in range(3)}
        err = attention_vs_oracle(a, layer, par, d, list(Ws), wl.q_dtype, wl.kv_dtype, samples, TOL["bf16"],
                                  label=f"wide + narrow d={d}")
        say(f"[attn] wide + narrow d={d}: vs stage-wise {np.max(np.abs(a - b)):.2e}, oracle {err:.3e}")
        outs[d] = out_a.clone()
    # repeated calls inside a graph, replayed twice
    out_g = torch.empty_like(outs[3])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for d in (0, 3):
            lib.beam_attn_decode(ws, dev["q"][d], dev["k_s"], dev["v_s"], None, None, dev["k_u"], dev["v_u"],
                                 parents, d, out_g)
    for _ in range(2):
        out_g.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, outs[3])
    assert ws.error_flags() == 0
