"""The device-flag contract of include/grw.h: precondition violations that only the device can
see do not stop the kernels; they set bits in the workspace's flag word, which grw_ws_error
reports and clears.  Each test plants one violation among valid inputs, checks its bit, that
every call returned normally, that the slots it does not touch still match the oracle, and
that a clean call afterwards leaves the word at zero.  Every guard sits before the load it
protects (an out-of-range parent or node is never used as an index)."""
import dataclasses

import numpy as np
import pytest
import torch

from synth import (attention_layer, build_trie_csr, catalog_items, logprob_rows, random_parents, request_shapes,
                   workload)
from tests.gpu_util import attention_vs_oracle, make_ws, say, trie_device, upload_layer

pytestmark = pytest.mark.gpu


def _attention_case(lib):
    wl = dataclasses.replace(workload("qwen06b"), n_requests=2, W=None, K=None, P=None, S=3, index=75)
    Ws = np.array([40, 9], np.int32)
    Ps = np.array([130, 64], np.int32)
    Ks = Ws.copy()
    layer = attention_layer(wl, 0, shapes=(Ws, Ks, Ps))
    par = random_parents(wl, shapes=(Ws, Ks, Ps))
    ws = make_ws(lib, Ws, Ks, Ps, C=16, S=wl.S)
    return wl, Ws, layer, par, ws, upload_layer(layer, wl.q_dtype, wl.kv_dtype)


@pytest.mark.parametrize("bad", ["out_of_range", "dead_ancestor"])
def test_bad_parent_flag(lib, bad):
    wl, Ws, layer, par, ws, dev = _attention_case(lib)
    d, b = 2, 17
    planted = par.copy()
    if bad == "out_of_range":
        planted[2, b] = Ws[0] + 3            # beyond request 0's slots (a slot of request 1)
    else:
        planted[1, planted[2, b]] = -1       # a live beam whose ancestor at depth 1 is dead
    touched = {int(b)} if bad == "out_of_range" else set(np.nonzero(par[2, :Ws[0]] == par[2, b])[0].tolist())
    say(f"[flags] bad parent ({bad}) at slot {b}, depth {d}")
    out = torch.zeros(int(Ws.sum()), wl.Hq, wl.D, device="cuda")
    lib.beam_attn_decode(ws, dev["q"][d], dev["k_s"], dev["v_s"], None, None, dev["k_u"], dev["v_u"],
                         torch.from_numpy(planted).cuda(), d, out)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_BAD_PARENT
    keep = [j for j in range(int(Ws[0])) if j not in touched]
    attention_vs_oracle(out.cpu().numpy(), layer, planted, d, list(Ws), wl.q_dtype, wl.kv_dtype,
                        {0: keep, 1: range(int(Ws[1]))}, 2e-2, label="bad parent, other slots")
    lib.beam_attn_decode(ws, dev["q"][d], dev["k_s"], dev["v_s"], None, None, dev["k_u"], dev["v_u"],
                         torch.from_numpy(par).cuda(), d, out)
    assert ws.error_flags() == 0


def _select_case(lib):
    wl = workload("tiny")
    W, K, P = request_shapes(wl)
    items = catalog_items(wl)
    trie = build_trie_csr(items, wl.C)
    ws = make_ws(lib, W, K, P, C=wl.C, S=wl.S, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, q_dtype="f32", kv_dtype="f32")
    return wl, W, K, trie, ws


def _outputs(n):
    return (torch.empty(n, dtype=torch.int32, device="cuda"), torch.empty(n, dtype=torch.int32, device="cuda"),
            torch.empty(n, dtype=torch.float32, device="cuda"), torch.empty(n, dtype=torch.int32, device="cuda"))


def test_bad_node_flag(lib):
    wl, W, K, trie, ws = _select_case(lib)
    t = trie_device(trie)
    n = int(W.sum())
    lp = torch.from_numpy(logprob_rows(wl, 1)).cuda()
    scores = torch.tensor([-1.0, -2.0, -3.0, -4.0], device="cuda")
    nodes = torch.tensor([1, 2, trie["n_internal"] + 5, 3], dtype=torch.int32, device="cuda")
    say("[flags] bad node on slot 2")
    tok, par, sc, nd = _outputs(n)
    lib.beam_select(ws, lp, scores, nodes, t[0], t[1], t[2], int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_BAD_NODE
    assert not (par == 2).any().item()          # the slot with the bad node contributes nothing
    nodes[2] = 4
    lib.beam_select(ws, lp, scores, nodes, t[0], t[1], t[2], int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    assert ws.error_flags() == 0


def test_positive_logprob_flag(lib):
    wl, W, K, trie, ws = _select_case(lib)
    n = int(W.sum())
    lp = torch.from_numpy(logprob_rows(wl, 0)).cuda()
    scores = torch.tensor([0.0] + [-np.inf] * (n - 1), device="cuda")
    nodes = torch.tensor([0] + [-1] * (n - 1), dtype=torch.int32, device="cuda")
    tok, par, sc, nd = _outputs(n)
    lp[0, 7] = 0.5
    say("[flags] positive log-probability in the live row")
    lib.beam_select(ws, lp, scores, nodes, None, None, 0, int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_POS_LOGPROB
    lp[0, 7] = -0.5
    lib.beam_select(ws, lp, scores, nodes, None, None, 0, int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    assert ws.error_flags() == 0


def test_dense_mask_code_missing_from_csr_flag(lib):
    """A dense child mask that names a code its CSR row lacks: when the selection keeps that
    code, CHILD_MISSING is raised and its output node is -1; the other outputs still name their
    CSR children."""
    wl, W, K, trie, ws = _select_case(lib)
    n = int(W.sum())
    row = trie["code"][trie["row_ptr"][0]:trie["row_ptr"][1]]
    missing = int(np.setdiff1d(np.arange(wl.C), row)[0])
    slot, masks = lib.trie_dense_build(trie["row_ptr"], trie["code"], trie["n_internal"], wl.C, 1)
    masks = masks.copy()
    masks[slot[0], missing >> 5] |= np.uint32(1 << (missing & 31))
    t = (torch.from_numpy(trie["row_ptr"]).cuda(), torch.from_numpy(trie["code"]).cuda(), int(trie["n_internal"]),
         torch.from_numpy(slot).cuda(), torch.from_numpy(masks.view(np.int32)).cuda())
    # one strong candidate per 64-code group of the prompt row (the planted code the best) and
    # every other code far below: exactly top_k = 4 candidates reach the per-beam stage, which
    # keeps them with their edges from the dense mask
    strong = [missing] + [int(row[(row >> 6) == grp][0]) for grp in range(4) if grp != missing >> 6]
    assert len(strong) == 4
    lp = torch.full((n, wl.C), -10.0, device="cuda")
    for i, c in enumerate(strong):
        lp[0, c] = -float(i)
    scores = torch.tensor([0.0] + [-np.inf] * (n - 1), device="cuda")
    nodes = torch.tensor([0] + [-1] * (n - 1), dtype=torch.int32, device="cuda")
    tok, par, sc, nd = _outputs(n)
    say(f"[flags] dense mask names code {missing}, which the root's CSR row lacks")
    lib.beam_select_ex(ws, lp, scores, nodes, t, int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    torch.cuda.synchronize()
    assert ws.error_flags() & lib.FLAG_CHILD_MISSING
    assert tok[0].item() == missing and nd[0].item() == -1
    live = (par >= 0).cpu().numpy()
    codes_out = tok.cpu().numpy()[live][1:]
    nodes_out = nd.cpu().numpy()[live][1:]
    assert np.all(trie["node_prefix"][nodes_out] == codes_out)   # depth-1 prefixes are the codes
    lp[0, missing] = -50.0                     # the planted code no longer kept
    lib.beam_select_ex(ws, lp, scores, nodes, t, int(W.max()), int(K.max()), wl.C, tok, par, sc, nd)
    assert ws.error_flags() == 0


def test_failed_bind_leaves_no_batch_bound(lib):
    """A bind that fails validation leaves the workspace unbound: step calls then report the
    call-order error instead of running against a half-updated batch."""
    ws = make_ws(lib, [8, 8], [8, 8], [64, 64], C=64, S=3)
    with pytest.raises(lib.GrwError):
        ws.bind_batch([8, 9000], [8, 8], [64, 64])
    n = 16
    tok, par, sc, nd = _outputs(n)
    lp = torch.zeros(n, 64, device="cuda")
    scores = torch.zeros(n, device="cuda")
    with pytest.raises(lib.GrwError) as e:
        lib.beam_select(ws, lp, scores, None, None, None, 0, 8, 8, 64, tok, par, sc, nd)
    assert e.value.status == 5
