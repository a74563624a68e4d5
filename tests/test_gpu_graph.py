"""The S-step decode loop captured as one HIP graph and replayed: every replay reproduces the
eager run bit for bit (selection state, semantic IDs, attention output), with eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

from synth import attention_layer, build_trie_csr, catalog_items, logprob_rows, request_shapes, workload
from tests.gpu_util import make_ws, say, trie_device, upload_layer

pytestmark = pytest.mark.gpu


def _state(loop, out):
    return [t.clone() for t in (loop.tokens, loop.parents, loop.sid, loop.final_scores(), loop.final_nodes(), out)]


def test_graph_replay_equals_eager(lib):
    wl = workload("qwen06b")
    W, K, P = request_shapes(wl)
    say(f"[graph] qwen06b R={len(W)} S={wl.S}")
    trie = build_trie_csr(catalog_items(wl), wl.C)
    ws = make_ws(lib, W, K, P, C=wl.C, S=wl.S)
    loop = lib.DecodeLoop(ws, wl.S, wl.C, trie_device(trie))
    layer = upload_layer(attention_layer(wl, 0), wl.q_dtype, wl.kv_dtype)
    lps = [torch.from_numpy(logprob_rows(wl, d)).cuda() for d in range(wl.S)]
    out = torch.empty(int(W.sum()), wl.Hq, wl.D, dtype=torch.float32, device="cuda")
    loop.run(lps, [layer], out)
    torch.cuda.synchronize()
    want = _state(loop, out)
    graph = loop.capture(lps, [layer], out)
    for rep in range(3):
        for t in (loop.tokens, loop.parents, loop.sid, out):
            t.fill_(-7)                       # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _state(loop, out)
        for name, a, b in zip(("tokens", "parents", "sid", "scores", "nodes", "out"), got, want):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), f"replay {rep}: {name}"
    assert ws.error_flags() == 0
