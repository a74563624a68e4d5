"""beam_select_noalloc — the selection of one request for callers that cannot allocate (its
scratch is the library's static device array): equal to beam_select on a workspace, bit for
bit, on two calls in a row, the second with a smaller input; sizes beyond the array refused
with nothing enqueued."""
import numpy as np
import pytest
import torch

from synth import build_trie_csr, catalog_items, logprob_rows, request_shapes, workload
from tests.gpu_util import make_ws, say, trie_device

pytestmark = pytest.mark.gpu


def _outputs(n):
    return (torch.full((n,), -7, dtype=torch.int32, device="cuda"),
            torch.full((n,), -7, dtype=torch.int32, device="cuda"),
            torch.full((n,), 7.0, dtype=torch.float32, device="cuda"),
            torch.full((n,), -7, dtype=torch.int32, device="cuda"))


def _case(lib, name, trie_items, steps_before):
    """A live beam state of request 0 of a workload after `steps_before` workspace selections,
    and the next step's log-probability rows."""
    wl = workload(name)
    W, K, C = int(wl.W), int(wl.K), wl.C
    trie = build_trie_csr(trie_items, C) if trie_items is not None else None
    t = trie_device(trie)
    ws = make_ws(lib, [W], [K], [64], C=C, S=wl.S)
    loop = lib.DecodeLoop(ws, wl.S, C, t)
    ws.beams_init(loop.scores[0], loop.nodes[0])
    shapes = (np.array([W], np.int32), np.array([K], np.int32), np.array([64], np.int32))
    for d in range(steps_before):
        loop.select_step(d, torch.from_numpy(logprob_rows(wl, d, shapes=shapes)).cuda())
    cur = steps_before % 2
    lp = torch.from_numpy(logprob_rows(wl, steps_before, shapes=shapes)).cuda()
    return dict(ws=ws, W=W, K=K, C=C, t=t, lp=lp, scores=loop.scores[cur].clone(), nodes=loop.nodes[cur].clone())


def _with_workspace(lib, c):
    out = _outputs(c["W"])
    t = c["t"] or (None, None, 0)
    lib.beam_select(c["ws"], c["lp"], c["scores"], c["nodes"], t[0], t[1], t[2], c["W"], c["K"], c["C"], *out)
    return out


def _without(lib, c, flags):
    out = _outputs(c["W"])
    t = c["t"] or (None, None, 0)
    lib.beam_select_noalloc(c["lp"], c["scores"], c["nodes"], t[0], t[1], t[2], c["W"], c["K"], c["C"], *out,
                            device_flags=flags)
    return out


def _same(a, b, label):
    for x, y, what in zip(a, b, ("tokens", "parents", "scores", "nodes")):
        x, y = x.cpu(), y.cpu()
        if what == "scores":
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{label}: {what} differ"


def test_noalloc_equals_workspace_select_twice(lib):
    say("[noalloc] W = K = 512 unconstrained over 8192 codes (third step, every beam live)")
    big = _case(lib, "wide512u", None, 2)
    say("[noalloc] W = K = 50 on the 1M-item trie (second step)")
    small = _case(lib, "qwen06b", catalog_items(workload("qwen06b")), 1)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref_big, ref_small = _with_workspace(lib, big), _with_workspace(lib, small)
    got_big = _without(lib, big, flags)
    got_small = _without(lib, small, flags)      # the second call, smaller, over the same scratch
    torch.cuda.synchronize()
    _same(ref_big, got_big, "W=K=512")
    _same(ref_small, got_small, "W=K=50 trie")
    assert int((got_big[1] >= 0).sum()) == 512 and int((got_small[1] >= 0).sum()) == 50
    assert flags.item() == 0
    # without a flag word of the caller's: the library's own word in the scratch
    again = _without(lib, small, None)
    torch.cuda.synchronize()
    _same(ref_small, again, "W=K=50 trie, library flag word")


def test_noalloc_refuses_sizes_beyond_its_scratch(lib):
    lp = torch.zeros(1025, 64, device="cuda")
    sc = torch.zeros(1025, device="cuda")
    out = _outputs(1025)
    for W, K, C in ((1025, 4, 64), (600, 600, 64), (16, 4, 8193)):
        with pytest.raises(lib.GrwError) as e:
            lib.beam_select_noalloc(lp, sc, None, None, None, 0, W, K, C, *out)
        assert e.value.status == 4, (W, K, C)
    with pytest.raises(lib.GrwError) as e:
        lib.beam_select_noalloc(lp, sc, None, None, None, 0, 0, 4, 64, *out)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(out[0] == -7)              # nothing was enqueued
