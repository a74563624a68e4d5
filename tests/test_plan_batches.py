"""Host-side slot-budget batching of the library (grw_plan_batches) against the oracle's
first fit in queue order, element by element; the mixed-width queue shape of the ragged
fp8 workload; invalid arguments.  Runs on the CPU (host code of the library)."""
import ctypes

import numpy as np
import pytest

from oracle.batching import oracle_plan_batches
from synth import request_shapes, workload


@pytest.fixture(scope="module")
def grw():
    import generative_recommendation_wide_amd as g
    return g


@pytest.mark.parametrize("seed", range(6))
def test_equals_oracle_on_random_queues(grw, seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        n = int(rng.integers(0, 300))
        budget = int(rng.integers(1, 5000))
        max_req = int(rng.integers(1, 40))
        kind = rng.integers(3)
        if kind == 0:
            W = rng.integers(1, budget + 1, size=n)
        elif kind == 1:      # narrow requests only: many share a batch
            W = rng.integers(1, max(2, budget // 20) + 1, size=n)
        else:                # widths near half the budget: pairing decisions
            W = np.clip(rng.integers(budget // 3, budget // 2 + 2, size=n), 1, budget)
        got, nb = grw.plan_batches(W, budget, max_req)
        want, wnb = oracle_plan_batches(W.tolist(), budget, max_req)
        assert nb == wnb
        np.testing.assert_array_equal(got, np.array(want, np.int32))


def test_large_queue_equals_oracle(grw):
    rng = np.random.default_rng(5)
    W = rng.integers(1, 1001, size=20000)
    got, nb = grw.plan_batches(W, 4096, 64)
    want, wnb = oracle_plan_batches(W.tolist(), 4096, 64)
    assert nb == wnb
    np.testing.assert_array_equal(got, np.array(want, np.int32))


def test_mixed_fp8_queue(grw):
    """The ragged fp8 workload's 101 requests (widths 2..100 and one of 1000) under the
    deployment guide's 4096-slot budget."""
    W, _, _ = request_shapes(workload("mixed_fp8"), 0)
    got, nb = grw.plan_batches(W, 4096, 128)
    want, wnb = oracle_plan_batches(W.tolist(), 4096, 128)
    np.testing.assert_array_equal(got, np.array(want, np.int32))
    load = np.bincount(got, weights=W, minlength=nb)
    assert nb == wnb == -(-int(W.sum()) // 4096) and load.max() <= 4096


def test_invalid_arguments(grw):
    L = grw._lib.load()
    nb = ctypes.c_int32(-7)
    out = np.zeros(4, np.int32)
    W = np.array([3, 9, 2, 1], np.int32)
    f = L.grw_plan_batches
    assert f(4, W.ctypes.data, 8, 4, out.ctypes.data, ctypes.byref(nb)) == 1       # 9 > budget
    W[1] = 0
    assert f(4, W.ctypes.data, 8, 4, out.ctypes.data, ctypes.byref(nb)) == 1       # width 0
    W[1] = 4
    assert f(-1, W.ctypes.data, 8, 4, out.ctypes.data, ctypes.byref(nb)) == 1
    assert f(4, None, 8, 4, out.ctypes.data, ctypes.byref(nb)) == 1
    assert f(4, W.ctypes.data, 8, 4, None, ctypes.byref(nb)) == 1
    assert f(4, W.ctypes.data, 8, 4, out.ctypes.data, None) == 1
    assert f(4, W.ctypes.data, 0, 4, out.ctypes.data, ctypes.byref(nb)) == 1
    assert f(4, W.ctypes.data, 8, 0, out.ctypes.data, ctypes.byref(nb)) == 1
    assert f(0, None, 8, 4, None, ctypes.byref(nb)) == 0 and nb.value == 0
    assert f(4, W.ctypes.data, 8, 4, out.ctypes.data, ctypes.byref(nb)) == 0
    assert nb.value == 2 and out.tolist() == [0, 0, 1, 0]
    with pytest.raises(grw._lib.GrwError):
        grw.plan_batches([5, 9], 8, 2)
