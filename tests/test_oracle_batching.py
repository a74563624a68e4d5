"""Pins of the slot-budget batching oracle (first fit in queue order).

* the deployment guide's examples (tests/golden/slot_budget_examples.txt);
* a worked example computed by hand, where next fit and first fit differ;
* brute force: the optimum number of batches over every assignment of tiny queues, and
  the first-fit bound FF <= floor(1.7 OPT) (Dosa and Sgall, "First Fit bin packing: a
  tight analysis", 2013);
* the characterisation of a first-fit result from its output alone (every request was
  refused by each earlier batch at its turn), checked by a function written from that
  statement, which a next-fit packing fails;
* special cases: equal widths, a queue that fits one batch, the request-count limit;
* the textbook property that at most one first-fit batch is at most half full.
"""
import itertools
import os

import numpy as np
import pytest

from oracle.batching import oracle_plan_batches

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_budget_examples.txt")


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(x) for x in line.split()))
    return rows


def is_first_fit(W, budget, max_req, batch_of):
    """True iff batch_of is the first-fit packing of W: limits hold, batches open in order,
    and each request found every lower-numbered batch full (rows or count) at its turn."""
    n = len(W)
    nb = max(batch_of) + 1 if n else 0
    rows = [0] * nb
    count = [0] * nb
    seen = -1
    for i in range(n):
        b = batch_of[i]
        if b > seen + 1:
            return False        # a batch opened out of order
        seen = max(seen, b)
        for e in range(b):
            if rows[e] + W[i] <= budget and count[e] < max_req:
                return False    # an earlier batch had room
        rows[b] += W[i]
        count[b] += 1
        if rows[b] > budget or count[b] > max_req:
            return False
    return True


def next_fit(W, budget, max_req):
    """A plausible mistake: close the current batch as soon as a request does not fit."""
    out, rows, cnt, b = [], 0, 0, 0
    for w in W:
        if out and (rows + w > budget or cnt >= max_req):
            b, rows, cnt = b + 1, 0, 0
        out.append(b)
        rows, cnt = rows + w, cnt + 1
    return out


def optimum(W, budget, max_req):
    """Fewest batches over every assignment (brute force, tiny queues)."""
    n = len(W)
    for k in range(1, n + 1):
        for assign in itertools.product(range(k), repeat=n):
            if len(set(assign)) != k:
                continue
            rows = [0] * k
            cnt = [0] * k
            for w, b in zip(W, assign):
                rows[b] += w
                cnt[b] += 1
            if max(rows) <= budget and max(cnt) <= max_req:
                return k
    raise AssertionError("unreachable")


@pytest.mark.parametrize("budget,width,n,per", golden_rows())
def test_deployment_guide_examples(budget, width, n, per):
    batch_of, nb = oracle_plan_batches([width] * n, budget, 10 ** 6)
    assert nb == -(-n // per)
    assert batch_of == [i // per for i in range(n)]


def test_worked_example_by_hand():
    # budget 800: 600 opens batch 0; 300 cannot join it (900) and opens batch 1; 300 joins
    # batch 1 (600); 200 joins batch 0 (800); 500 fits neither (1300, 1100) and opens batch 2
    W = [600, 300, 300, 200, 500]
    assert oracle_plan_batches(W, 800, 10) == ([0, 1, 1, 0, 2], 3)
    assert next_fit(W, 800, 10) == [0, 1, 1, 1, 2]
    assert not is_first_fit(W, 800, 10, next_fit(W, 800, 10))
    # at most two requests per batch: the same result (batch 0 holds one request when the
    # 200 arrives, batch 1 is full by count); one request per batch: one batch each
    assert oracle_plan_batches(W, 800, 2) == ([0, 1, 1, 0, 2], 3)
    assert oracle_plan_batches(W, 800, 1) == ([0, 1, 2, 3, 4], 5)


def test_brute_force_optimum_and_first_fit_bound():
    rng = np.random.default_rng(7)
    for _ in range(300):
        n = int(rng.integers(1, 7))
        budget = int(rng.integers(4, 20))
        W = [int(x) for x in rng.integers(1, budget + 1, size=n)]
        batch_of, nb = oracle_plan_batches(W, budget, n)
        opt = optimum(W, budget, n)
        assert opt <= nb <= int(np.floor(1.7 * opt)), (W, budget, nb, opt)
        assert is_first_fit(W, budget, n, batch_of)


def test_characterisation_on_random_queues():
    rng = np.random.default_rng(11)
    for _ in range(200):
        n = int(rng.integers(0, 80))
        budget = int(rng.integers(1, 300))
        max_req = int(rng.integers(1, 12))
        W = [int(x) for x in rng.integers(1, budget + 1, size=n)]
        batch_of, nb = oracle_plan_batches(W, budget, max_req)
        assert len(batch_of) == n and nb == (max(batch_of) + 1 if n else 0)
        assert is_first_fit(W, budget, max_req, batch_of)
        if n >= 3 and next_fit(W, budget, max_req) != batch_of:
            assert not is_first_fit(W, budget, max_req, next_fit(W, budget, max_req))


def test_special_cases():
    # equal widths: floor(budget / w) per batch, or the request limit if smaller
    for w, budget, max_req, n in ((3, 10, 100, 17), (5, 5, 4, 6), (7, 100, 4, 30)):
        per = min(max_req, budget // w)
        batch_of, nb = oracle_plan_batches([w] * n, budget, max_req)
        assert batch_of == [i // per for i in range(n)] and nb == -(-n // per)
    # a queue that fits one batch stays one batch
    assert oracle_plan_batches([5, 1, 9, 3], 18, 4) == ([0, 0, 0, 0], 1)
    assert oracle_plan_batches([], 8, 2) == ([], 0)
    with pytest.raises(ValueError):
        oracle_plan_batches([9], 8, 2)
    with pytest.raises(ValueError):
        oracle_plan_batches([0], 8, 2)


def test_at_most_one_batch_half_full():
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(1, 200))
        budget = int(rng.integers(2, 1000))
        W = rng.integers(1, budget + 1, size=n)
        batch_of, nb = oracle_plan_batches(W, budget, n)
        load = np.bincount(batch_of, weights=W, minlength=nb)
        assert np.sum(2 * load <= budget) <= 1
        assert nb >= -(-int(W.sum()) // budget)
