"""Oracle slot-budget batching — TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* FlashRec announcement (SGLang PR thread): scheduling by a beam-row slot budget, so that
  the rows of several requests share one decode step.
* FlashRec deployment guide, wide-beam section: with the default 800 slots one 512-beam
  request fills a wave on its own; with 4096 slots about four 1000-beam requests run
  together; troubleshooting: wide-beam throughput stops growing with concurrency when the
  slot count is below beam width times concurrency.

Reading where the pages are silent: the pages give the budget (beam rows per step) but no
packing order.  The plainest policy that never reorders a batch and never lets a request
wait while an earlier batch has room for it is first fit in queue order: request i joins
the lowest-numbered batch that still has room for its W_i rows (and, when the number of
requests per batch is bounded, a free request slot); otherwise it opens a new batch.
Batches are numbered in the order they open.
"""
from __future__ import annotations


def oracle_plan_batches(W, slot_budget: int, max_requests: int):
    """First fit in queue order; returns (batch_of list, number of batches).

    Written as the definition: for each request in order, scan the open batches from the
    first and take the first with room, else open a new one."""
    if slot_budget < 1 or max_requests < 1:
        raise ValueError("slot_budget and max_requests must be >= 1")
    rows, count, batch_of = [], [], []
    for w in (int(x) for x in W):
        if not 1 <= w <= slot_budget:
            raise ValueError(f"width {w} outside [1, {slot_budget}]")
        for b in range(len(rows)):
            if rows[b] + w <= slot_budget and count[b] < max_requests:
                rows[b] += w
                count[b] += 1
                batch_of.append(b)
                break
        else:
            rows.append(w)
            count.append(1)
            batch_of.append(len(rows) - 1)
    return batch_of, len(rows)
