"""Model of the multi-stage prefetch ring (test infrastructure only).

Source: "（二）CUTLASS —— 掌握 Tensor Memory Accelerator（TMA）", section
"TMA 典型场景 Prefetching Data": in an iterative copy + compute loop the copy
of a future batch overlaps the compute of the current one, and the fetched
batch always runs num_stages ahead of the computed one
(fetch_batch = compute_batch + num_stages); the page's worked case for two
stages computes batch 0 while fetching 2, batch 1 while fetching 3, and so on.

Reading for the buffer count (the page does not give it): while batch i is
computed, batches i+1 .. i+S are in flight or resident, so the ring holds
S + 1 slots; batch j lives in slot j mod (S + 1), and the slot refilled at
iteration i held batch i - 1, whose reads must have retired first.
"""
from __future__ import annotations


def prefetch_schedule(n_batches: int, num_stages: int):
    """(prologue_fetches, [(compute_batch, fetch_batch_or_None), ...])."""
    S = num_stages
    prologue = list(range(min(S, n_batches)))
    steady = []
    for i in range(n_batches):
        f = i + S
        steady.append((i, f if f < n_batches else None))
    return prologue, steady


def ring_trace(n_batches: int, num_stages: int, n_slots: int | None = None):
    """Event list of the ring: ('fetch', batch, slot) and ('compute', batch, slot).

    Within an iteration the fetch is issued before the compute (the two
    overlap), which is what the page's schedule describes.
    """
    S = num_stages
    slots = S + 1 if n_slots is None else n_slots
    prologue, steady = prefetch_schedule(n_batches, S)
    ev = [("fetch", j, j % slots) for j in prologue]
    for i, f in steady:
        if f is not None:
            ev.append(("fetch", f, f % slots))
        ev.append(("compute", i, i % slots))
    return ev


def check_ring(events, n_batches: int):
    """Validate a trace: every batch fetched once before it is computed, computed
    once and in order, and no slot overwritten while it holds an uncomputed batch
    or the batch being computed in the same iteration.  Returns a list of problems."""
    problems = []
    resident = {}          # slot -> batch held and not yet computed
    fetched, computed = set(), []
    pending_fetch_slot = None
    for op, b, s in events:
        if op == "fetch":
            if b in fetched:
                problems.append("batch %d fetched twice" % b)
            if s in resident:
                problems.append("slot %d refilled with %d while batch %d unread" % (s, b, resident[s]))
            resident[s] = b
            fetched.add(b)
            pending_fetch_slot = s
        else:
            if resident.get(s) != b:
                problems.append("batch %d computed from slot %d holding %r" % (b, s, resident.get(s)))
            if s == pending_fetch_slot and resident.get(s) != b:
                problems.append("slot %d overlaps fetch and compute" % s)
            computed.append(b)
            resident.pop(s, None)
            pending_fetch_slot = None
    if computed != list(range(n_batches)):
        problems.append("compute order %r" % computed)
    return problems
