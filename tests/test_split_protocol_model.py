"""A model of the split-row exchange on the CPU, run under random interleavings.

The kernels (reduce_moe_finalize_amd/csrc/fused_boundary.hip, latency and
balanced kernels) combine a row's partial sums of squares across the
workgroups that share the row through 64-bit slots {32-bit epoch, value} in
the row's workspace record.  This file restates that protocol step by step as
a small state machine and lets a seeded random scheduler interleave the
workgroups of one row over many consecutive calls, with bounded waits that
give up (as the host-set wait limit forces them to), workgroups that start
late, a split that changes from call to call, the 32-bit epoch wrap and a
residual updated in place.  Memory is sequentially consistent here: the
ordering the kernels get from their fences (a workgroup's part is visible
before it overwrites an in-place residual) is the order of the steps.

Checked after every call:
  * every workgroup ends with the row's exact total (a part recomputed from a
    region that its owner had already overwritten in place would be wrong);
  * all 32 slots of the row carry one epoch, whatever split the next call uses.

A planted mistake (a workgroup storing its in-place residual before its part
is visible) must be caught, so the checker is shown to see the race it is for.
"""
import random

import pytest

SLOTS = 32           # slots in use per row record
EPOCH_MASK = 0xFFFFFFFF


class Row:
    """One row record and the row's in-place residual, region by region."""

    def __init__(self, epoch, nregions_max=SLOTS):
        self.slots = [(epoch, 0.0) for _ in range(SLOTS)]
        self.overwritten = [False] * nregions_max


def workgroup(row, s, sp, part_of, spin_limit, in_place, store_before_publish=False,
              epoch_from_slot0=False):
    """Workgroup s of a row split sp ways, as a generator: each `yield` is one
    step the scheduler may interleave with other workgroups' steps.  Returns
    its total through StopIteration.value.  The two keyword flags plant
    mistakes for the checker to catch."""
    # own slot: no other workgroup writes it during the call
    epoch = (row.slots[0 if epoch_from_slot0 else s][0] + 1) & EPOCH_MASK
    yield
    mine = part_of(s)
    if in_place and store_before_publish:   # the planted mistake
        row.overwritten[s] = True
        yield
    if not in_place:
        row.overwritten[s] = False           # a separate residual_out: inputs stay
    row.slots[s] = (epoch, mine)             # publish
    if s == 0:                               # stamp the slots this call leaves unused
        for k in range(sp, SLOTS):
            row.slots[k] = (epoch, 0.0)
    yield
    spins = 0
    total = None
    while spins < spin_limit:
        seen = [row.slots[k] for k in range(sp)]
        yield
        if all(e == epoch for e, _ in seen):
            total = sum(v for _, v in seen)
            break
        spins += 1
    if total is None:                        # gave up: take or recompute each part
        total = 0.0
        for s2 in range(sp):
            if s2 == s:
                total += mine
                continue
            e, v = row.slots[s2]
            yield
            if e == epoch:
                total += v
                continue
            clean = not row.overwritten[s2]  # the sibling's inputs as read now
            recomputed = part_of(s2) if clean else float("nan")
            yield
            e, v = row.slots[s2]             # read again once the inputs are in
            total += v if e == epoch else recomputed
    if in_place and not store_before_publish:
        row.overwritten[s] = True            # residual stored after the exchange
    yield
    return total


def run_call(rng, row, sp, spin_limit, in_place, store_before_publish=False, late=0.3,
             epoch_from_slot0=False):
    parts = [rng.uniform(0.5, 2.0) for _ in range(sp)]
    row.overwritten = [False] * SLOTS        # a fresh residual for this call
    gens = {s: workgroup(row, s, sp, lambda k: parts[k], spin_limit, in_place,
                         store_before_publish, epoch_from_slot0) for s in range(sp)}
    # some workgroups start late: they are only scheduled once the others have run a while
    start_after = {s: (rng.randint(1, 12) if rng.random() < late else 0) for s in gens}
    totals = {}
    step = 0
    while gens:
        ready = [s for s in gens if start_after[s] <= step] or list(gens)
        s = rng.choice(ready)
        try:
            next(gens[s])
        except StopIteration as stop:
            totals[s] = stop.value
            del gens[s]
        step += 1
    expected = sum(parts)
    return totals, expected


def check_row(row):
    epochs = {e for e, _ in row.slots}
    assert len(epochs) == 1, f"slots disagree on the epoch: {sorted(epochs)}"


@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_exchange_is_exact_under_random_interleavings(in_place):
    rng = random.Random(2024 + in_place)
    for trial in range(300):
        start = rng.choice([0, 7, EPOCH_MASK - 2, EPOCH_MASK])  # the wrap included
        row = Row(start)
        for call in range(6):
            sp = rng.choice([2, 3, 4, 7, 14, 32])
            spin_limit = rng.choice([0, 1, 2, 5, 1000])          # 0: give up at once
            totals, expected = run_call(rng, row, sp, spin_limit, in_place)
            for s, t in totals.items():
                assert t == pytest.approx(expected, rel=0, abs=1e-12), (trial, call, sp, s)
            check_row(row)
            assert row.slots[0][0] == (start + call + 1) & EPOCH_MASK


def test_late_workgroup_reads_its_own_calls_epoch():
    """Workgroups 0..2 run to the end before workgroup 3 starts: they give up
    waiting for it and recompute its part from its untouched region.  Then 3
    runs: it still reads this call's epoch from its own slot, sees every part
    published and finishes exactly; the next call exchanges normally."""
    rng = random.Random(7)
    row = Row(41)
    sp = 4
    parts = [1.0, 2.0, 3.0, 4.0]
    gens = {s: workgroup(row, s, sp, lambda k: parts[k], 3, True) for s in range(sp)}
    totals = {}
    for s in (0, 1, 2, 3):
        while True:
            try:
                next(gens[s])
            except StopIteration as stop:
                totals[s] = stop.value
                break
    assert totals == {0: 10.0, 1: 10.0, 2: 10.0, 3: 10.0}
    check_row(row)
    assert row.slots[0][0] == 42
    totals, expected = run_call(rng, row, 7, 1000, True, late=0.0)
    assert all(t == pytest.approx(expected) for t in totals.values())
    check_row(row)


def test_planted_mistake_store_before_publish_is_caught():
    """Storing the in-place residual before the part is visible lets a sibling
    that gave up recompute the part from an overwritten region; the model finds
    such an interleaving."""
    rng = random.Random(99)
    caught = False
    for _ in range(400):
        row = Row(rng.choice([0, 5]))
        totals, expected = run_call(rng, row, rng.choice([2, 4, 7]), rng.choice([0, 1]), True,
                                    store_before_publish=True)
        if any(t != t or abs(t - expected) > 1e-12 for t in totals.values()):
            caught = True
            break
    assert caught, "the checker did not see the in-place race"


def test_planted_mistake_shared_epoch_slot_is_caught():
    """Reading the epoch from slot 0 (written by workgroup 0 during the call)
    instead of the workgroup's own slot lets a late workgroup take the next
    call's epoch: the model finds a call that leaves the slots disagreeing or a
    total wrong."""
    rng = random.Random(5)
    caught = False
    for _ in range(400):
        row = Row(3)
        try:
            for _call in range(3):
                totals, expected = run_call(rng, row, rng.choice([2, 4, 7]), rng.choice([0, 1, 3]),
                                            False, late=0.6, epoch_from_slot0=True)
                if any(abs(t - expected) > 1e-12 for t in totals.values()):
                    raise AssertionError("wrong total")
                check_row(row)
        except AssertionError:
            caught = True
            break
    assert caught, "the checker did not see the late-workgroup epoch race"
