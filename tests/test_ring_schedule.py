"""Barrier audit of the GEMM's LDS ring (host only).

The GEMM kernel streams K-stages into a ring of LDS slots with direct
global -> LDS copies, waits for them with vmcnt counts, and synchronizes the
workgroup with s_barrier between the stage being consumed and the slot being
refilled.  Every wave runs the same program, so one wave's program, replayed
here event by event for every stage count nk, shows whether the waits and
barriers are enough:

* a stage's slot is read only after every copy of that stage completed (each
  wave waited for its own copies before a barrier the readers passed);
* a slot is refilled only after a barrier that follows every read of the
  stage it held (the waits before barriers also drain the LDS reads);
* between a stage's copies and its reads no copy of another stage lands in
  that slot;
* every stage is copied exactly once and read, and no copy is still in flight
  when the last stage has been read (a copy landing after the workgroup ends
  would write another workgroup's LDS).

The program below follows the kernel's structure (csrc/gemm_kernel.h): the
prologue, the steady-state loop of two phases per stage, the straight-line
last stages, and the generic loop for short K and 4-bit operands, with the
ring depths, copy counts and wait counts of every tile shape the library
builds.
"""

import pytest


def ring_params(bits: int, tn: int, waves: int):
    """(slots, copies per wave and stage, copies issued in phase 1) of a tile
    shape, from the stage sizes: a 32-row group chunk of a 128-element stage
    holds 16 * bits bytes per row, scales are 128 bytes per chunk."""
    chunk = 32 * 128 * bits // 8
    stage_x, stage_w = 8 * chunk, (tn // 32) * chunk
    scales_w = (tn // 32) * 128
    slot = stage_x + stage_w + 1024 + scales_w
    slots = 3 if tn == 256 and 3 * slot <= 160 * 1024 else 2
    copies = stage_x // 1024 // waves + stage_w // 1024 // waves + (1 if waves == 8 else 2)
    first = (copies + 1) // 2 if slots == 3 else copies
    return slots, copies, first


# every tile shape the library builds: (element bits, tile width, waves)
SHAPES = [(6, 256, 4), (6, 256, 8), (6, 128, 4), (4, 256, 4), (4, 256, 8), (8, 256, 4), (8, 256, 8)]


def program(nk: int, slots: int, copies: int, first: int, peeled: bool):
    """One wave's events: ("issue", stage, slot, copy), ("wait", vmcnt),
    ("barrier",), ("read", stage, slot)."""
    ev = []
    nxt = lambda s: 0 if s + 1 == slots else s + 1
    issue = lambda st, sl, a, n: ev.extend(("issue", st, sl, c) for c in range(a, a + n))
    read = lambda st, sl: ev.append(("read", st, sl))
    wait = lambda n: ev.append(("wait", n))
    barrier = lambda: ev.append(("barrier",))
    second = copies - first
    mid_wait = copies if slots == 3 else 0
    # prologue
    if nk > 0:
        issue(0, 0, 0, copies)
    if nk > 1:
        issue(1, 1, 0, copies)
    if slots == 3:
        if nk > 2:
            issue(2, 2, 0, first)
        wait(copies + first if nk > 2 else copies if nk > 1 else 0)
    else:
        wait(copies if nk > 1 else 0)
    barrier()
    if nk > 0:  # the kernel reads slot 0 unconditionally; with nk = 0 nothing is used
        read(0, 0)
    ks, slot = 0, 0
    # steady state: phase 0 (read this stage's second half, copy the rest of stage
    # ks + 2), wait + barrier, phase 1 (read stage ks + 1, start stage ks + slots in
    # the slot just consumed)
    while ks + slots < nk:
        nsl = nxt(slot)
        read(ks, slot)
        issue(ks + 2, nxt(nsl), first, second)
        wait(mid_wait)
        barrier()
        read(ks + 1, nsl)
        issue(ks + slots, slot, 0, first)
        slot = nsl
        ks += 1
    # the last ring-depth stages, straight-line
    if peeled and nk >= slots:
        if slots == 3:
            nsl = nxt(slot)
            read(ks, slot)
            issue(ks + 2, nxt(nsl), first, second)
            wait(copies)
            barrier()
            read(ks + 1, nsl)
            slot = nsl
            ks += 1
        nsl = nxt(slot)
        read(ks, slot)
        wait(0)
        barrier()
        read(ks + 1, nsl)
        slot = nsl
        ks += 1
        read(ks, slot)
        ks = nk
    # generic loop: K shorter than the ring, and the 4-bit operands' tail
    while ks < nk:
        nsl = nxt(slot)
        if slots == 3 and ks + 2 < nk:
            issue(ks + 2, nxt(nsl), first, second)
        read(ks, slot)
        if ks + 1 < nk:
            wait(copies if slots == 3 and ks + 2 < nk else 0)
            barrier()
            read(ks + 1, nsl)
        slot = nsl
        ks += 1
    return ev


def audit(ev, nk: int, copies: int):
    """Replays the events and returns the violations found (empty if none)."""
    bad = []
    issued = []                 # (stage, slot, copy) in issue order
    done = set()                # copies this wave has waited for
    visible = set()             # copies every wave had waited for at the last barrier
    last_read = {}              # slot -> (stage, event index) of the latest read
    barrier_after_wait = []     # event indices of barriers that follow a wait
    seen_wait = False
    first_issue = {}            # (stage, slot) -> event index of its first copy
    reads = set()
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "issue":
            _, st, sl, c = e
            if any(x == (st, sl, c) for x in issued):
                bad.append(f"stage {st} copy {c} issued twice")
            if not 0 <= st < nk:
                bad.append(f"copy of stage {st} outside 0..{nk - 1}")
            prev = last_read.get(sl)
            if prev is not None and prev[0] != st:
                # a barrier (after a wait, which drains the LDS reads) must separate them
                if not any(prev[1] < b < i for b in barrier_after_wait):
                    bad.append(f"slot {sl} refilled with stage {st} at event {i} before every wave "
                               f"finished reading stage {prev[0]}")
            issued.append((st, sl, c))
            first_issue.setdefault((st, sl), i)
        elif kind == "wait":
            n = e[1]
            done.update(issued[:max(len(issued) - n, 0)])
            seen_wait = True
        elif kind == "barrier":
            visible = set(done)
            if seen_wait:
                barrier_after_wait.append(i)
            seen_wait = False
        elif kind == "read":
            _, st, sl = e
            need = {(st, sl, c) for c in range(copies)}
            if not need <= visible:
                bad.append(f"stage {st} read from slot {sl} at event {i} before all of its copies landed")
            start = first_issue.get((st, sl))
            if start is not None:
                others = [x for j, x in enumerate(ev[start:i]) if x[0] == "issue" and x[2] == sl and x[1] != st]
                if others:
                    bad.append(f"slot {sl} overwritten by stage {others[0][1]} before stage {st} was read")
            last_read[sl] = (st, i)
            reads.add(st)
    for st in range(nk):
        if {(st, sl, c) for (s2, sl, c) in issued if s2 == st} and len([x for x in issued if x[0] == st]) != copies:
            bad.append(f"stage {st}: {len([x for x in issued if x[0] == st])} copies, not {copies}")
        if not any(x[0] == st for x in issued):
            bad.append(f"stage {st} never copied")
        if st not in reads:
            bad.append(f"stage {st} never read")
    if set(issued) - done:
        bad.append(f"{len(set(issued) - done)} copies still in flight after the last stage")
    return bad


@pytest.mark.parametrize("bits,tn,waves", SHAPES)
def test_ring_is_race_free_for_every_stage_count(bits, tn, waves):
    slots, copies, first = ring_params(bits, tn, waves)
    assert copies + first <= 63, "vmcnt counts at most 63 outstanding copies"
    for nk in list(range(0, 13)) + [24, 96, 97, 128]:
        ev = program(nk, slots, copies, first, peeled=bits != 4)
        assert audit(ev, nk, copies) == [], (bits, tn, waves, nk)


def test_ring_params_of_the_built_shapes():
    # the values the kernel's Ring<> works out (stage bytes / 1 KB per wave, plus scale copies)
    assert ring_params(6, 256, 4) == (3, 14, 7)
    assert ring_params(6, 256, 8) == (3, 7, 4)
    assert ring_params(6, 128, 4) == (2, 11, 11)
    assert ring_params(4, 256, 8) == (3, 5, 3)
    assert ring_params(8, 256, 4) == (2, 18, 18)


@pytest.mark.parametrize("mutation", ["mid_wait_too_loose", "no_mid_barrier", "refill_before_barrier",
                                      "prologue_wait_too_loose", "tail_wait_too_loose"])
def test_audit_catches_a_broken_schedule(mutation):
    """Plausible mistakes in the schedule, planted in this model (not in the
    kernel), each caught by the audit: it is not vacuous."""
    slots, copies, first = ring_params(6, 256, 8)
    nk = 24
    ev = program(nk, slots, copies, first, peeled=True)
    if mutation == "mid_wait_too_loose":
        i = next(i for i, e in enumerate(ev) if e == ("wait", copies) and i > 30)
        ev[i] = ("wait", copies + 1)
    elif mutation == "no_mid_barrier":
        i = next(i for i, e in enumerate(ev) if e == ("barrier",) and i > 30)
        del ev[i]
    elif mutation == "refill_before_barrier":
        # issue the phase-1 copies of one stage ahead of its barrier
        b = next(i for i, e in enumerate(ev) if e == ("barrier",) and i > 40)
        j = next(i for i in range(b, len(ev)) if ev[i][0] == "issue" and ev[i][3] == 0)
        ev.insert(b - 1, ev.pop(j))
    elif mutation == "prologue_wait_too_loose":
        i = next(i for i, e in enumerate(ev) if e[0] == "wait")
        ev[i] = ("wait", ev[i][1] + 1)
    elif mutation == "tail_wait_too_loose":
        i = max(i for i, e in enumerate(ev) if e == ("wait", 0))
        ev[i] = ("wait", 1)
    assert audit(ev, nk, copies) != []
