"""The set schedule of the GEMM whose waves split K (``gemm_wsplit_kernel`` in
``csrc/gemm.hip``, both its 64 x 64 and 128 x 128 forms), checked on the host for every
number of sets from 1 to 12.

The kernel loads a set (KS stages of K) into one of two LDS buffer groups while the waves
compute the previous one. All four waves run the same sequence of loads, waits, barriers
and LDS reads, so the schedule is modelled as one event list in which a barrier is a point
every wave reaches; the checks are the ones the kernel's correctness rests on:

* every set is loaded once, into the group its compute reads;
* a group is read for a set only after that set's loads were waited for (each wave waits
  for its own loads) and a barrier followed, and before anything else is loaded into it;
* loads into a group start only after a barrier that follows the last read of what the group
  held before;
* the epilogue reuses the LDS only after a barrier that follows every read and every
  wait for the loads.
"""
import pytest


def schedule(nset):
    """The kernel's event list: ("load", set, group), ("wait",), ("barrier",),
    ("read", set, group), ("reduce",)."""
    ev = []
    ev.append(("load", 0, 0))
    if nset > 1:
        ev.append(("load", 1, 1))
        ev.append(("wait", 0))       # vmcnt(kLoads): set 0 landed, set 1 may be in flight
    else:
        ev.append(("wait", None))    # vmcnt(0)
    ev.append(("barrier",))
    ev.append(("read", 0, 0))        # set 0's first chunk

    def run_set(t, pr, loads, last):
        ev.append(("read", t, pr))   # k-step 0: the stage's second chunk
        if not last:                 # k-step 4
            ev.append(("wait", None))
            ev.append(("barrier",))
            ev.append(("read", t + 1, pr ^ 1))
        if loads:                    # k-steps 4 .. 7
            ev.append(("load", t + 2, pr))

    t = 0
    while t + 4 <= nset:
        run_set(t, 0, True, False)
        run_set(t + 1, 1, True, False)
        t += 2
    rest = nset - t
    if rest == 3:
        run_set(t, 0, True, False)
        run_set(t + 1, 1, False, False)
        run_set(t + 2, 0, False, True)
    elif rest == 2:
        run_set(t, 0, False, False)
        run_set(t + 1, 1, False, True)
    else:
        assert rest == 1
        run_set(t, 0, False, True)
    ev.append(("wait", None))
    ev.append(("barrier",))
    ev.append(("reduce",))
    return ev


def check(ev, nset):
    """Raise AssertionError where the event list breaks one of the rules above."""
    content = {0: None, 1: None}          # set last loaded into each group
    outstanding = []                      # loads issued and not yet waited for, in order
    landed_unsynced = set()               # sets waited for by the waves, no barrier since
    visible = set()                       # sets every wave may read
    last_read = {0: -2, 1: -2}            # event index of the last read of each group (none yet)
    last_barrier = -1
    loaded = []
    reads = {}
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "load":
            _, s, p = e
            assert s < nset, f"set {s} past the end is loaded"
            assert last_read[p] < last_barrier, f"set {s} loaded into group {p} before a barrier after its last read"
            content[p] = s
            visible.discard(s)
            outstanding.append(s)
            loaded.append(s)
        elif kind == "wait":
            if e[1] is None:
                landed_unsynced.update(outstanding)
                outstanding = []
            else:
                # vmcnt(kLoads): all but the most recent set's loads have landed
                landed_unsynced.update(outstanding[:-1])
                outstanding = outstanding[-1:]
                assert e[1] in landed_unsynced
        elif kind == "barrier":
            visible |= landed_unsynced
            landed_unsynced = set()
            last_barrier = i
        elif kind == "read":
            _, s, p = e
            if s >= nset:
                continue
            assert content[p] == s, f"set {s} read from group {p} holding set {content[p]}"
            assert s in visible, f"set {s} read before its loads were waited for and synchronized"
            last_read[p] = i
            reads[s] = reads.get(s, 0) + 1
        elif kind == "reduce":
            assert not outstanding, "loads in flight when the LDS is reused"
            assert max(last_read.values()) < last_barrier, "LDS reused before a barrier after the last read"
    assert sorted(loaded) == list(range(nset)), f"sets loaded: {sorted(loaded)}"
    assert all(reads.get(s) == 2 for s in range(nset)), f"chunk reads per set: {reads}"


@pytest.mark.parametrize("nset", range(1, 13))
def test_wsplit_set_schedule(nset):
    check(schedule(nset), nset)


def _mutations(ev):
    """Event lists with one plausible mistake each: a load into the other buffer group, a
    dropped wait before a barrier (the final one aside: no load is in flight there), a
    read moved ahead of the barrier it follows."""
    out = []
    for i, e in enumerate(ev):
        if e[0] == "load" and e[1] >= 2:
            out.append(ev[:i] + [("load", e[1], e[2] ^ 1)] + ev[i + 1:])
        if e[0] == "wait" and ev[i + 1][0] == "barrier" and 5 < i < len(ev) - 3:
            out.append(ev[:i] + ev[i + 1:])
        if e[0] == "barrier" and i + 1 < len(ev) and ev[i + 1][0] == "read" and i > 5:
            out.append(ev[:i - 1] + [ev[i + 1], ev[i - 1], e] + ev[i + 2:])
    return out


@pytest.mark.parametrize("nset", [3, 6, 7])
def test_wsplit_schedule_check_catches_mistakes(nset):
    muts = _mutations(schedule(nset))
    assert len(muts) >= 3
    for m in muts:
        with pytest.raises(AssertionError):
            check(m, nset)
