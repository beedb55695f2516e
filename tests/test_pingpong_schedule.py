"""The ping-pong schedule of the prefill and backward kernels, checked on a
host model of its events (no GPU).

Both the prefill (tiles 0..T) and the backward kernels (dK/dV items, dQ
tiles) run their two wave groups as

    group 0:  for t in 0..n-1: start(t); products(t); vector(t)
              start(n); products(n)
    group 1:  start(0); products(0)
              for t in 0..n-1: start(t + 1); vector(t); products(t + 1)

where start(t) = [wait for this wave's loads of t (group 0 may leave the
loads of t + 1 in flight, group 1 none), when t < n] + barrier;
products(t) reads unit t's first operands (t < n) and unit t - 1's second
operands (t >= 1); vector(t) issues this wave's loads of unit t + 2 into the
stage (t + 2) mod 4 (when t + 2 < n).  Units 0 and 1 are loaded before the
loop.  The model replays that order per group and checks, for every n, that
the groups meet the same number of barriers, that every read of a unit
happens after a barrier both groups reached after their loads of it were
complete, and that no load lands in a stage before every read of the unit
that held it is past a barrier.
"""
import pytest

STAGES = 4


def events(group, n):
    """Per-wave event list: ('bar',), ('wait', unit set still allowed in flight
    is implied by the rule), ('load', u), ('read', u)."""
    ev = []
    issued = [0, 1][: min(n, 2)]
    ev += [("load", u) for u in issued]

    def start(t):
        if t < n:
            ev.append(("wait", t, group == 0 and t + 1 < n))
        ev.append(("bar",))

    def products(t):
        if t >= 1:
            ev.append(("read", t - 1))
        if t < n:
            ev.append(("read", t))

    def vector(t):
        if t + 2 < n:
            ev.append(("load", t + 2))

    if group == 0:
        for t in range(n):
            start(t)
            products(t)
            vector(t)
        start(n)
        products(n)
    else:
        start(0)
        products(0)
        for t in range(n):
            start(t + 1)
            vector(t)
            products(t + 1)
    return ev


def replay(group, n):
    """Interval index (number of barriers passed) of each load issue, each
    completed wait and each read, for one wave of `group`."""
    ev = events(group, n)
    interval = 0
    in_flight = []  # units whose loads this wave issued and has not waited for, in issue order
    loaded_at, done_by, reads = {}, {}, {}
    for e in ev:
        if e[0] == "bar":
            interval += 1
        elif e[0] == "load":
            loaded_at[e[1]] = interval
            in_flight.append(e[1])
        elif e[0] == "wait":
            t, keep_one = e[1], e[2]
            # the hardware counter retires loads in issue order: waiting until
            # at most one unit's loads are pending completes all older ones
            keep = 1 if keep_one else 0
            while len(in_flight) > keep:
                done_by[in_flight.pop(0)] = interval
            assert t in done_by, f"group {group}, n {n}: the wait before unit {t} leaves it in flight"
        else:
            reads.setdefault(e[1], []).append(interval)
    return interval, loaded_at, done_by, reads


@pytest.mark.parametrize("n", list(range(1, 40)) + [63, 64, 65, 257])
def test_pingpong_schedule(n):
    r0 = replay(0, n)
    r1 = replay(1, n)
    assert r0[0] == r1[0], "both groups meet the same number of barriers"
    for u in range(n):
        # complete in every wave before the barrier that precedes the first read
        first_read = min(min(r[3].get(u, [10 ** 9])) for r in (r0, r1))
        for r in (r0, r1):
            assert u in r[2] and r[2][u] < first_read, f"unit {u} read before its loads are waited for"
        # its stage is taken over by unit u + 4, whose loads must come after
        # every read of u, with a barrier in between
        if u + STAGES < n:
            last_read = max(max(r[3][u]) for r in (r0, r1))
            for r in (r0, r1):
                assert r[1][u + STAGES] > last_read, f"unit {u + STAGES} overwrites unit {u} while it is read"
        # every unit is read by both groups: first operands, then second
        for r in (r0, r1):
            assert len(r[3][u]) == 2
