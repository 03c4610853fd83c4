"""Pins of the oracle LRU (ensure_experts) and copy_missing.

1. A hand-worked trace (tests/golden/lru_trace_s3_e3.txt).
2. An independent textbook LRU - a recency list with move-to-MRU, written here
   without timestamps - must agree step for step with the timestamp oracle on
   random traces and on every short trace of a tiny pool.
3. Invariants: every requested id resident afterwards, owners unique, no
   member of the request evicted, copies == misses, capacity failure leaves the
   state unchanged, only cold misses when the pool holds every id.
4. ensure_experts_hybrid: a hand-worked trace (tests/golden/
   lru_hybrid_trace_s3_e4.txt); on random traces it equals the plain LRU step on
   the requests that keep a slot (overflow pairs map to -1); with a cap at or
   above the misses it equals the plain step; the cap's closed forms.
5. Slot-pool resize: a hand-worked example (tests/golden/lru_resize_s5.txt);
   the LRU stack property - a table shrunk to S' holds exactly what an
   independent textbook LRU of S' slots holds after the same trace, and both
   miss the same ids afterwards; a grown table behaves step for step like a
   textbook LRU of the larger size given the same contents; the slot bytes
   follow the slot map.
"""
import itertools
import os
import random

import numpy as np
import pytest

from oracle import copy as ocopy
from oracle import formulas
from oracle.lru import ERR_ARG, ERR_CAPACITY, OK, SlotTable, hybrid_cap

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints(s):
    return [int(v) for v in s.split(",")] if s.strip() not in ("", "-") else None


def _rows(s):
    s = s.strip()
    return None if s == "-" else [_ints(r) for r in s.split(";")]


def test_hand_worked_trace():
    lines = [l.split("#")[0].strip() for l in open(os.path.join(GOLDEN, "lru_trace_s3_e3.txt"))]
    lines = [l for l in lines if l]
    pool = dict(kv.split("=") for kv in lines[0].split()[1:])
    t = SlotTable(int(pool["S"]), int(pool["L"]), int(pool["E"]))
    init = dict(kv.split("=") for kv in lines[1].split()[1:])
    t.set_state(_ints(init["owner"]), _ints(init["stamp"]), int(init["clock"]))
    for line in lines[2:]:
        lhs, rhs = line.split("->")
        _, layer, ids = lhs.split()
        status, slots, misses, owner, stamp, ev = [p.strip() for p in rhs.split("|")]
        r = t.ensure(int(layer), _rows(ids))
        assert r.status == int(status), line
        if r.status == OK:
            assert r.slot_ids.tolist() == _rows(slots), line
            want = [tuple(int(v) for v in m.split(":")) for m in misses.split()]
            assert r.misses == want, line
            assert r.evictions == int(ev), line
        assert t.owner.tolist() == _ints(owner), line
        assert t.stamp.tolist() == _ints(stamp), line


def test_capacity_leaves_state():
    t = SlotTable(2, 1, 3)
    before = t.snapshot()
    r = t.ensure(0, [[0, 1, 2]])
    assert r.status == ERR_CAPACITY
    after = t.snapshot()
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    assert before[2] == after[2]
    # exactly S distinct ids fit
    assert t.ensure(0, [[0, 1]]).status == OK


def test_arg_errors():
    t = SlotTable(4, 2, 3)
    assert t.ensure(2, [[0]]).status == ERR_ARG
    assert t.ensure(-1, [[0]]).status == ERR_ARG
    assert t.ensure(0, [[3]]).status == ERR_ARG
    assert t.ensure(0, [[-1]]).status == ERR_ARG


class TextbookLRU:
    """Recency list (LRU first) with move-to-MRU; no timestamps.

    Batch rule: misses (ascending) take victims from the LRU end, skipping
    slots that hold requested ids; then the slots of all requested ids move to
    the MRU end in ascending id order.  Empty slots start at the LRU end.
    """

    def __init__(self, S, L, E, owner=None, order=None):
        self.S, self.L, self.E = S, L, E
        self.owner = list(owner) if owner is not None else [-1] * S
        self.order = list(order) if order is not None else list(range(S))

    def step(self, layer, ids):
        flat = [[layer * self.E + e for e in row] for row in ids]
        U = sorted({f for row in flat for f in row})
        pos = {o: s for s, o in enumerate(self.owner) if o >= 0}
        miss = [u for u in U if u not in pos]
        victims = [s for s in self.order if self.owner[s] not in U]
        if len(miss) > len(victims):
            return None
        installs = []
        for u, s in zip(miss, victims):
            self.owner[s] = u
            pos[u] = s
            installs.append((s, u))
        for u in U:
            self.order.remove(pos[u])
            self.order.append(pos[u])
        return [[pos[f] for f in row] for row in flat], installs


def _compare_trace(S, L, E, steps):
    a = SlotTable(S, L, E)
    b = TextbookLRU(S, L, E)
    for layer, ids in steps:
        ra = a.ensure(layer, ids)
        rb = b.step(layer, ids)
        if rb is None:
            assert ra.status == ERR_CAPACITY
            continue
        assert ra.status == OK
        assert ra.slot_ids.tolist() == rb[0]
        assert ra.misses == rb[1]
        assert a.owner.tolist() == b.owner


def test_random_traces_against_textbook_lru():
    rng = random.Random(1234)
    for _ in range(100):
        L, E, S = rng.randint(1, 3), rng.randint(1, 6), rng.randint(1, 5)
        steps = []
        for _ in range(100):
            n, k = rng.randint(1, 3), rng.randint(1, 2)
            steps.append((rng.randrange(L), [[rng.randrange(E) for _ in range(k)] for _ in range(n)]))
        _compare_trace(S, L, E, steps)


def test_exhaustive_short_traces():
    L, E = 2, 3
    singles = [(l, [[e]]) for l in range(L) for e in range(E)]
    pairs = [(l, [[e1, e2]]) for l in range(L) for e1 in range(E) for e2 in range(E)]
    alphabet = singles + pairs
    for S in (1, 2, 3):
        for length in (1, 2, 3):
            for trace in itertools.product(alphabet, repeat=length):
                _compare_trace(S, L, E, list(trace))
    # length-4 traces over single requests
    for S in (1, 2, 3):
        for trace in itertools.product(singles, repeat=4):
            _compare_trace(S, L, E, list(trace))


def test_invariants_random():
    rng = np.random.default_rng(7)
    for _ in range(200):
        L, E = int(rng.integers(1, 4)), int(rng.integers(2, 9))
        S = int(rng.integers(1, 10))
        t = SlotTable(S, L, E)
        for _ in range(30):
            layer = int(rng.integers(L))
            ids = rng.integers(0, E, size=(int(rng.integers(1, 4)), int(rng.integers(1, 3))))
            before = t.snapshot()
            U = sorted(set((layer * E + ids).ravel().tolist()))
            r = t.ensure(layer, ids)
            if r.status == ERR_CAPACITY:
                assert len(U) > S
                assert np.array_equal(before[0], t.owner) and np.array_equal(before[1], t.stamp)
                continue
            assert r.status == OK
            owners = [o for o in t.owner.tolist() if o >= 0]
            assert len(owners) == len(set(owners))
            for u in U:
                assert u in owners
            # requested ids that were resident stayed in their slots
            for s, o in enumerate(before[0].tolist()):
                if o in U:
                    assert t.owner[s] == o
            assert len(r.misses) == len(U) - r.hits
            assert np.array_equal(t.owner[r.slot_ids], layer * E + ids)


def test_only_cold_misses_when_pool_holds_everything():
    L, E = 2, 4
    t = SlotTable(L * E, L, E)
    seen = set()
    rng = np.random.default_rng(3)
    for _ in range(200):
        layer = int(rng.integers(L))
        ids = rng.integers(0, E, size=(2, 2))
        flat = set((layer * E + ids).ravel().tolist())
        r = t.ensure(layer, ids)
        assert {m[1] for m in r.misses} == flat - seen
        seen |= flat


def test_copy_missing_moves_rows_and_keeps_sentinel():
    E, S = 5, 4
    rng = np.random.default_rng(0)
    row_bytes = [32, 16]
    host = [[rng.integers(0, 256, size=(E, rb), dtype=np.uint8)] for rb in row_bytes]
    slots = [np.full((S, rb), 0xA5, dtype=np.uint8) for rb in row_bytes]
    t = SlotTable(S, 1, E)
    r = t.ensure(0, [[4, 1]])
    moved = ocopy.copy_missing(r.misses, host, slots, E)
    assert moved == 2 * sum(row_bytes)
    touched = {s for s, _ in r.misses}
    for b in range(2):
        for s in range(S):
            if s in touched:
                fid = dict(r.misses)[s]
                assert np.array_equal(slots[b][s], host[b][0][fid])
            else:
                assert (slots[b][s] == 0xA5).all()


def test_zero_and_full_miss_rate():
    E, S, n, k = 16, 8, 4, 2
    active = formulas.active_unique(n, k, E)
    assert formulas.num_misses(active, 0.0) == 0
    assert formulas.num_misses(active, 1.0) == active


# ------------------------------------------------------------------ hybrid
def test_hybrid_hand_worked_trace():
    lines = [l.split("#")[0].strip() for l in open(os.path.join(GOLDEN, "lru_hybrid_trace_s3_e4.txt"))]
    lines = [l for l in lines if l]
    pool = dict(kv.split("=") for kv in lines[0].split()[1:])
    t = SlotTable(int(pool["S"]), int(pool["L"]), int(pool["E"]))
    init = dict(kv.split("=") for kv in lines[1].split()[1:])
    t.set_state(_ints(init["owner"]), _ints(init["stamp"]), int(init["clock"]))
    for line in lines[2:]:
        lhs, rhs = line.split("->")
        _, layer, ids, mf, frac = lhs.split()
        slots, misses, over, ni, nf, owner, stamp, clock, ev = [p.strip() for p in rhs.split("|")]
        r = t.ensure_hybrid(int(layer), _rows(ids), int(mf), None if frac == "-" else float(frac))
        assert r.status == OK, line
        assert r.slot_ids.tolist() == _rows(slots), line
        want = [] if misses == "-" else [tuple(int(v) for v in m.split(":")) for m in misses.split()]
        assert r.misses == want, line
        assert r.overflow == (_ints(over) or []), line
        assert (r.num_indices, r.num_missing_full, r.evictions) == (int(ni), int(nf), int(ev)), line
        assert t.owner.tolist() == _ints(owner), line
        assert t.stamp.tolist() == _ints(stamp), line
        assert t.clock == int(clock), line


def test_hybrid_cap_closed_forms():
    assert hybrid_cap(7, 3) == 3 and hybrid_cap(7, 0) == 0 and hybrid_cap(2, 9) == 9
    assert hybrid_cap(7, -1) == 1 and hybrid_cap(0, -1) == 1          # no profile: a fixed cap of one
    assert hybrid_cap(5, -1, 0.5) == 2 and hybrid_cap(3, -1, 0.5) == 2  # 2.5 -> 2, 1.5 -> 2 (half to even)
    assert hybrid_cap(4, -1, 2.0) == 4 and hybrid_cap(8, -1, 0.0) == 0
    assert formulas.hybrid_fetch_fraction(25.0, 100.0) == 0.25
    assert formulas.hybrid_fetch_fraction(55.0, 50.0) == 1.0
    # the ideal overlap of the pages: fetched : cpu = pcie : (cpu - pcie)
    f = formulas.hybrid_fetch_fraction(30.0, 80.0)
    assert abs(f / (1 - f) - 30.0 / (80.0 - 30.0)) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_hybrid_equals_plain_step_on_kept_requests(seed):
    rng = random.Random(seed)
    S, L, E = rng.randint(2, 12), rng.randint(1, 3), rng.randint(3, 16)
    th, tp = SlotTable(S, L, E), SlotTable(S, L, E)
    for _ in range(60):
        layer = rng.randrange(L)
        k = rng.randint(1, 4)
        ids = np.array([[rng.randrange(E) for _ in range(k)] for _ in range(rng.randint(1, 3))])
        mf = rng.choice([-1, 0, 1, 2, 5])
        frac = rng.choice([None, 0.0, 0.25, 0.5, 1.0])
        r = th.ensure_hybrid(layer, ids, mf, frac)
        assert r.status == OK
        over = set(r.overflow)
        assert len(over) == r.num_missing_full - r.num_indices
        keep = [[int(v) for v in row if layer * E + int(v) not in over] for row in ids]
        flat_keep = [v for row in keep for v in row]
        if flat_keep:
            rp = tp.ensure(layer, np.array([flat_keep]))
            assert rp.status == OK
            assert rp.misses == r.misses
            got = [s for row in r.slot_ids.tolist() for s in row if s >= 0]
            assert got == rp.slot_ids.ravel().tolist()
        else:
            tp.clock += 1            # a step that keeps nothing still advances the clock
        assert all(s == -1 for row, srow in zip(ids, r.slot_ids.tolist()) for v, s in zip(row, srow)
                   if layer * E + int(v) in over)
        assert np.array_equal(th.owner, tp.owner) and np.array_equal(th.stamp, tp.stamp) and th.clock == tp.clock


def test_hybrid_without_cap_equals_plain():
    rng = random.Random(9)
    S, L, E = 10, 2, 8
    th, tp = SlotTable(S, L, E), SlotTable(S, L, E)
    for _ in range(40):
        layer = rng.randrange(L)
        ids = np.array([[rng.randrange(E) for _ in range(3)] for _ in range(2)])
        r, rp = th.ensure_hybrid(layer, ids, 64), tp.ensure(layer, ids)
        assert rp.status == OK and r.status == OK and r.overflow == []
        assert r.slot_ids.tolist() == rp.slot_ids.tolist() and r.misses == rp.misses
        assert r.num_indices == r.num_missing_full == len(rp.misses)


# ------------------------------------------------------------------ resize
def _golden_resize():
    lines = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "lru_resize_s5.txt"))]
    return [l for l in lines if l]


def _fields(tokens):
    out, key = {}, None
    for tok in tokens:
        if tok.lstrip("-").isdigit() or ":" in tok:
            out[key].append(tok)
        else:
            key = tok
            out[key] = []
    return out


def test_resize_hand_worked():
    lines = _golden_resize()
    owner = [int(v) for v in lines[0][1:]]
    stamp = [int(v) for v in lines[1][1:]]
    clock = int(lines[2][1])
    for line in lines[3:]:
        t = SlotTable(len(owner), 1, 10)
        t.set_state(owner, stamp, clock)
        f = _fields(line)
        if line[0] == "resize":
            src = t.resize(int(f["resize"][0]))
            assert src == [int(v) for v in f["src"]]
            assert t.owner.tolist() == [int(v) for v in f["owner"]]
            assert t.stamp.tolist() == [int(v) for v in f["stamp"]]
            assert t.clock == clock and t.S == len(src)
        else:  # a step after the shrink to 3
            t.resize(3)
            r = t.ensure(0, [[int(v) for v in f["ids"]]])
            assert r.status == OK
            assert r.slot_ids.tolist() == [[int(v) for v in f["slots"]]]
            assert r.misses == [tuple(int(x) for x in m.split(":")) for m in f["misses"]]
            assert t.owner.tolist() == [int(v) for v in f["owner"]]
            assert t.stamp.tolist() == [int(v) for v in f["stamp"]]
            assert t.clock == int(f["clock"][0])


def _trace(rng, L, E, steps, max_distinct):
    out = []
    for _ in range(steps):
        layer = rng.randrange(L)
        n, k = rng.randint(1, 2), rng.randint(1, 2)
        while True:
            ids = [[rng.randrange(E) for _ in range(k)] for _ in range(n)]
            if len({e for r in ids for e in r}) <= max_distinct:
                break
        out.append((layer, ids))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_shrink_holds_what_a_smaller_lru_holds(seed):
    """LRU is a stack algorithm: after any trace, a pool of S' slots holds the S'
    most recently used ids, whatever larger pool ran beside it."""
    rng = random.Random(100 + seed)
    for _ in range(40):
        L, E = rng.randint(1, 3), rng.randint(2, 7)
        S = rng.randint(2, 8)
        S2 = rng.randint(1, S)
        before = _trace(rng, L, E, rng.randint(0, 30), min(S2, 4))
        after = _trace(rng, L, E, 20, min(S2, 4))
        big, small = SlotTable(S, L, E), TextbookLRU(S2, L, E)
        for layer, ids in before:
            assert big.ensure(layer, ids).status == OK
            assert small.step(layer, ids) is not None
        src = big.resize(S2)
        assert sorted(o for o in big.owner.tolist() if o >= 0) == sorted(o for o in small.owner if o >= 0)
        assert len(src) == S2 and sorted(s for s in src if s >= 0) == [s for s in src if s >= 0]
        for layer, ids in after:
            ra = big.ensure(layer, ids)
            rb = small.step(layer, ids)
            assert ra.status == OK and rb is not None
            assert sorted(m[1] for m in ra.misses) == sorted(m[1] for m in rb[1])
            assert sorted(o for o in big.owner.tolist() if o >= 0) == sorted(o for o in small.owner if o >= 0)


@pytest.mark.parametrize("seed", range(4))
def test_grow_behaves_like_a_larger_lru(seed):
    rng = random.Random(200 + seed)
    for _ in range(40):
        L, E = rng.randint(1, 3), rng.randint(2, 8)
        S = rng.randint(1, 5)
        S2 = S + rng.randint(0, 4)
        t = SlotTable(S, L, E)
        for layer, ids in _trace(rng, L, E, rng.randint(0, 20), min(S, 4)):
            assert t.ensure(layer, ids).status == OK
        owner_before, stamp_before = t.owner.copy(), t.stamp.copy()
        src = t.resize(S2)
        assert src == list(range(S)) + [-1] * (S2 - S)
        assert t.owner[:S].tolist() == owner_before.tolist() and (t.owner[S:] == -1).all()
        assert t.stamp[:S].tolist() == stamp_before.tolist()
        # the textbook LRU's recency list: empty slots by index, then by (stamp, owner)
        empty = [s for s in range(S2) if t.owner[s] == -1]
        used = sorted((s for s in range(S2) if t.owner[s] >= 0), key=lambda s: (int(t.stamp[s]), int(t.owner[s])))
        ref = TextbookLRU(S2, L, E, owner=t.owner.tolist(), order=empty + used)
        for layer, ids in _trace(rng, L, E, 20, min(S2, 5)):
            ra, rb = t.ensure(layer, ids), ref.step(layer, ids)
            if rb is None:
                assert ra.status == ERR_CAPACITY
                continue
            assert ra.status == OK
            assert ra.slot_ids.tolist() == rb[0] and ra.misses == rb[1]


def test_resize_same_size_and_round_trip():
    rng = np.random.default_rng(3)
    t = SlotTable(6, 2, 5)
    for _ in range(12):
        t.ensure(int(rng.integers(2)), rng.integers(0, 5, size=(1, 2)))
    o, st, c = t.snapshot()
    assert t.resize(6) == list(range(6))
    assert t.owner.tolist() == o.tolist() and t.stamp.tolist() == st.tolist() and t.clock == c
    kept = t.resize(3)
    survivors = {int(o[s]) for s in kept if o[s] >= 0}
    t.resize(9)
    assert {int(v) for v in t.owner.tolist() if v >= 0} == survivors
    with pytest.raises(ValueError):
        t.resize(0)


def test_resize_moves_slot_bytes():
    rng = np.random.default_rng(5)
    banks = [rng.integers(0, 256, size=(5, rb), dtype=np.uint8) for rb in (32, 16)]
    t = SlotTable(5, 1, 10)
    t.set_state([7, -1, 3, 9, 4], [2, 0, 5, 5, 1], 5)
    src = t.resize(3)
    new = ocopy.resize_slots(banks, src)
    for b in range(2):
        assert np.array_equal(new[b], banks[b][[0, 2, 3]])
    grown = ocopy.resize_slots(banks, list(range(5)) + [-1])
    for b in range(2):
        assert np.array_equal(grown[b][:5], banks[b]) and (grown[b][5] == 0xA5).all()
