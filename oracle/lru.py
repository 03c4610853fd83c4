"""ensure_experts: the global LRU remap of flat expert ids onto a fixed slot pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FreeToken MoE benchmark guide §4.1 and §4.3, FreeToken architecture
walk-through §5: the GPU holds one expert slot cache shared by every layer;
experts are named by a flat id (layer * E + expert); a step remaps the routed
experts onto slots with a global LRU policy, and the missing ones are then
gathered from the host banks.

The pages give the policy (LRU), not its batch rules.  The readings taken here
(all "parity unpinned" against the pages, pinned against a textbook LRU in the
tests) are:

  * a step first forms U, the sorted set of distinct flat ids it requests;
  * ids already owned by a slot are hits; the others, M, are missing, taken in
    ascending id order;
  * slots whose owner is not in U may be evicted; they are ordered by
    (not empty, stamp, owner, slot) - empty slots first, then least recently
    used, ties broken by lower owner id and then lower slot index;
  * the i-th missing id takes the i-th slot of that order;
  * if there are more misses than evictable slots the step fails with a
    capacity error and changes nothing;
  * on success the clock advances by one and every slot owning a member of U
    gets the new clock value as its stamp.
"""
from dataclasses import dataclass, field

import numpy as np

OK, ERR_ARG, ERR_CAPACITY = 0, -1, -2


@dataclass
class EnsureResult:
    status: int
    slot_ids: np.ndarray = None          # int32 [n, k], slot owning each request (-1: not fetched)
    misses: list = field(default_factory=list)   # [(slot, flat_id)] in install order
    hits: int = 0
    evictions: int = 0                   # misses that displaced a non-empty slot
    num_indices: int = 0                 # hybrid: misses fetched this step (within the cap)
    num_missing_full: int = 0            # hybrid: misses before the cap
    overflow: list = field(default_factory=list)  # hybrid: flat ids left to the CPU executor, ascending


def hybrid_cap(num_missing_full: int, max_fetch: int, fetch_fraction=None) -> int:
    """Fetch cap of a hybrid step (FreeToken MoE benchmark guide §5.4): an explicit
    hybrid_max_fetch >= 0 is the cap; otherwise the measured fetch fraction
    (pcie_bw / cpu_bw, at most 1) of this step's misses, rounded half to even;
    with no fraction (no bandwidth profile) a fixed cap of one."""
    if max_fetch >= 0:
        return int(max_fetch)
    if fetch_fraction is None or fetch_fraction < 0:
        return 1
    return int(round(num_missing_full * min(1.0, float(fetch_fraction))))


class SlotTable:
    """State of the slot pool: owner (int64, -1 = empty) and stamp (uint64) per slot, plus a clock."""

    def __init__(self, num_slots: int, num_layers: int, num_experts: int):
        self.S, self.L, self.E = int(num_slots), int(num_layers), int(num_experts)
        self.owner = np.full(self.S, -1, dtype=np.int64)
        self.stamp = np.zeros(self.S, dtype=np.uint64)
        self.clock = 0

    def set_state(self, owner, stamp, clock=None):
        self.owner = np.array(owner, dtype=np.int64).copy()
        self.stamp = np.array(stamp, dtype=np.uint64).copy()
        if clock is None:
            clock = int(self.stamp.max()) if self.S else 0
        self.clock = int(clock)

    def snapshot(self):
        return self.owner.copy(), self.stamp.copy(), self.clock

    def resize(self, num_slots: int) -> list:
        """Runtime resize of the slot pool (FreeToken architecture walk-through §4:
        VRAM moves between the expert cache and the KV cache at run time, with no
        restart and no weight reload).

        Readings (the page names the feature only): growing keeps every slot
        where it is and appends empty slots; shrinking keeps the num_slots slots
        that come last in the victim order of ensure() - empty slots leave
        first, then the least recently used - and packs them, in ascending old
        index, into slots [0, num_slots).  Stamps and the clock are kept, so the
        kept experts keep their LRU order; the experts of the dropped slots are
        no longer resident.

        Returns src: new slot i holds what old slot src[i] held (-1: a new,
        empty slot)."""
        num_slots = int(num_slots)
        if num_slots < 1:
            raise ValueError("num_slots must be positive")
        if num_slots >= self.S:
            src = list(range(self.S)) + [-1] * (num_slots - self.S)
        else:
            order = sorted(range(self.S), key=lambda s: (int(self.owner[s]) != -1, int(self.stamp[s]),
                                                         int(self.owner[s]), s))
            src = sorted(order[self.S - num_slots:])
        owner = np.full(num_slots, -1, dtype=np.int64)
        stamp = np.zeros(num_slots, dtype=np.uint64)
        for i, s in enumerate(src):
            if s >= 0:
                owner[i] = self.owner[s]
                stamp[i] = self.stamp[s]
        self.owner, self.stamp, self.S = owner, stamp, num_slots
        return src

    def ensure(self, layer: int, ids) -> EnsureResult:
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim == 1:
            ids = ids[None, :]
        # step 1: validate the request and form flat ids
        if not (0 <= layer < self.L) or ids.size and (ids.min() < 0 or ids.max() >= self.E):
            return EnsureResult(status=ERR_ARG)
        flat = layer * self.E + ids
        # step 2: distinct requested ids, ascending
        U = sorted(set(int(f) for f in flat.ravel()))
        in_U = set(U)
        where = {int(o): s for s, o in enumerate(self.owner) if o >= 0}
        # step 3: hits and misses
        missing = [u for u in U if u not in where]
        # step 4-5: evictable slots in victim order
        evictable = [s for s in range(self.S) if int(self.owner[s]) not in in_U]
        evictable.sort(key=lambda s: (int(self.owner[s]) != -1, int(self.stamp[s]),
                                      int(self.owner[s]), s))
        # step 6: capacity
        if len(missing) > len(evictable):
            return EnsureResult(status=ERR_CAPACITY)
        # step 7: install
        installs, evictions = [], 0
        for i, u in enumerate(missing):
            s = evictable[i]
            if self.owner[s] != -1:
                evictions += 1
            self.owner[s] = u
            where[u] = s
            installs.append((s, u))
        # step 8: stamp every slot holding a member of U
        self.clock += 1
        for u in U:
            self.stamp[where[u]] = np.uint64(self.clock)
        # step 9: slot map
        slot_ids = np.vectorize(lambda f: where[int(f)], otypes=[np.int64])(flat).astype(np.int32)
        return EnsureResult(status=OK, slot_ids=slot_ids, misses=installs,
                            hits=len(U) - len(missing), evictions=evictions)

    def ensure_hybrid(self, layer: int, ids, max_fetch: int = -1, fetch_fraction=None) -> EnsureResult:
        """ensure_experts_hybrid (FreeToken MoE benchmark guide §5.4): only the first
        cap missing ids (ascending) get slots and copies; the others keep no slot,
        their requests map to -1 and they go to the CPU executor.  Readings: the
        cap is hybrid_cap(); it is further bounded by the evictable slots, so a
        hybrid step never fails for capacity; ids left to the CPU are not stamped
        (they own no slot); the clock advances as in ensure()."""
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim == 1:
            ids = ids[None, :]
        if not (0 <= layer < self.L) or ids.size and (ids.min() < 0 or ids.max() >= self.E):
            return EnsureResult(status=ERR_ARG)
        flat = layer * self.E + ids
        U = sorted(set(int(f) for f in flat.ravel()))
        in_U = set(U)
        where = {int(o): s for s, o in enumerate(self.owner) if o >= 0}
        missing = [u for u in U if u not in where]
        evictable = [s for s in range(self.S) if int(self.owner[s]) not in in_U]
        evictable.sort(key=lambda s: (int(self.owner[s]) != -1, int(self.stamp[s]),
                                      int(self.owner[s]), s))
        take = min(hybrid_cap(len(missing), max_fetch, fetch_fraction), len(missing), len(evictable))
        fetched, overflow = missing[:take], missing[take:]
        installs, evictions = [], 0
        for i, u in enumerate(fetched):
            s = evictable[i]
            if self.owner[s] != -1:
                evictions += 1
            self.owner[s] = u
            where[u] = s
            installs.append((s, u))
        self.clock += 1
        for u in U:
            if u in where:
                self.stamp[where[u]] = np.uint64(self.clock)
        slot_ids = np.vectorize(lambda f: where.get(int(f), -1), otypes=[np.int64])(flat).astype(np.int32)
        return EnsureResult(status=OK, slot_ids=slot_ids, misses=installs, hits=len(U) - len(missing),
                            evictions=evictions, num_indices=take, num_missing_full=len(missing),
                            overflow=overflow)
