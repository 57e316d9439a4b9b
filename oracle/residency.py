"""ORACLE (test infrastructure only) — global LRU expert cache and miss split.

Passages followed (zhichai.net article, section 2):
* Decode paragraph: most routed experts hit a device-resident LRU expert
  cache; the m misses of a step are split by the two measured bandwidths,
  q* = m * B_P / B_H of them filled over PCIe into the cache and the rest run
  in place on the host cores. B_P is the measured host-to-device transfer
  bandwidth, B_H the measured host memory bandwidth. Sending every miss to the
  host would forgo future cache hits, so the cache does keep filling.
* LRU paragraph: one global LRU over all layers' experts exploits the temporal
  locality of routing.

Readings of what the pages leave open (integer arithmetic throughout, so the
device implementation can match it bit for bit):
1. key = layer * E + expert; one clock tick per lookup call; hits take
   stamp = clock.
2. q* is rounded with an integer credit c (starts at 0):
       q = min(m, floor((c + m*B_P) / B_H)),  c <- min(c + m*B_P - q*B_H, B_H - 1)
   so the long-run filled share is exactly B_P / B_H (B_P, B_H in integer MB/s).
   q is clamped to m when B_P > B_H.
3. Capacity clamp: q_fill = min(q, C - h); the overflow runs on the host.
4. Misses are ranked by (token count descending, expert id ascending); the
   first q_fill are filled, the rest run on the host and are NOT inserted.
5. Victims: evict max(0, q_fill - f) occupied slots (f = empty slots) that were
   not touched in this call, in (stamp ascending, key ascending) order. The
   empty and freed slots, in ascending slot index, go to the fills in rank
   order; each takes the new key and stamp = clock.
6. The cache starts empty; prefill streaming does not touch it.

Elastic resize (zhichai.net article, section 2, the elastic VRAM paragraph:
the expert cache is a run-time quantity, rebuilt at scheduler safe points
without restarting the engine or reloading weights). Reading, between two
lookup calls, to a new capacity C':
7. If more than C' experts are resident, the least recently used are evicted
   in (stamp ascending, key ascending) order until C' remain.
8. A survivor in a slot below C' stays there; the survivors in slots >= C',
   in ascending order of their old slot, move to the empty slots below C' in
   ascending order (a device-to-device copy, not a reload from the pool).
9. Stamps, clock and credit are unchanged; slots C..C'-1 of a grown cache are
   empty.

Static placements, for the placement-policy comparison (zhichai.net article,
section 2, LRU paragraph: the same routing trace replayed under the global LRU,
under a placement fixed from prefill routing, and under a routing-blind static
split). Reading: a static placement puts the given keys in slots 0..n-1 (stamp
0, the rest empty) and freezes the cache: lookups still count hits, stamp them
and run the credit split, but nothing is filled or evicted (q_fill = 0), so
every miss runs on the host. Clearing it returns to the LRU from that state.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class Plan:
    layer: int
    clock: int
    m: int
    q: int
    q_fill: int
    credit: int                      # credit after this call
    hits: list = field(default_factory=list)     # [(expert, slot)], expert ascending
    fills: list = field(default_factory=list)    # [(expert, slot)], rank order
    host: list = field(default_factory=list)     # [expert], rank order
    evicted: list = field(default_factory=list)  # [key], eviction order
    counts: dict = field(default_factory=dict)   # expert -> tokens routed to it


class Residency:
    def __init__(self, capacity: int, layers: int, experts: int, bp_mbps: int, bh_mbps: int):
        if capacity < 0 or bp_mbps <= 0 or bh_mbps <= 0:
            raise ValueError("capacity >= 0 and positive bandwidths required")
        self.C, self.L, self.E = capacity, layers, experts
        self.bp, self.bh = int(bp_mbps), int(bh_mbps)
        self.slot_key = [-1] * capacity
        self.slot_stamp = [0] * capacity
        self.clock = 0
        self.credit = 0
        self.frozen = False

    def set_bandwidth(self, bp_mbps: int, bh_mbps: int) -> None:
        self.bp, self.bh = int(bp_mbps), int(bh_mbps)
        self.credit = min(self.credit, self.bh - 1)

    def resident(self) -> dict:
        return {k: s for s, k in enumerate(self.slot_key) if k >= 0}

    def lookup_plan(self, layer: int, ids) -> Plan:
        self.clock += 1
        counts: dict = {}
        for row in ids:
            for e in row:
                counts[int(e)] = counts.get(int(e), 0) + 1
        where = self.resident()
        hits, misses = [], []
        for e in sorted(counts):
            key = layer * self.E + e
            if key in where:
                s = where[key]
                self.slot_stamp[s] = self.clock
                hits.append((e, s))
            else:
                misses.append(e)
        h, m = len(hits), len(misses)

        q = min(m, (self.credit + m * self.bp) // self.bh)
        self.credit = min(self.credit + m * self.bp - q * self.bh, self.bh - 1)
        q_fill = 0 if self.frozen else min(q, self.C - h)

        ranked = sorted(misses, key=lambda e: (-counts[e], e))
        fill_experts, host = ranked[:q_fill], ranked[q_fill:]

        empty = [s for s in range(self.C) if self.slot_key[s] < 0]
        need = max(0, q_fill - len(empty))
        candidates = sorted((s for s in range(self.C)
                             if self.slot_key[s] >= 0 and self.slot_stamp[s] < self.clock),
                            key=lambda s: (self.slot_stamp[s], self.slot_key[s]))
        freed = candidates[:need]
        evicted = [self.slot_key[s] for s in freed]
        for s in freed:
            self.slot_key[s] = -1
        pool = sorted(empty + freed)[:q_fill]
        fills = []
        for e, s in zip(fill_experts, pool):
            self.slot_key[s] = layer * self.E + e
            self.slot_stamp[s] = self.clock
            fills.append((e, s))
        return Plan(layer=layer, clock=self.clock, m=m, q=q, q_fill=q_fill, credit=self.credit,
                    hits=hits, fills=fills, host=host, evicted=evicted, counts=counts)

    def snapshot(self):
        return list(self.slot_key), list(self.slot_stamp), self.clock, self.credit

    def resize(self, capacity: int):
        """Resize to `capacity` slots; returns (evicted keys in eviction order,
        moves [(old slot, new slot)] in order)."""
        if capacity < 0:
            raise ValueError("capacity >= 0")
        occupied = [s for s in range(self.C) if self.slot_key[s] >= 0]
        excess = max(0, len(occupied) - capacity)
        victims = sorted(occupied, key=lambda s: (self.slot_stamp[s], self.slot_key[s]))[:excess]
        evicted = [self.slot_key[s] for s in victims]
        for s in victims:
            self.slot_key[s] = -1
        keep = {s: (self.slot_key[s], self.slot_stamp[s]) for s in range(self.C)
                if self.slot_key[s] >= 0}
        key = [-1] * capacity
        stamp = [0] * capacity
        for s, (k, t) in keep.items():
            if s < capacity:
                key[s], stamp[s] = k, t
        movers = sorted(s for s in keep if s >= capacity)
        holes = [s for s in range(capacity) if key[s] < 0]
        moves = []
        for s, d in zip(movers, holes):
            key[d], stamp[d] = keep[s]
            moves.append((s, d))
        self.C, self.slot_key, self.slot_stamp = capacity, key, stamp
        return evicted, moves

    def set_static(self, keys) -> None:
        """Static placement: keys in slots 0..n-1 (stamp 0), cache frozen."""
        keys = [int(k) for k in keys]
        if len(keys) > self.C or len(set(keys)) != len(keys) or \
                any(k < 0 or k >= self.L * self.E for k in keys):
            raise ValueError("at most C distinct keys in range")
        self.slot_key = keys + [-1] * (self.C - len(keys))
        self.slot_stamp = [0] * self.C
        self.frozen = True

    def clear_static(self) -> None:
        self.frozen = False
