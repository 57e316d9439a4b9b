"""Pins for the oracle's global LRU cache and q* miss split — CPU only."""
import json
import os

import numpy as np
import pytest

import synth
from oracle.residency import Residency


def test_hand_worked_lru_sequence():
    r = Residency(capacity=2, layers=1, experts=4, bp_mbps=1, bh_mbps=1)
    p = r.lookup_plan(0, [[0, 1]])
    assert p.fills == [(0, 0), (1, 1)] and p.host == [] and p.hits == []
    p = r.lookup_plan(0, [[2]])           # both stamps 1: key 0 is the lower key
    assert p.evicted == [0] and p.fills == [(2, 0)]
    p = r.lookup_plan(0, [[1, 3]])        # 1 hits (now stamp 3); 2 is the only victim
    assert p.hits == [(1, 1)] and p.evicted == [2] and p.fills == [(3, 0)]
    p = r.lookup_plan(0, [[0, 2]])        # both at stamp 3: evict key 1, then key 3
    assert p.evicted == [1, 3] and p.fills == [(0, 0), (2, 1)]
    p = r.lookup_plan(0, [[0, 1], [2, 3]])  # 2 hits fill the cache: overflow to host
    assert p.hits == [(0, 0), (2, 1)] and p.q == 2 and p.q_fill == 0 and p.host == [1, 3]
    assert r.snapshot() == ([0, 2], [5, 5], 5, 0)


def test_misses_ranked_by_token_count_then_id():
    r = Residency(capacity=8, layers=1, experts=4, bp_mbps=1, bh_mbps=2)
    p = r.lookup_plan(0, [[0, 1], [1, 2], [1, 0]])  # counts 0:2, 1:3, 2:1
    # m = 3, q = floor(3*1/2) = 1: the most-routed expert is filled
    assert p.q == 1 and [e for e, _ in p.fills] == [1] and p.host == [0, 2]
    assert p.counts == {0: 2, 1: 3, 2: 1} and p.credit == 1


def test_credit_hand_worked_quarter_split():
    # B_P / B_H = 1/4 with one miss per call: every fourth miss is filled
    r = Residency(capacity=100, layers=100, experts=1, bp_mbps=1, bh_mbps=4)
    qs = [r.lookup_plan(l, [[0]]).q for l in range(12)]
    assert qs == [0, 0, 0, 1] * 3


def _random_calls(seed, n, L, E, k, T=1):
    rng = np.random.default_rng(seed)
    calls = []
    for _ in range(n):
        l = int(rng.integers(0, L))
        ids = [list(rng.choice(E, size=k, replace=False)) for _ in range(T)]
        calls.append((l, ids))
    return calls


@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_random_calls(seed):
    rng = np.random.default_rng(100 + seed)
    L, E, k = 3, 12, int(rng.integers(1, 5))
    C = int(rng.integers(0, 3 * k + 2))
    bp, bh = int(rng.integers(1, 200)), int(rng.integers(1, 200))
    r = Residency(C, L, E, bp, bh)
    for l, ids in _random_calls(seed, 200, L, E, k, T=int(rng.integers(1, 4))):
        before = r.resident()
        stamps = list(r.slot_stamp)
        p = r.lookup_plan(l, ids)
        after = r.resident()
        keys = {l * E + int(e) for row in ids for e in row}
        assert len(p.hits) + p.m == len(keys)
        assert all(l * E + e in before for e, _ in p.hits)
        assert all(l * E + e not in before for e in p.host)
        assert all(after.get(l * E + e) == s for e, s in p.fills)
        assert all(l * E + e not in after for e in p.host)
        assert len(after) <= C and len(set(r.slot_key) - {-1}) == len(after)
        assert p.q_fill == min(p.q, C - len(p.hits)) and 0 <= p.credit < bh
        # victims were the least recently used among the slots not touched now
        untouched = [(stamps[s], key) for key, s in before.items()
                     if key not in keys]
        worst = sorted(untouched)[:len(p.evicted)]
        assert sorted(p.evicted) == sorted(kk for _, kk in worst)


def test_matches_ordered_list_lru_when_every_miss_fills():
    L, E, k, C = 4, 16, 4, 10
    r = Residency(C, L, E, 7, 7)
    last_use = {}
    for n, (l, ids) in enumerate(_random_calls(7, 400, L, E, k), start=1):
        r.lookup_plan(l, ids)
        for e in ids[0]:
            last_use[l * E + int(e)] = n
        top = sorted(last_use, key=lambda key: (last_use[key], key), reverse=True)[:C]
        assert set(r.resident()) == set(top)


def test_mattson_inclusion():
    L, E, k = 4, 16, 4
    calls = _random_calls(9, 300, L, E, k)
    misses, sets = [], []
    for C in range(k, 40):
        r = Residency(C, L, E, 5, 5)
        tot = 0
        for l, ids in calls:
            tot += r.lookup_plan(l, ids).m
        misses.append(tot)
        sets.append(set(r.resident()))
    assert all(a >= b for a, b in zip(misses, misses[1:]))
    assert all(a <= b for a, b in zip(sets, sets[1:]))


def test_full_capacity_gives_compulsory_misses_only():
    L, E, k = 3, 8, 3
    calls = _random_calls(11, 150, L, E, k)
    r = Residency(L * E, L, E, 3, 3)
    seen, tot = set(), 0
    for l, ids in calls:
        tot += r.lookup_plan(l, ids).m
        seen |= {l * E + int(e) for e in ids[0]}
    assert tot == len(seen)


@pytest.mark.parametrize("bp,bh", [(11800, 47500), (9, 10), (1, 3), (123, 124)])
def test_q_closed_form(bp, bh):
    rng = np.random.default_rng(bp)
    r = Residency(8, 500, 8, bp, bh)  # q does not depend on capacity
    ms, qs = [], []
    for n in range(500):
        m = int(rng.integers(0, 9))
        p = r.lookup_plan(n, [list(range(m))] if m else [[]])
        ms.append(m)
        qs.append(p.q)
        assert p.q in (m * bp // bh, -(-m * bp // bh))
    assert sum(qs) == (sum(ms) * bp) // bh


def test_equal_bandwidths_fill_every_miss():
    r = Residency(64, 1000, 8, 50, 50)
    for n in range(100):
        p = r.lookup_plan(n, [[0, 1, 2]])
        assert p.q == p.q_fill == 3 and p.host == []


def test_page_worked_splits(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q_split_pages.json")))
    lap = g["laptop_lpddr5"]
    bp, bh = int(lap["B_P_GBps"] * 1000), int(lap["B_H_GBps"] * 1000)
    trace = synth.sticky_zipf_trace(0, 200, 4, 32, 4)
    r = Residency(16, 4, 32, bp, bh)
    m = q = 0
    for s in range(trace.shape[0]):
        for l in range(4):
            p = r.lookup_plan(l, [trace[s, l]])
            m, q = m + p.m, q + p.q
    assert abs((m - q) / m - lap["host_share_about"]) < 0.02
    desk = g["desktop_ddr5"]
    r = Residency(16, 4, 32, 900, 1000)  # B_P slightly below B_H
    m = q = 0
    for s in range(trace.shape[0]):
        for l in range(4):
            p = r.lookup_plan(l, [trace[s, l]])
            m, q = m + p.m, q + p.q
    assert abs(q / m - desk["fill_share_about"]) < 0.02


def test_capacity_below_k_overflows_to_host():
    r = Residency(2, 1, 8, 1, 1)
    p = r.lookup_plan(0, [[0, 1, 2, 3]])
    assert p.q == 4 and p.q_fill == 2 and p.fills == [(0, 0), (1, 1)] and p.host == [2, 3]


def test_resize_hand_worked():
    # 1 layer, 8 experts, 4 slots, every miss filled
    r = Residency(4, 1, 8, 1, 1)
    for ids in ([[0]], [[1]], [[2]], [[3]], [[1]]):  # slots 0..3 <- 0,1,2,3; 1 touched again
        r.lookup_plan(0, ids)
    assert r.snapshot()[:2] == ([0, 1, 2, 3], [1, 5, 3, 4])
    # shrink to 2: LRU order is key 0 (stamp 1), key 2 (3), key 3 (4), key 1 (5) -> evict 0, 2;
    # survivors: key 1 in slot 1 stays, key 3 in slot 3 moves to the hole at slot 0
    evicted, moves = r.resize(2)
    assert evicted == [0, 2] and moves == [(3, 0)]
    assert r.snapshot() == ([3, 1], [4, 5], 5, 0)
    # grow to 5: everything stays, slots 2..4 empty; the next misses fill them in order
    assert r.resize(5) == ([], [])
    assert r.snapshot()[:2] == ([3, 1, -1, -1, -1], [4, 5, 0, 0, 0])
    p = r.lookup_plan(0, [[6, 7]])
    assert p.fills == [(6, 2), (7, 3)] and p.evicted == []


def test_resize_keeps_the_most_recent_keys():
    # brute force: after shrinking, the resident keys are the C' largest (stamp, key)
    rng = np.random.default_rng(11)
    r = Residency(24, 3, 16, 1, 1)
    for _ in range(80):
        l = int(rng.integers(0, 3))
        r.lookup_plan(l, [list(rng.choice(16, size=3, replace=False))])
    keys, stamps, clock, credit = r.snapshot()
    before = {k: t for k, t in zip(keys, stamps) if k >= 0}
    for cap in (20, 9, 1, 0):
        evicted, moves = r.resize(cap)
        keys, stamps, c2, cr2 = r.snapshot()
        assert (c2, cr2) == (clock, credit) and len(keys) == cap
        want = sorted(before, key=lambda k: (before[k], k))[-cap:] if cap else []
        assert sorted(k for k in keys if k >= 0) == sorted(want)
        assert all(before[k] == t for k, t in zip(keys, stamps) if k >= 0)
        assert sorted(evicted) == sorted(set(before) - set(want))
        before = {k: before[k] for k in want}
        # moved blocks only go down into holes, and each source is a distinct old slot
        assert all(d < cap <= s for s, d in moves)


def test_resize_then_lookups_match_a_cache_built_at_that_size():
    # shrinking to C' keeps the same recency order the smaller cache would have,
    # so with every miss filled the resident sets agree from then on (LRU is a
    # stack algorithm); slot positions may differ
    rng = np.random.default_rng(5)
    calls = [(int(rng.integers(0, 2)), [list(rng.choice(12, size=2, replace=False))])
             for _ in range(120)]
    a, b = Residency(16, 2, 12, 1, 1), Residency(6, 2, 12, 1, 1)
    for l, ids in calls[:60]:
        a.lookup_plan(l, ids)
        b.lookup_plan(l, ids)
    a.resize(6)
    assert set(a.resident()) == set(b.resident())
    for l, ids in calls[60:]:
        pa, pb = a.lookup_plan(l, ids), b.lookup_plan(l, ids)
        assert [e for e, _ in pa.hits] == [e for e, _ in pb.hits]
        assert set(a.resident()) == set(b.resident())


def test_static_placement_frozen_then_lru():
    r = Residency(3, 2, 4, 5, 5)  # B_P = B_H: the LRU would fill every miss
    r.set_static([5, 0, 7])       # layer 1 expert 1, layer 0 expert 0, layer 1 expert 3
    p = r.lookup_plan(0, [[0, 2]])
    assert p.hits == [(0, 1)] and p.q == 1 and p.q_fill == 0 and p.fills == [] and p.host == [2]
    p = r.lookup_plan(1, [[1, 2], [3, 2]])
    assert p.hits == [(1, 0), (3, 2)] and p.host == [2] and p.evicted == []
    assert r.snapshot() == ([5, 0, 7], [2, 1, 2], 2, 0)
    r.clear_static()              # LRU again from this state: key 0 (stamp 1) goes first
    p = r.lookup_plan(0, [[3]])
    assert p.fills == [(3, 1)] and p.evicted == [0]
    with pytest.raises(ValueError):
        r.set_static([1, 1])


def test_static_placement_miss_rate_is_membership():
    # frozen: a key hits iff it is in the placement, whatever the order of calls
    rng = np.random.default_rng(2)
    keys = list(rng.choice(48, size=10, replace=False))
    r = Residency(12, 3, 16, 1, 3)
    r.set_static(keys)
    for _ in range(50):
        l = int(rng.integers(0, 3))
        ids = [list(rng.choice(16, size=4, replace=False))]
        p = r.lookup_plan(l, ids)
        assert sorted(e for e, _ in p.hits) == sorted(e for e in ids[0] if l * 16 + e in keys)
        assert p.q_fill == 0 and not p.fills and not p.evicted
    assert sorted(k for k in r.snapshot()[0] if k >= 0) == sorted(int(k) for k in keys)


def test_set_bandwidth_clamps_the_credit_hand_worked():
    """Re-setting B_P / B_H between calls keeps the cache and clock and clips
    the credit below the new B_H (the split remainder can never reach B_H)."""
    r = Residency(capacity=100, layers=100, experts=1, bp_mbps=9, bh_mbps=10)
    p = r.lookup_plan(0, [[0]])        # q = floor((0 + 9) / 10) = 0, credit 9
    assert (p.q, p.credit) == (0, 9) and p.host == [0]
    r.set_bandwidth(1, 4)              # credit min(9, 4 - 1) = 3
    assert r.credit == 3 and r.clock == 1
    p = r.lookup_plan(1, [[0]])        # q = floor((3 + 1) / 4) = 1, credit 3 + 1 - 4 = 0
    assert (p.q, p.q_fill, p.credit) == (1, 1, 0)
    p = r.lookup_plan(2, [[0]])        # q = floor((0 + 1) / 4) = 0, credit 1
    assert (p.q, p.credit) == (0, 1)
    # without the clip the credit would have stayed 9: q = 1 with credit 3 at
    # the second call and q = 1 again at the third
    r.set_bandwidth(1, 1000)           # a larger B_H leaves the credit as it is
    assert r.credit == 1
    assert r.snapshot()[2] == 3        # clock unchanged by the re-split
    assert r.resident() == {1 * 1 + 0: 0}  # the one filled key (layer 1) kept in slot 0
