"""Pins for the INT4 / INT8 region split and the side-cache ring (exhaustive on small cases)."""

import json
import os

from oracle.regions import int4_region, int8_region, int8_written, ring_entry

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    for s in range(0, 6):
        for w in range(0, 9):
            for L in range(0, 30):
                yield L, s, w


def test_regions_partition_the_context():
    for L, s, w in _cases():
        r8 = int8_region(L, s, w)
        r4 = list(int4_region(L, s, w))
        assert len(set(r8)) == len(r8)
        assert set(r8).isdisjoint(r4)
        assert sorted(r8 + r4) == list(range(L))
        assert len(r8) == min(L, s + w)


def test_ring_entries_of_region_are_distinct_and_dense():
    for L, s, w in _cases():
        r8 = int8_region(L, s, w)
        ents = [ring_entry(p, s, w) for p in r8]
        assert sorted(ents) == list(range(min(L, s + w)))


def _simulate(s, w, appends):
    """Apply appends [(positions, L_after)] to a ring, returning entry -> last position."""
    ring = {}
    for positions, L_after in appends:
        written = {}
        for p in positions:
            if int8_written(p, L_after, s, w):
                e = ring_entry(p, s, w)
                assert e not in written, "two positions of one append share a ring entry"
                written[e] = p
        ring.update(written)
    return ring


def test_sequential_and_bulk_appends_leave_the_region_in_the_ring():
    for L, s, w in _cases():
        if L == 0:
            continue
        want = {ring_entry(p, s, w): p for p in int8_region(L, s, w)}
        seq = _simulate(s, w, [([p], p + 1) for p in range(L)])
        bulk = _simulate(s, w, [(list(range(L)), L)])
        assert {e: seq[e] for e in want} == want
        assert bulk == want
        # a prefill followed by one decode append (the decode step of a workload)
        two = _simulate(s, w, [(list(range(L - 1)), L - 1), ([L - 1], L)])
        assert {e: two[e] for e in want} == want


def test_page_default_budget():
    g = json.load(open(os.path.join(GOLDEN, "protection_defaults.json")))
    L = 10_000
    assert len(int8_region(L, g["sink"], g["recent"])) == g["budget"]
