"""INT4 / INT8 regions and the INT8 side-cache ring.

KV4-RL ("Key Contributions" item 4, "Methodology in Plain English"): the first
s positions (attention sinks) and the most recent w positions are kept in an
INT8 side cache, the rest of the context in INT4; the two sets are attended as
disjoint regions, so the INT8 work is bounded by s + w per sequence.

Readings where the pages are silent:

* every position is also written to the INT4 cache (the INT8 store is a *side*
  cache), so a position leaving the recent window needs no re-quantization;
* the side cache is a fixed ring of s + w entries (the RLKV page, section 4.3,
  stores its sink-plus-local tokens in a fixed-size circular buffer): position
  p < s goes to entry p, any other position to entry s + ((p - s) mod w);
* an append writes the INT8 copy only when the position is a sink or lies in
  the final recent window of the sequence after that append, which keeps bulk
  appends free of two writes to one ring entry;
* when L <= s + w the two sets overlap and their union is used; the INT4
  region is then empty.
"""

from __future__ import annotations


def int8_region(L: int, s: int, w: int) -> list[int]:
    """Positions attended from INT8: [0, min(s, L)) U [max(s, L - w), L)."""
    sinks = list(range(0, min(s, L)))
    recent = list(range(max(s, L - w), L))
    return sinks + recent


def int4_region(L: int, s: int, w: int) -> range:
    """Positions attended from INT4: [s, L - w) when non-empty."""
    lo, hi = s, L - w
    return range(lo, hi) if hi > lo else range(0)


def ring_entry(p: int, s: int, w: int) -> int:
    """Side-cache entry of position p (valid for positions that are stored in INT8)."""
    if p < s:
        return p
    return s + (p - s) % w


def int8_written(p: int, L_after: int, s: int, w: int) -> bool:
    """Whether an append of position p (sequence length L_after afterwards) writes INT8."""
    return p < s or p >= L_after - w
