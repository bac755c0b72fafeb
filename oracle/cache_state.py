"""Integer state of a streaming head's constant-length cache (test oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, never by the library.

Streaming heads keep a constant-length cache of attention sinks and recent
tokens (DuoAttention abstract; sourcepulse card, "How It Works").  The pages
give no slot layout (pith.science referee report, minor comment 3), so the
layout read here is: ``sink`` sink slots, where slot s holds position s, then
``recent`` ring slots.  The ring is an ordinary ring buffer: free slots are
taken in order, and once all are used a new token replaces the oldest recent
token.

Two independent forms are given and pinned against each other in the tests:

* ``CacheSimulator`` -- token-at-a-time bookkeeping with an explicit
  oldest-first eviction list (the behaviour described above);
* ``streaming_slot_of_position`` -- the closed form of the same map,
  slot(p) = p for p < sink, else sink + (p - sink) mod recent.
"""

from __future__ import annotations

from collections import deque

import numpy as np


def streaming_slot_of_position(p: int, sink: int, recent: int) -> int:
    """Closed-form slot of position ``p`` in a sink+ring cache."""
    if p < 0:
        raise ValueError("position must be >= 0")
    if p < sink:
        return p
    return sink + (p - sink) % recent


def streaming_slot_positions(n_tokens: int, sink: int, recent: int) -> np.ndarray:
    """Position held by every slot after ``n_tokens`` appends (-1 = empty).

    Closed form: a slot holds the LARGEST position p < n_tokens that maps to
    it, because later tokens overwrite earlier ones.
    """
    slots = np.full(sink + recent, -1, dtype=np.int64)
    for p in range(n_tokens):
        slots[streaming_slot_of_position(p, sink, recent)] = p
    return slots


class CacheSimulator:
    """Token-at-a-time model of one streaming head's sink + ring cache."""

    def __init__(self, sink: int, recent: int):
        if sink < 0 or recent < 1:
            raise ValueError("need sink >= 0 and recent >= 1")
        self.sink = sink
        self.recent = recent
        self.n = 0
        self.slots = [-1] * (sink + recent)
        self._free_ring = list(range(sink, sink + recent))  # taken in order
        self._ring_fifo = deque()  # (position, slot), oldest first

    def append(self) -> int:
        """Store the next position; return the slot it went to."""
        p = self.n
        if p < self.sink:
            slot = p
        elif self._free_ring:
            slot = self._free_ring.pop(0)
            self._ring_fifo.append((p, slot))
        else:
            _old, slot = self._ring_fifo.popleft()
            self._ring_fifo.append((p, slot))
        self.slots[slot] = p
        self.n += 1
        return slot

    def positions(self) -> np.ndarray:
        """Positions currently cached, in increasing order."""
        return np.array(sorted(p for p in self.slots if p >= 0), dtype=np.int64)

    def slot_positions(self) -> np.ndarray:
        return np.array(self.slots, dtype=np.int64)
