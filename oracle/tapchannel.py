"""Plain model of the tap mailbox (test infrastructure only).

What the pages state (rcap.io explainer, the TapChannel paragraph and its
per-microbatch pseudo-code; evolve.pub review, "Frequently asked questions"):
every source pipeline stage has a mailbox slot, allocated in advance in the
draft stage's memory; after its forward pass of a microbatch the source writes
its taps into that slot under a sequence stamp, and the draft stage, before its
own forward, waits for and reads the tap of that stamp. Data flows one way.

Where the pages stop (no slot layout, no rule for an early, late or repeated
stamp), this model takes the plainest reading that keeps "the stamp orders the
writes and reads": a slot keeps the stamp of its last committed tap and the
last stamp its reader consumed; a write must carry a larger stamp than the slot
holds and may not replace a tap that has not been read; a read must ask for
exactly the stamp the slot holds, once. Every refusal leaves the slot as it was.

The model is a Python object holding bytes; nothing here is shared with the
library.
"""
from __future__ import annotations

OK, NOT_READY, SKIPPED, DUPLICATE, STALE, BUSY, TOO_BIG = range(7)
NAMES = {OK: "OK", NOT_READY: "NOT_READY", SKIPPED: "SKIPPED", DUPLICATE: "DUPLICATE", STALE: "STALE",
         BUSY: "BUSY", TOO_BIG: "TOO_BIG"}


class Slot:
    """One mailbox slot of a fixed payload capacity."""

    def __init__(self, capacity: int):
        self.capacity = int(capacity)
        self.stamp = 0          # stamp of the tap in the slot (0: nothing written yet)
        self.consumed = 0       # last stamp the reader took
        self.payload = b""

    def write(self, data: bytes, stamp: int) -> int:
        """The source's side: put ``data`` in the slot under ``stamp``."""
        if stamp <= self.stamp:
            return STALE                 # stamps only move forward
        if self.consumed < self.stamp:
            return BUSY                  # the tap now in the slot has not been read
        if len(data) > self.capacity:
            return TOO_BIG
        self.payload = bytes(data)
        self.stamp = stamp
        return OK

    def read(self, expected: int, room: int):
        """The draft's side: take the tap stamped ``expected`` (at most ``room``
        bytes). Returns (status, bytes or None)."""
        if self.stamp < expected:
            return NOT_READY, None       # that microbatch's tap has not landed
        if self.stamp > expected:
            return SKIPPED, None         # a later tap replaced it: it was never written
        if self.consumed >= expected:
            return DUPLICATE, None       # already taken
        if len(self.payload) > room:
            return TOO_BIG, None
        self.consumed = expected
        return OK, self.payload


class Mailbox:
    """The draft stage's slots, one per source stage."""

    def __init__(self, capacities):
        self.slots = [Slot(c) for c in capacities]

    def write(self, src: int, data: bytes, stamp: int) -> int:
        return self.slots[src].write(data, stamp)

    def read(self, src: int, expected: int, room: int):
        return self.slots[src].read(expected, room)
