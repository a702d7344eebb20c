"""The tap mailbox on the CPU: the plain model in oracle/tapchannel.py pinned by
properties the pages fix (taps of one source arrive one way, in stamp order,
each exactly once, never mixed up) and by hand-worked scripts; then the
library's own decision functions against the model over every small state."""
import itertools
import random

import pytest

from oracle import tapchannel as T

sda = pytest.importorskip("speculative_draft_branch_amd")
from speculative_draft_branch_amd import tapchannel as tc  # noqa: E402


def _payload(stamp, n=5):
    return bytes((stamp * 31 + i) % 256 for i in range(n))


def _run_schedule(order, n):
    """A writer sending stamps 1..n (retrying while BUSY) and a reader taking
    1..n (retrying while NOT_READY), interleaved by ``order`` (a sequence of
    'w'/'r' turns). Returns what the reader received and every status seen."""
    slot = T.Slot(64)
    w_next, r_next, got, seen = 1, 1, [], []
    for who in order:
        if who == "w" and w_next <= n:
            st = slot.write(_payload(w_next), w_next)
            seen.append(("w", st))
            if st == T.OK:
                w_next += 1
        elif who == "r" and r_next <= n:
            st, data = slot.read(r_next, 64)
            seen.append(("r", st))
            if st == T.OK:
                got.append((r_next, data))
                r_next += 1
    return got, seen


def test_every_interleaving_delivers_each_tap_once_in_order():
    """All interleavings of 2n writer and 2n reader turns (n = 3): whatever the
    timing, the reader gets exactly the taps that were written, each once, in
    stamp order, with their own bytes; the only refusals are the two waits."""
    n = 3
    turns = 2 * n
    count = 0
    for pos in itertools.combinations(range(2 * turns), turns):
        order = ["r"] * (2 * turns)
        for p in pos:
            order[p] = "w"
        got, seen = _run_schedule(order, n)
        count += 1
        assert [s for s, _ in got] == list(range(1, len(got) + 1))
        assert all(d == _payload(s) for s, d in got)
        assert {st for _, st in seen} <= {T.OK, T.BUSY, T.NOT_READY}
        # the writer only ever waits (BUSY) and the reader only ever waits (NOT_READY)
        assert not any(who == "w" and st == T.NOT_READY for who, st in seen)
        assert not any(who == "r" and st == T.BUSY for who, st in seen)
    assert count == 924  # C(12, 6)


def test_long_random_schedules_deliver_everything():
    rng = random.Random(7)
    for _ in range(200):
        n = rng.randint(1, 12)
        order = [rng.choice("wr") for _ in range(20 * n)] + ["w", "r"] * (2 * n)
        got, _ = _run_schedule(order, n)
        assert [s for s, _ in got] == list(range(1, n + 1))


def test_hand_worked_script():
    """Statuses worked out by hand from the protocol rules, step by step."""
    s = T.Slot(8)
    script = [
        ("r", 1, T.NOT_READY),   # nothing written yet
        ("w", 1, T.OK),
        ("w", 2, T.BUSY),        # tap 1 not read yet
        ("r", 2, T.NOT_READY),   # the slot holds 1 < 2
        ("r", 1, T.OK),
        ("r", 1, T.DUPLICATE),   # taken already
        ("w", 1, T.STALE),       # stamps only move forward
        ("w", 3, T.OK),          # stamp 2 skipped by the writer
        ("r", 2, T.SKIPPED),     # the slot holds 3 > 2
        ("r", 3, T.OK),
        ("w", 4, T.OK),
        ("w", 9, T.BUSY),
    ]
    for who, stamp, want in script:
        if who == "w":
            assert s.write(_payload(stamp), stamp) == want, (who, stamp)
        else:
            st, data = s.read(stamp, 8)
            assert st == want, (who, stamp)
            assert (data == _payload(stamp)) if st == T.OK else data is None
    # too big in both directions, each leaving the slot unchanged
    s2 = T.Slot(4)
    assert s2.write(b"12345", 1) == T.TOO_BIG and (s2.stamp, s2.payload) == (0, b"")
    assert s2.write(b"1234", 1) == T.OK
    assert s2.read(1, 3) == (T.TOO_BIG, None) and s2.consumed == 0
    assert s2.read(1, 4) == (T.OK, b"1234")


def test_refusals_leave_the_slot_unchanged():
    rng = random.Random(3)
    for _ in range(500):
        s = T.Slot(6)
        s.stamp = rng.randint(0, 4)
        s.consumed = rng.randint(0, s.stamp)
        s.payload = bytes(rng.randint(0, 6))
        before = (s.stamp, s.consumed, s.payload)
        st = s.write(bytes(rng.randint(0, 8)), rng.randint(0, 6))
        if st != T.OK:
            assert (s.stamp, s.consumed, s.payload) == before
        before = (s.stamp, s.consumed, s.payload)
        st, _ = s.read(rng.randint(0, 6), rng.randint(0, 8))
        if st != T.OK:
            assert (s.stamp, s.consumed, s.payload) == before


def test_library_decisions_match_the_model_on_every_small_state():
    cap = 16
    for slot_stamp in range(5):
        for consumed in range(slot_stamp + 1):
            for stamp in range(7):
                for nbytes in (0, cap, cap + 1):
                    m = T.Slot(cap)
                    m.stamp, m.consumed = slot_stamp, consumed
                    want = m.write(bytes(nbytes), stamp)
                    assert tc.write_decision(slot_stamp, consumed, stamp, nbytes, cap) == want, \
                        (slot_stamp, consumed, stamp, nbytes)
                for room in (0, 8, cap):
                    m = T.Slot(cap)
                    m.stamp, m.consumed, m.payload = slot_stamp, consumed, bytes(8)
                    want, _ = m.read(stamp, room)
                    assert tc.read_decision(slot_stamp, consumed, stamp, 8, room) == want, \
                        (slot_stamp, consumed, stamp, room)


def test_status_codes_agree():
    assert (tc.TAP_OK, tc.TAP_NOT_READY, tc.TAP_SKIPPED, tc.TAP_DUPLICATE, tc.TAP_STALE, tc.TAP_BUSY,
            tc.TAP_TOO_BIG) == (T.OK, T.NOT_READY, T.SKIPPED, T.DUPLICATE, T.STALE, T.BUSY, T.TOO_BIG)


def test_slot_bytes():
    assert tc.slot_bytes(0) == 256
    assert tc.slot_bytes(1) == 512
    assert tc.slot_bytes(256) == 512
    assert tc.slot_bytes(1 << 20) == 256 + (1 << 20)
