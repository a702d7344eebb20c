"""ctypes binding of the tap mailbox (include/tapchannel.h): argument checks and
pointer marshalling only; the protocol runs in the library's kernels."""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from ._abi import check, lib

TAP_OK, TAP_NOT_READY, TAP_SKIPPED, TAP_DUPLICATE, TAP_STALE, TAP_BUSY, TAP_TOO_BIG = range(7)

_vp, _sz, _u64, _st = C.c_void_p, C.c_size_t, C.c_uint64, C.c_int
lib.ba_tap_slot_bytes.argtypes = [_sz]
lib.ba_tap_slot_bytes.restype = _sz
lib.ba_tap_slot_init.argtypes = [_vp, _sz, _vp]
lib.ba_tap_slot_init.restype = _st
lib.ba_tap_write.argtypes = [_vp, _sz, _vp, _sz, _u64, _vp, _vp, _vp]
lib.ba_tap_write.restype = _st
lib.ba_tap_read.argtypes = [_vp, _sz, _vp, _sz, _u64, _vp, _vp, _vp]
lib.ba_tap_read.restype = _st
lib.ba_tap_wait_and_read.argtypes = [_vp, _sz, _vp, _sz, _u64, _vp, _vp, _vp, _vp]
lib.ba_tap_wait_and_read.restype = _st
lib.ba_tap_write_decision.argtypes = [_u64, _u64, _u64, _sz, _sz]
lib.ba_tap_write_decision.restype = C.c_int32
lib.ba_tap_read_decision.argtypes = [_u64, _u64, _u64, _u64, _sz]
lib.ba_tap_read_decision.restype = C.c_int32

SYMBOLS = ["ba_tap_slot_bytes", "ba_tap_slot_init", "ba_tap_write", "ba_tap_read", "ba_tap_wait_and_read",
           "ba_tap_write_decision", "ba_tap_read_decision"]


def slot_bytes(capacity: int) -> int:
    return int(lib.ba_tap_slot_bytes(int(capacity)))


def write_decision(slot_stamp: int, consumed: int, stamp: int, nbytes: int, capacity: int) -> int:
    return int(lib.ba_tap_write_decision(slot_stamp, consumed, stamp, nbytes, capacity))


def read_decision(slot_stamp: int, consumed: int, expected: int, nbytes: int, dst_bytes: int) -> int:
    return int(lib.ba_tap_read_decision(slot_stamp, consumed, expected, nbytes, dst_bytes))


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _event_handle(ev: Optional[torch.cuda.Event]):
    if ev is None:
        return None
    if not ev.cuda_event:  # torch creates the event on its first record
        ev.record()
    return ev.cuda_event


class Slot:
    """A mailbox slot in device memory (a torch byte tensor owns it)."""

    def __init__(self, capacity: int, device="cuda"):
        self.capacity = int(capacity)
        self.mem = torch.empty(slot_bytes(self.capacity), dtype=torch.uint8, device=device)
        check(lib.ba_tap_slot_init(self.mem.data_ptr(), self.capacity, _stream()), "ba_tap_slot_init")

    def write(self, src: torch.Tensor, stamp: int, status: torch.Tensor, done_event=None):
        """Enqueue on the current stream; status: an int32 GPU tensor of one element."""
        _dev(src, "src")
        _dev(status, "status")
        check(lib.ba_tap_write(self.mem.data_ptr(), self.capacity, src.data_ptr() if src.numel() else None,
                               _nbytes(src), int(stamp), status.data_ptr(), _event_handle(done_event), _stream()),
              "ba_tap_write")

    def read(self, dst: torch.Tensor, expected: int, status: torch.Tensor, nbytes: Optional[torch.Tensor] = None,
             written_event=None):
        """Enqueue on the current stream (after waiting for written_event, if given)."""
        _dev(dst, "dst")
        _dev(status, "status")
        nb = None if nbytes is None else nbytes.data_ptr()
        args = (self.mem.data_ptr(), self.capacity, dst.data_ptr() if dst.numel() else None, _nbytes(dst),
                int(expected), status.data_ptr(), nb)
        if written_event is None:
            check(lib.ba_tap_read(*args, _stream()), "ba_tap_read")
        else:
            check(lib.ba_tap_wait_and_read(*args, _event_handle(written_event), _stream()), "ba_tap_wait_and_read")
