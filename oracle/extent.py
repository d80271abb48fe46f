"""Extent bookkeeping oracle for the fresh combine output. Test infrastructure only.

OpenPipe/ART PR 971 ("Price HybridEP recompute outputs at the live communication extent",
description and reviews): while an earlier, larger graph is live its communication extent is
kept as a high-water mark; a later call's combine allocates a fresh [P, H] output at that live
extent, rounded up to four rows, and crops it to its own logical rows; the output's bytes enter
the workspace estimate as a maximum with the other stages, not a sum; once the earlier graph is
released, the call's own extent applies again.
"""
from __future__ import annotations

from .routing import round4


class ExtentTracker:
    """Live extents by handle; current(required) = round4(max(required, largest live extent))."""

    def __init__(self):
        self._live = {}
        self._next = 1

    def acquire(self, rows: int) -> int:
        if rows < 0:
            raise ValueError("rows must be non-negative")
        h = self._next
        self._next += 1
        self._live[h] = int(rows)
        return h

    def release(self, handle: int) -> None:
        if handle not in self._live:
            raise KeyError(handle)
        del self._live[handle]

    def high_water(self) -> int:
        return max(self._live.values(), default=0)

    def current(self, required_rows: int) -> int:
        return round4(max(int(required_rows), self.high_water()))


def output_bytes(P_out: int, H: int, elem_size: int) -> int:
    """Backing bytes of the fresh [P_out, H] combine output."""
    return int(P_out) * int(H) * int(elem_size)


def workspace_floor(existing_bytes: int, P_out: int, H: int, elem_size: int) -> int:
    """Workspace floor: the larger of the other stages' workspace and the combine output."""
    return max(int(existing_bytes), output_bytes(P_out, H, elem_size))
