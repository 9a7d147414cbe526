"""Oracle: the host-side slot / page allocator as a plain state machine.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows the ``PageTable`` class on [continuous-batching compare]
scripts/benchmarks/flex_paged_attention.py:

* free pages start as ``reversed(range(1, n_pages))`` and are used as a stack;
  page 0 is never handed out (reserved);
* free slots start as ``reversed(range(1, max_batch))``; slot 0 is the reserved
  no-op slot, so the first ``allocate`` returns 1, then 2, ...;
* ``allocate`` pops a slot, zeroes its capacity and resets its device row to
  ``-1``;
* ``reserve(slot, seq_len)`` grows capacity (tokens, a multiple of the page
  size) to at least ``seq_len`` by taking the LAST ``k`` entries of the free
  stack, in stack order, as the next logical pages; ``dry_run`` only reports
  whether it would fit; without ``dry_run`` running out of pages is an error
  and nothing changes;
* ``can_reserve(size)`` for a new request: enough free pages for ``size``
  tokens and a free slot; for an existing slot: a dry-run ``reserve``;
* ``erase(slot)`` returns the slot and pushes its pages back in reverse order;
  the device row is left stale until the next ``allocate`` of that slot;
* the device table starts at ``-1`` everywhere except row 0, which is all 0.

The companion commit message of [moe-qwen3 compare] explains why callers size
the table at ``max_batch + 1`` slots: slot 0 is not usable.
"""

from __future__ import annotations

import numpy as np


def _cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


class PageTableModel:
    def __init__(self, n_pages: int, page_size: int, max_slots: int):
        self.n_pages = n_pages
        self.page_size = page_size
        self.max_slots = max_slots
        self.device_table = -np.ones((max_slots, n_pages), dtype=np.int64)
        self.device_table[0, :] = 0
        self.rows = [[] for _ in range(max_slots)]
        self.capacity = [0] * max_slots
        self.free_pages = list(reversed(range(1, n_pages)))
        self.free_slots = list(reversed(range(1, max_slots)))

    @property
    def pages_available(self) -> int:
        return len(self.free_pages)

    def can_reserve(self, size: int, slot: int | None = None) -> bool:
        if slot is None:
            return self.pages_available * self.page_size >= size and len(self.free_slots) > 0
        return self.reserve(slot, size, dry_run=True)

    def allocate(self) -> int:
        if not self.free_slots:
            raise RuntimeError("no free slot")
        s = self.free_slots.pop()
        self.capacity[s] = 0
        self.device_table[s, :] = -1
        return s

    def reserve(self, slot: int, seq_len: int, dry_run: bool = False) -> bool:
        if seq_len <= self.capacity[slot]:
            return True
        k = _cdiv(seq_len - self.capacity[slot], self.page_size)
        fits = k <= self.pages_available
        if dry_run:
            return fits
        if not fits:
            raise RuntimeError(
                f"cannot reserve {k} pages for length {seq_len} in slot {slot}: "
                f"{self.pages_available} free, capacity {self.capacity[slot]}")
        start = self.capacity[slot] // self.page_size
        granted = self.free_pages[-k:]
        self.device_table[slot, start:start + k] = granted
        self.rows[slot] += granted
        self.free_pages = self.free_pages[:-k]
        self.capacity[slot] += k * self.page_size
        return True

    def erase(self, slot: int) -> None:
        self.free_slots.append(slot)
        self.free_pages.extend(reversed(self.rows[slot]))
        self.rows[slot] = []

    def table(self, pages_per_slot: int) -> np.ndarray:
        """Device-format table ``[max_slots][pages_per_slot]`` (int32)."""
        return self.device_table[:, :pages_per_slot].astype(np.int32)
