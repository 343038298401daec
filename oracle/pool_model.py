"""Plain model of the host page pool -- TEST INFRASTRUCTURE ONLY (tests/ may use it;
nothing on the product path imports it).  It shares no code with the library.

[P2] TensorFold PR #1170, commit 1ac2075: single pages leave a free stack from the
low end of the arena; findRun / claimRun / releaseRun take runs of k adjacent free
pages from the high end; a request that finds no such run, the pool being too
fragmented, waits.

Readings where the pages are silent:
  * the free stack is last-in first-out, and a fresh pool hands out page 0, then
    1, 2, ... (the bottom of the arena first);
  * a run is the highest k consecutive free pages; its pages leave the free stack
    (the others keep their order) and come back onto it with the run's lowest page
    on top; only a run exactly as it was claimed can be released (not part of one,
    not two together, not twice);
  * freed pages go back onto the stack in list order, the last listed on top;
  * a request that cannot be met takes nothing ("waits"); freeing a page that was
    not handed out, or listing one twice, is refused and changes nothing.

Parity: pinned by hand-worked sequences in tests/test_pool.py.
"""
from __future__ import annotations

from typing import List, Optional

FREE, PAGE, RUN = 0, 1, 2


class PagePool:
    def __init__(self, n_pages: int):
        assert n_pages >= 1
        self.n = n_pages
        self.stack: List[int] = list(range(n_pages - 1, -1, -1))  # top = last element = page 0
        self.kind = [FREE] * n_pages
        self.runs = {}  # lowest page of each claimed run -> its length

    def free_count(self) -> int:
        return len(self.stack)

    def alloc(self, n: int) -> Optional[List[int]]:
        """n pages off the top of the stack, or None (nothing taken) when fewer are free."""
        if n > len(self.stack):
            return None
        out = []
        for _ in range(n):
            p = self.stack.pop()
            self.kind[p] = PAGE
            out.append(p)
        return out

    def free(self, pages: List[int]) -> bool:
        if len(set(pages)) != len(pages) or any(not (0 <= p < self.n) or self.kind[p] != PAGE for p in pages):
            return False
        for p in pages:
            self.kind[p] = FREE
            self.stack.append(p)
        return True

    def claim_run(self, k: int) -> Optional[int]:
        """Lowest page of the highest k consecutive free pages, or None when there is none."""
        for first in range(self.n - k, -1, -1):
            if all(self.kind[p] == FREE for p in range(first, first + k)):
                for p in range(first, first + k):
                    self.kind[p] = RUN
                self.runs[first] = k
                self.stack = [p for p in self.stack if self.kind[p] == FREE]
                return first
        return None

    def release_run(self, first: int, k: int) -> bool:
        if self.runs.get(first) != k:
            return False
        del self.runs[first]
        for p in range(first + k - 1, first - 1, -1):
            self.kind[p] = FREE
            self.stack.append(p)
        return True
