"""Python model of the paged KV-cache page allocator.

TEST INFRASTRUCTURE (see the package docstring).

Follows the allocator of "TensorRT-LLM 深度实战", section 3.1: a pool of
``num_pages`` pages of ``page_size`` tokens, a free-page list initialised to
``range(num_pages)`` that hands out pages from its END and takes released
pages back at its end, and a page table mapping each sequence to its list of
page ids.  ``allocate`` takes ``ceil(num_tokens / page_size)`` pages;
``append_tokens`` adds ``ceil((usage + new - capacity) / page_size)`` pages
when the new tokens overflow the current pages; ``release`` returns every page.

Readings where the section's sketch is incomplete:

* allocation is all-or-nothing: an allocation or append that cannot get all
  of its pages raises ``OutOfPages`` and changes nothing (the sketch would
  leave already-popped pages orphaned, and its append never checks);
* a sequence's token count is tracked (the sketch calls an undefined helper)
  and starts at ``num_tokens``;
* allocating an existing id raises ``SequenceExists`` (the sketch would
  overwrite and leak its pages); unknown ids raise ``UnknownSequence``;
* a token's slot id is ``page * page_size + offset``.

Block reuse (the KV-cache reuse / prefix caching the TensorRT-LLM pages
enable for shared prefixes): ``fork`` gives a new sequence the pages of an
existing one, each page counting its owners.  Readings:

* a released page returns to the free list only when its last owner
  releases it;
* appending to a sequence whose last page is partly filled and shared
  copies that page first (copy-on-write): a fresh page, taken from the free
  list before any overflow pages, replaces it in the appending sequence, and
  the (old, new) pair is reported so that the caller copies the page's
  contents on the device before writing the new tokens; a full shared last
  page needs no copy (new tokens go to new pages);
* the plain ``append_tokens`` refuses an append that needs a copy
  (``SharedLastPage``) so that no caller can skip the copy unknowingly;
  ``append_tokens_cow`` performs it.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import numpy as np


class PoolError(Exception):
    pass


class OutOfPages(PoolError):
    pass


class SequenceExists(PoolError):
    pass


class UnknownSequence(PoolError):
    pass


class SharedLastPage(PoolError):
    pass


def pages_needed(num_tokens: int, page_size: int) -> int:
    return (num_tokens + page_size - 1) // page_size


class PagePoolModel:
    def __init__(self, page_size: int, num_pages: int,
                 initial_free_order: Optional[Iterable[int]] = None):
        if page_size <= 0 or num_pages < 0:
            raise ValueError("bad pool shape")
        self.page_size = page_size
        self.num_pages = num_pages
        if initial_free_order is None:
            self.free_pages: List[int] = list(range(num_pages))
        else:
            self.free_pages = [int(p) for p in initial_free_order]
            if sorted(self.free_pages) != list(range(num_pages)):
                raise ValueError("initial free order must be a permutation of the pages")
        self.page_table: Dict[int, List[int]] = {}
        self.token_count: Dict[int, int] = {}
        self.refcount: Dict[int, int] = {}       # owners of every page in use

    def _slots(self, seq_id: int, first: int, count: int) -> List[int]:
        pages = self.page_table[seq_id]
        ps = self.page_size
        return [pages[t // ps] * ps + t % ps for t in range(first, first + count)]

    def allocate(self, seq_id: int, num_tokens: int) -> List[int]:
        if num_tokens < 0:
            raise ValueError("negative token count")
        if seq_id in self.page_table:
            raise SequenceExists(seq_id)
        need = pages_needed(num_tokens, self.page_size)
        if need > len(self.free_pages):
            raise OutOfPages(need)
        self.page_table[seq_id] = [self.free_pages.pop() for _ in range(need)]
        for page in self.page_table[seq_id]:
            self.refcount[page] = 1
        self.token_count[seq_id] = num_tokens
        return self._slots(seq_id, 0, num_tokens)

    def fork(self, parent_id: int, child_id: int) -> None:
        if parent_id not in self.page_table:
            raise UnknownSequence(parent_id)
        if child_id in self.page_table:
            raise SequenceExists(child_id)
        self.page_table[child_id] = list(self.page_table[parent_id])
        self.token_count[child_id] = self.token_count[parent_id]
        for page in self.page_table[child_id]:
            self.refcount[page] += 1

    def _needs_copy(self, seq_id: int, n_new: int) -> bool:
        pages = self.page_table[seq_id]
        usage = self.token_count[seq_id]
        return n_new > 0 and usage % self.page_size != 0 and self.refcount[pages[-1]] > 1

    def append_tokens(self, seq_id: int, n_new: int) -> List[int]:
        if n_new < 0:
            raise ValueError("negative token count")
        if seq_id not in self.page_table:
            raise UnknownSequence(seq_id)
        if self._needs_copy(seq_id, n_new):
            raise SharedLastPage(seq_id)
        return self.append_tokens_cow(seq_id, n_new)[0]

    def append_tokens_cow(self, seq_id: int, n_new: int):
        """Returns (slots, copy) with copy = (old page, new page) or None."""
        if n_new < 0:
            raise ValueError("negative token count")
        if seq_id not in self.page_table:
            raise UnknownSequence(seq_id)
        pages = self.page_table[seq_id]
        capacity = len(pages) * self.page_size
        usage = self.token_count[seq_id]
        copy_needed = self._needs_copy(seq_id, n_new)
        over = pages_needed(usage + n_new - capacity, self.page_size) if usage + n_new > capacity else 0
        if over + (1 if copy_needed else 0) > len(self.free_pages):
            raise OutOfPages(over + (1 if copy_needed else 0))
        copy = None
        if copy_needed:
            old, new = pages[-1], self.free_pages.pop()
            self.refcount[old] -= 1
            self.refcount[new] = 1
            pages[-1] = new
            copy = (old, new)
        for _ in range(over):
            page = self.free_pages.pop()
            self.refcount[page] = 1
            pages.append(page)
        self.token_count[seq_id] = usage + n_new
        return self._slots(seq_id, usage, n_new), copy

    def release(self, seq_id: int) -> None:
        if seq_id not in self.page_table:
            raise UnknownSequence(seq_id)
        for page in self.page_table.pop(seq_id):
            self.refcount[page] -= 1
            if self.refcount[page] == 0:
                del self.refcount[page]
                self.free_pages.append(page)
        del self.token_count[seq_id]

    def free_page_count(self) -> int:
        return len(self.free_pages)

    def seq_info(self, seq_id: int):
        if seq_id not in self.page_table:
            raise UnknownSequence(seq_id)
        return self.token_count[seq_id], len(self.page_table[seq_id])

    def block_tables(self, seq_ids: List[int], max_blocks: int):
        bt = np.full((len(seq_ids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seq_ids), dtype=np.int32)
        for i, s in enumerate(seq_ids):
            if s not in self.page_table:
                raise UnknownSequence(s)
            pages = self.page_table[s]
            if len(pages) > max_blocks:
                raise ValueError("max_blocks too small")
            bt[i, :len(pages)] = pages
            lens[i] = self.token_count[s]
        return bt, lens
