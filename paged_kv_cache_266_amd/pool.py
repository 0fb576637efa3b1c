"""KVPool: the host page allocator of libpagedkv behind a Python object.

Mirrors the allocator of "TensorRT-LLM 深度实战" (chenxutan.com), section
3.1 -- allocate, append_tokens, release, a page table per sequence, and an
out-of-memory error (``KVCacheOOM``) when the free list runs dry -- with every
operation carried out by the C library.
"""

from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from ._lib import PoolDesc, check, lib


class KVPool:
    def __init__(self, num_pages: int, page_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        L = lib()
        self._order = None
        ptr = None
        if initial_free_order is not None:
            self._order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            ptr = self._order.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        desc = PoolDesc(num_pages, page_size, ptr)
        h = ctypes.c_void_p()
        check(L.pkv_pool_create(ctypes.byref(desc), ctypes.byref(h)), "pkv_pool_create")
        self._h = h
        self.num_pages = num_pages
        self.page_size = page_size

    # -- lifetime
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- allocator
    def allocate(self, seq_id: int, num_tokens: int) -> np.ndarray:
        """Admit a sequence; returns the slot ids of its tokens."""
        slots = np.empty(max(num_tokens, 1), dtype=np.int64)
        check(lib().pkv_seq_alloc(self._h, seq_id, num_tokens,
                                  slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
              "allocate")
        return slots[:num_tokens]

    def append_tokens(self, seq_id: int, n_new: int) -> np.ndarray:
        """Grow a sequence; returns the slot ids of the new tokens."""
        slots = np.empty(max(n_new, 1), dtype=np.int64)
        check(lib().pkv_append_tokens(self._h, seq_id, n_new,
                                      slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
              "append_tokens")
        return slots[:n_new]

    def append_tokens_cow(self, seq_id: int, n_new: int):
        """Grow a sequence whose last page may be shared.  Returns (slots,
        copy) where copy is (old page, new page) to copy on the device before
        writing the new tokens, or None."""
        slots = np.empty(max(n_new, 1), dtype=np.int64)
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        check(lib().pkv_append_tokens_cow(self._h, seq_id, n_new,
                                          slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          ctypes.byref(src), ctypes.byref(dst)), "append_tokens_cow")
        return slots[:n_new], (None if src.value < 0 else (src.value, dst.value))

    def fork(self, parent_id: int, child_id: int) -> None:
        """New sequence child_id sharing parent_id's pages (prefix reuse)."""
        check(lib().pkv_seq_fork(self._h, parent_id, child_id), "fork")

    def page_owners(self, page: int) -> int:
        return int(lib().pkv_page_owners(self._h, page))

    def release(self, seq_id: int) -> None:
        check(lib().pkv_seq_release(self._h, seq_id), "release")

    def seq_info(self, seq_id: int) -> Tuple[int, int]:
        n, p = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pkv_seq_info(self._h, seq_id, ctypes.byref(n), ctypes.byref(p)), "seq_info")
        return n.value, p.value

    def pages(self, seq_id: int) -> List[int]:
        _, npg = self.seq_info(seq_id)
        buf = np.empty(max(npg, 1), dtype=np.int32)
        cnt = ctypes.c_int32()
        check(lib().pkv_seq_pages(self._h, seq_id, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  npg, ctypes.byref(cnt)), "pages")
        return buf[:cnt.value].tolist()

    def free_page_count(self) -> int:
        return int(lib().pkv_free_page_count(self._h))

    def free_pages(self) -> List[int]:
        n = self.free_page_count()
        buf = np.empty(max(n, 1), dtype=np.int32)
        cnt = ctypes.c_int32()
        check(lib().pkv_free_pages(self._h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n,
                                   ctypes.byref(cnt)), "free_pages")
        return buf[:cnt.value].tolist()

    def block_tables(self, seq_ids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        B = ids.shape[0]
        bt = np.empty((max(B, 1), max(max_blocks, 1)), dtype=np.int32)
        lens = np.empty(max(B, 1), dtype=np.int32)
        check(lib().pkv_build_block_tables(
            self._h, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), B, max_blocks,
            bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))), "block_tables")
        return bt[:B, :max_blocks], lens[:B]


def kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, batch: int, dtype: str) -> int:
    from ._lib import DTYPE_CODES

    v = lib().pkv_kv_bytes(layers, kv_heads, head_dim, tokens, batch, DTYPE_CODES[dtype])
    if v < 0:
        raise ValueError("kv_bytes: negative argument or overflow")
    return int(v)
