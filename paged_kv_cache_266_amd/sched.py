"""Continuous-batching step driver (libpagedkv's pkv_sched_* calls).

Argument marshalling only; the scheduler itself is native (csrc/sched.cpp).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List

import numpy as np

from ._lib import (PKV_SCHED_CONTINUOUS, PKV_SCHED_STATIC, SchedStats, SchedStepOut, check, lib)
from .pool import KVPool

CONTINUOUS, STATIC = PKV_SCHED_CONTINUOUS, PKV_SCHED_STATIC


@dataclass
class Step:
    step: int                   # clock of this step
    seq_ids: np.ndarray         # int64 [n]: the batch, admission order
    new_slots: np.ndarray       # int64 [n]: where each sequence's new token's K/V goes
    context_lens: np.ndarray    # int32 [n]: tokens after the append
    admitted: np.ndarray        # int64: joined this step
    retired: np.ndarray         # int64: left this step


class Scheduler:
    """Runs requests over a KVPool, max_batch sequences per step."""

    def __init__(self, pool: KVPool, max_batch: int, policy: int = CONTINUOUS):
        h = ctypes.c_void_p()
        check(lib().pkv_sched_create(pool._h, max_batch, policy, ctypes.byref(h)), "pkv_sched_create")
        self._h = h
        self.pool = pool            # the pool must outlive the scheduler
        self.max_batch = max_batch
        n = max_batch
        self._ids = np.empty(n, np.int64)
        self._slots = np.empty(n, np.int64)
        self._lens = np.empty(n, np.int32)
        self._adm = np.empty(n, np.int64)
        self._ret = np.empty(n, np.int64)
        p64, p32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
        self._out = SchedStepOut()
        self._argv = (self._ids.ctypes.data_as(p64), self._slots.ctypes.data_as(p64),
                      self._lens.ctypes.data_as(p32), self._adm.ctypes.data_as(p64),
                      self._ret.ctypes.data_as(p64), ctypes.byref(self._out))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().pkv_sched_destroy(self._h)
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

    def submit(self, seq_id: int, prompt_len: int, max_new_tokens: int, arrive_step: int = 0) -> None:
        check(lib().pkv_sched_submit(self._h, seq_id, prompt_len, max_new_tokens, arrive_step), "submit")

    def finish(self, seq_id: int) -> None:
        check(lib().pkv_sched_finish(self._h, seq_id), "finish")

    def step(self) -> Step:
        check(lib().pkv_sched_step(self._h, self.max_batch, *self._argv), "step")
        out = self._out
        n = out.n_running
        return Step(out.step, self._ids[:n].copy(), self._slots[:n].copy(), self._lens[:n].copy(),
                    self._adm[:out.n_admitted].copy(), self._ret[:out.n_retired].copy())

    def batch_tables(self, max_blocks: int, block_tables=None, context_lens=None):
        """Block tables [n][max_blocks] and context lengths [n] (int32) of the
        last step's batch.  Writes into the given arrays (host memory of at
        least max_batch rows, e.g. pinned staging) when passed; returns the
        filled views."""
        p32 = ctypes.POINTER(ctypes.c_int32)
        bt = np.empty((self.max_batch, max_blocks), np.int32) if block_tables is None else block_tables
        lens = np.empty(self.max_batch, np.int32) if context_lens is None else context_lens
        if bt.dtype != np.int32 or lens.dtype != np.int32 or not bt.flags.c_contiguous or bt.shape[1] != max_blocks:
            raise ValueError("block_tables must be C-contiguous int32 [rows][max_blocks], context_lens int32")
        cap = min(bt.shape[0], lens.shape[0])
        n = ctypes.c_int32()
        check(lib().pkv_sched_batch_tables(self._h, cap, max_blocks, bt.ctypes.data_as(p32),
                                           lens.ctypes.data_as(p32), ctypes.byref(n)), "batch_tables")
        return bt[:n.value], lens[:n.value]

    def stats(self) -> dict:
        st = SchedStats()
        check(lib().pkv_sched_get_stats(self._h, ctypes.byref(st)), "stats")
        return {"now": st.now, "waiting": st.waiting, "running": st.running,
                "finished": st.finished, "wait_sum": st.wait_sum}

    def done(self) -> bool:
        st = self.stats()
        return st["waiting"] == 0 and st["running"] == 0
