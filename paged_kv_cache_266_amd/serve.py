"""One serving step per call (libpagedkv's pkv_serve_* calls).

Argument marshalling only: the scheduler step, the staging of the step's
data, the K/V appends and the decode are the library's (csrc/serve.cpp and
the kernels it launches).  PyTorch provides the device buffers, the pinned
host staging ring and the stream.
"""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import DTYPE_CODES, ServeDesc, ServeStepOut, WriteArgs, check, lib
from .ops import _check_tensor, _dtype_name, _ptr, _stream_handle, alloc_merge_counters, alloc_workspace, \
    decode_args
from .sched import Scheduler


class ServeLoop:
    """Runs a Scheduler's steps over one layer's pools: each ``step()`` is one
    library call that schedules, stages, appends the admitted prompts' and
    the new tokens' K/V and decodes the batch, asynchronously on ``stream``.

    q, out [max_batch][Hq][D]; k_new, v_new [max_batch][Hkv][D] (the new
    tokens' K/V rows, in batch order); k_prompt, v_prompt
    [max_prompt_tokens][Hkv][D] (the admitted prompts' rows, packed in
    admission order); rows are in q's type (quantised on the device for int8 /
    fp8 pools) or already in the pool's type."""

    def __init__(self, sched: Scheduler, q, k_pool, v_pool, scale: float, *, k_new, v_new, k_prompt, v_prompt,
                 max_blocks: int, out=None, k_scale=None, v_scale=None, ring: int = 4, num_splits: int = 0,
                 stream=None):
        import torch

        device = q.device
        self.sched = sched                       # keeps the scheduler (and its pool) alive
        self.max_batch = sched.max_batch
        if q.shape[0] != self.max_batch:
            raise ValueError("q must have max_batch rows")
        for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_prompt, "k_prompt"), (v_prompt, "v_prompt")):
            _check_tensor(t, n, device, 3)
        num_pages, Hkv, PS, D = k_pool.shape
        self.out = torch.empty_like(q) if out is None else out
        # placeholders for the per-step tables (the library points the decode
        # at its device staging buffer)
        bt0 = torch.empty((self.max_batch, max_blocks), dtype=torch.int32, device=device)
        ctx0 = torch.empty(self.max_batch, dtype=torch.int32, device=device)
        a = decode_args(q, k_pool, v_pool, bt0, ctx0, scale, max_context_len=max_blocks * PS, out=self.out,
                        k_scale=k_scale, v_scale=v_scale, num_splits=num_splits)
        self._ws = alloc_workspace(a, device)
        self._ctr = alloc_merge_counters(a, device)
        a.workspace, a.workspace_bytes = _ptr(self._ws), 0 if self._ws is None else self._ws.numel()
        a.merge_counters = _ptr(self._ctr)
        a.merge_counter_bytes = 0 if self._ctr is None else 4 * self._ctr.numel()
        w = WriteArgs()
        w.k_new, w.v_new = _ptr(k_new), _ptr(v_new)
        w.k_pool, w.v_pool = _ptr(k_pool), _ptr(v_pool)
        w.k_scale, w.v_scale = _ptr(k_scale), _ptr(v_scale)
        w.num_kv_heads, w.head_dim, w.page_size, w.num_pages = Hkv, D, PS, num_pages
        w.kv_dtype = DTYPE_CODES[_dtype_name(k_pool)]
        w.src_dtype = DTYPE_CODES[_dtype_name(k_new)]
        d = ServeDesc()
        d.sched = sched._h.value
        d.max_blocks = max_blocks
        d.max_prompt_tokens = k_prompt.shape[0]
        d.ring = ring
        d.decode = a
        d.append = w
        d.k_prompt, d.v_prompt = _ptr(k_prompt), _ptr(v_prompt)
        n = ctypes.c_size_t()
        check(lib().pkv_serve_slot_bytes(ctypes.byref(d), ctypes.byref(n)), "pkv_serve_slot_bytes")
        self.slot_bytes = int(n.value)
        self._host = torch.empty(ring * self.slot_bytes, dtype=torch.uint8, pin_memory=True)
        self._dev = torch.empty(self.slot_bytes, dtype=torch.uint8, device=device)
        d.host_staging, d.dev_staging = self._host.data_ptr(), self._dev.data_ptr()
        self._keep = (q, k_pool, v_pool, k_scale, v_scale, k_new, v_new, k_prompt, v_prompt, bt0, ctx0)
        self._desc = d
        h = ctypes.c_void_p()
        check(lib().pkv_serve_create(ctypes.byref(d), ctypes.byref(h)), "pkv_serve_create")
        self._h = h
        self._stream = _stream_handle(stream, device)
        self._res = ServeStepOut()
        self.seq_ids = np.empty(self.max_batch, np.int64)
        self._ids_p = self.seq_ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def step(self) -> ServeStepOut:
        """One step; the batch's ids are then seq_ids[:result.sched.n_running]."""
        check(lib().pkv_serve_step(self._h, self._stream, ctypes.byref(self._res), self._ids_p), "pkv_serve_step")
        return self._res

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().pkv_serve_destroy(self._h)
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
