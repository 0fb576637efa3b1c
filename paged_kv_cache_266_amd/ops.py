"""Decode attention and K/V writes on torch tensors, through libpagedkv.

These functions only marshal arguments: tensor data pointers, sizes and the
current HIP stream go to the C ABI, and every step runs in the library's HIP
kernels.  PyTorch provides device memory and streams.
"""

from __future__ import annotations

import ctypes
from typing import Optional

from ._lib import DTYPE_CODES, CopyArgs, DecodeArgs, PrefillArgs, WriteArgs, check, lib


def _dtype_name(t) -> str:
    import torch

    m = {torch.float16: "f16", torch.bfloat16: "bf16", torch.int8: "i8", torch.float8_e4m3fn: "fp8"}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream, device) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_tensor(t, name, device, ndim=None):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def decode_args(q, k_pool, v_pool, block_tables, context_lens, scale: float, *,
                max_context_len: int, out=None, k_scale=None, v_scale=None,
                workspace=None, merge_counters=None, num_splits: int = 0) -> DecodeArgs:
    """Fill the C argument struct from tensors (no device work)."""
    import torch

    device = q.device
    for t, n, nd in ((q, "q", 3), (k_pool, "k_pool", 4), (v_pool, "v_pool", 4),
                     (block_tables, "block_tables", 2), (context_lens, "context_lens", 1),
                     (out, "out", 3), (k_scale, "k_scale", 3), (v_scale, "v_scale", 3)):
        _check_tensor(t, n, device, nd)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    B, Hq, D = q.shape
    num_pages, Hkv, PS, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shape does not match q")
    a = DecodeArgs()
    a.q, a.k_pool, a.v_pool = _ptr(q), _ptr(k_pool), _ptr(v_pool)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.block_tables, a.context_lens = _ptr(block_tables), _ptr(context_lens)
    a.out = _ptr(out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.merge_counters = _ptr(merge_counters)
    a.merge_counter_bytes = 0 if merge_counters is None else merge_counters.numel() * merge_counters.element_size()
    a.batch, a.num_q_heads, a.num_kv_heads, a.head_dim = B, Hq, Hkv, D
    a.page_size, a.num_pages = PS, num_pages
    a.max_blocks = block_tables.shape[1]
    a.max_context_len = int(max_context_len)
    a.num_splits = int(num_splits)
    a.q_dtype = DTYPE_CODES[_dtype_name(q)]
    a.kv_dtype = DTYPE_CODES[_dtype_name(k_pool)]
    a.scale = float(scale)
    return a


def workspace_bytes(args: DecodeArgs) -> int:
    n = ctypes.c_size_t()
    check(lib().pkv_decode_workspace_bytes(ctypes.byref(args), ctypes.byref(n)), "workspace_bytes")
    return int(n.value)


def counter_bytes(args: DecodeArgs) -> int:
    n = ctypes.c_size_t()
    check(lib().pkv_decode_counter_bytes(ctypes.byref(args), ctypes.byref(n)), "counter_bytes")
    return int(n.value)


def alloc_workspace(args: DecodeArgs, device):
    """A workspace tensor for these arguments (None when none is needed)."""
    import torch

    n = workspace_bytes(args)
    if n == 0:
        return None
    # torch's caching allocator hands out 512-byte aligned blocks
    return torch.empty(n, dtype=torch.uint8, device=device)


def alloc_merge_counters(args: DecodeArgs, device, at_least: int = 0):
    """A zero-filled merge-counter array for these arguments (None when none
    is needed).  Keep it for later calls: each call leaves it zero again, so
    it needs no clearing as long as calls using it do not overlap in time."""
    import torch

    n = max(counter_bytes(args), at_least)
    if n == 0:
        return None
    return torch.zeros((n + 3) // 4, dtype=torch.int32, device=device)


def paged_attn_decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, *,
                      max_context_len: int, out=None, k_scale=None, v_scale=None,
                      workspace=None, merge_counters=None, num_splits: int = 0, stream=None):
    """Single-token decode attention over a paged KV cache.

    q [B][Hq][D] f16/bf16; k_pool, v_pool [num_pages][Hkv][PS][D] of the same
    type as q, or int8 / float8_e4m3fn (then k_scale, v_scale
    [num_pages][Hkv][PS] fp32);
    block_tables [B][max_blocks] int32; context_lens [B] int32 (device).
    ``max_context_len`` is a host-side bound on context_lens.  ``num_splits``
    is the number of waves sharing the batch's tiles (0 = library default).
    When ``workspace`` or ``merge_counters`` is not given, a buffer kept per
    (device, stream) is used, grown when a call needs more (see
    _stream_buffers): calls on one stream run in order, so they can share
    it, and the counters need no clearing because every call leaves them
    zero.
    Returns ``out`` [B][Hq][D] in q's dtype.
    """
    import torch

    if out is None:
        out = torch.empty_like(q)
    a = decode_args(q, k_pool, v_pool, block_tables, context_lens, scale,
                    max_context_len=max_context_len, out=out, k_scale=k_scale, v_scale=v_scale,
                    workspace=workspace, merge_counters=merge_counters, num_splits=num_splits)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if workspace is None or merge_counters is None:
        ws, ctr = _stream_buffers(a, q.device, stream)
        if workspace is None:
            a.workspace = _ptr(ws)
            a.workspace_bytes = 0 if ws is None else ws.numel()
        if merge_counters is None:
            a.merge_counters = _ptr(ctr)
            a.merge_counter_bytes = 0 if ctr is None else 4 * ctr.numel()
    check(lib().pkv_paged_attn_decode(ctypes.byref(a), stream.cuda_stream), "paged_attn_decode")
    return out


# (device index, stream handle) -> [workspace, merge counters]
_STREAM_BUFFERS: dict = {}


def _stream_buffers(args: DecodeArgs, device, stream):
    """The workspace and merge counters kept for calls on ``stream``.

    They are made on that stream, so when a larger call replaces them,
    torch's allocator hands their memory out again only behind the work
    already queued there.  A fresh counter array is zero; after that every
    call leaves it zero.  One entry per stream a caller has used stays
    until the process ends (or release_stream_buffers)."""
    import torch

    key = (torch.device(device).index, stream.cuda_stream)
    entry = _STREAM_BUFFERS.setdefault(key, [None, None])
    need_ws = workspace_bytes(args)
    need_ctr = counter_bytes(args)
    with torch.cuda.stream(stream):
        if need_ws and (entry[0] is None or entry[0].numel() < need_ws):
            entry[0] = torch.empty(need_ws, dtype=torch.uint8, device=device)
        if need_ctr and (entry[1] is None or 4 * entry[1].numel() < need_ctr):
            entry[1] = torch.zeros((need_ctr + 3) // 4, dtype=torch.int32, device=device)
    return (entry[0] if need_ws else None), (entry[1] if need_ctr else None)


def release_stream_buffers() -> None:
    """Drop the buffers paged_attn_decode keeps per stream."""
    _STREAM_BUFFERS.clear()


def paged_prefill(q, k_pool, v_pool, block_tables, q_start, context_lens, scale: float, *,
                  max_context_len: int, max_q_len: int, out=None, k_scale=None, v_scale=None, stream=None):
    """Chunked prefill attention over a paged cache.

    q [n_q][Hq][D] f16/bf16: sequence b's new tokens are rows
    q_start[b] .. q_start[b+1]-1 (q_start int32 [B+1], device); the pools
    (of q's type, or int8 / float8_e4m3fn with k_scale, v_scale
    [num_pages][Hkv][PS] fp32) already hold their K/V, and context_lens [B]
    counts them.  Query i of sequence b attends to keys
    0 .. context_lens[b] - nq_b + i.  Returns out [n_q][Hq][D] in q's type."""
    import torch

    device = q.device
    for t, n, nd in ((q, "q", 3), (k_pool, "k_pool", 4), (v_pool, "v_pool", 4),
                     (block_tables, "block_tables", 2), (q_start, "q_start", 1),
                     (context_lens, "context_lens", 1), (out, "out", 3)):
        _check_tensor(t, n, device, nd)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or q_start.dtype != torch.int32:
        raise TypeError("block_tables, q_start and context_lens must be int32")
    n_q, Hq, D = q.shape
    num_pages, Hkv, PS, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shape does not match q")
    if out is None:
        out = torch.empty_like(q)
    a = PrefillArgs()
    a.q, a.k_pool, a.v_pool = _ptr(q), _ptr(k_pool), _ptr(v_pool)
    a.block_tables, a.q_start, a.context_lens, a.out = _ptr(block_tables), _ptr(q_start), _ptr(context_lens), _ptr(out)
    a.batch, a.n_q, a.num_q_heads, a.num_kv_heads, a.head_dim = context_lens.shape[0], n_q, Hq, Hkv, D
    a.page_size, a.num_pages, a.max_blocks = PS, num_pages, block_tables.shape[1]
    a.max_context_len, a.max_q_len = int(max_context_len), int(max_q_len)
    a.q_dtype = DTYPE_CODES[_dtype_name(q)]
    a.kv_dtype = DTYPE_CODES[_dtype_name(k_pool)]
    a.scale = float(scale)
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is not None:
            _check_tensor(t, n, device, 3)
            if t.dtype != torch.float32:
                raise TypeError(f"{n} must be float32")
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    check(lib().pkv_paged_prefill(ctypes.byref(a), _stream_handle(stream, device)), "paged_prefill")
    return out


def write_kv(k_new, v_new, slots, k_pool, v_pool, *, k_scale_new=None, v_scale_new=None,
             k_scale=None, v_scale=None, stream=None) -> None:
    """Scatter appended tokens' K/V ([n][Hkv][D]) into their pool slots.

    With an int8 / fp8 pool, k_new / v_new are either already encoded (same
    dtype as the pool, with k_scale_new / v_scale_new [n][Hkv]) or f16 /
    bf16 rows that the library quantises on the device (scales written to
    k_scale / v_scale)."""
    import torch

    device = k_pool.device
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (slots, "slots"), (k_pool, "k_pool"),
                 (v_pool, "v_pool"), (k_scale_new, "k_scale_new"), (v_scale_new, "v_scale_new"),
                 (k_scale, "k_scale"), (v_scale, "v_scale")):
        _check_tensor(t, n, device)
    if slots.dtype != torch.int64:
        raise TypeError("slots must be int64")
    num_pages, Hkv, PS, D = k_pool.shape
    a = WriteArgs()
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
    a.k_scale_new, a.v_scale_new = _ptr(k_scale_new), _ptr(v_scale_new)
    a.slots = _ptr(slots)
    a.k_pool, a.v_pool = _ptr(k_pool), _ptr(v_pool)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.n = k_new.shape[0]
    a.num_kv_heads, a.head_dim, a.page_size, a.num_pages = Hkv, D, PS, num_pages
    a.kv_dtype = DTYPE_CODES[_dtype_name(k_pool)]
    a.src_dtype = DTYPE_CODES[_dtype_name(k_new)]
    check(lib().pkv_write_kv(ctypes.byref(a), _stream_handle(stream, device)), "write_kv")


def copy_pages(pairs, k_pool, v_pool, *, k_scale=None, v_scale=None, stream=None) -> None:
    """Copy whole pages (all KV heads) of one layer's pools: pairs is an
    int32 device tensor [n][2] of (source page, destination page), as the
    copy-on-write of append_tokens_cow reports them."""
    import torch

    device = k_pool.device
    for t, n in ((pairs, "pairs"), (k_pool, "k_pool"), (v_pool, "v_pool"), (k_scale, "k_scale"),
                 (v_scale, "v_scale")):
        _check_tensor(t, n, device)
    if pairs.dtype != torch.int32:
        raise TypeError("pairs must be int32")
    num_pages, Hkv, PS, D = k_pool.shape
    a = CopyArgs()
    a.k_pool, a.v_pool = _ptr(k_pool), _ptr(v_pool)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.pairs = _ptr(pairs)
    a.n = pairs.shape[0]
    a.num_pages, a.num_kv_heads, a.page_size, a.head_dim = num_pages, Hkv, PS, D
    a.kv_dtype = DTYPE_CODES[_dtype_name(k_pool)]
    check(lib().pkv_copy_pages(ctypes.byref(a), _stream_handle(stream, device)), "copy_pages")
