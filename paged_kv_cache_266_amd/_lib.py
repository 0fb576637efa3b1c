"""ctypes binding of libpagedkv (include/pagedkv.h).

Argument marshalling only.  The library must have been built in-tree
(``python -m paged_kv_cache_266_amd.build``); there is no fallback of any
kind when it is missing -- loading raises.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OOM = -2
PKV_ERR_NO_SEQ = -3
PKV_ERR_SEQ_EXISTS = -4
PKV_ERR_UNSUPPORTED = -5
PKV_ERR_WORKSPACE = -6
PKV_ERR_DEVICE = -7
PKV_ERR_SHARED_PAGE = -8

PKV_F16, PKV_BF16, PKV_I8, PKV_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODES = {"f16": PKV_F16, "bf16": PKV_BF16, "i8": PKV_I8, "fp8": PKV_FP8_E4M3}

EXPORTED = [
    "pkv_abi_version", "pkv_status_string", "pkv_last_error", "pkv_device_count",
    "pkv_pool_create", "pkv_pool_destroy", "pkv_seq_alloc", "pkv_append_tokens",
    "pkv_seq_release", "pkv_seq_info", "pkv_seq_pages", "pkv_free_page_count",
    "pkv_free_pages", "pkv_build_block_tables", "pkv_kv_bytes",
    "pkv_decode_workspace_bytes", "pkv_decode_counter_bytes", "pkv_decode_num_splits",
    "pkv_decode_validate",
    "pkv_paged_attn_decode", "pkv_paged_attn_decode_partitions", "pkv_splitk_reduce",
    "pkv_paged_attn_decode_noalloc", "pkv_write_kv", "pkv_seq_fork", "pkv_append_tokens_cow", "pkv_page_owners", "pkv_copy_pages",
    "pkv_sched_create", "pkv_sched_destroy", "pkv_sched_submit", "pkv_sched_finish", "pkv_sched_step",
    "pkv_sched_get_stats", "pkv_sched_batch_tables", "pkv_paged_prefill",
    "pkv_serve_slot_bytes", "pkv_serve_create", "pkv_serve_destroy", "pkv_serve_step",
]

# The host-only build (page pool, scheduler, status codes; no GPU entry
# points): the sanitizer build of the host code loads it through the
# PKV_HOST_LIBRARY environment variable instead of libpagedkv.so.
HOST_EXPORTED = [
    "pkv_abi_version", "pkv_status_string", "pkv_last_error",
    "pkv_pool_create", "pkv_pool_destroy", "pkv_seq_alloc", "pkv_append_tokens",
    "pkv_seq_release", "pkv_seq_info", "pkv_seq_pages", "pkv_free_page_count",
    "pkv_free_pages", "pkv_build_block_tables", "pkv_kv_bytes",
    "pkv_seq_fork", "pkv_append_tokens_cow", "pkv_page_owners",
    "pkv_sched_create", "pkv_sched_destroy", "pkv_sched_submit", "pkv_sched_finish", "pkv_sched_step",
    "pkv_sched_get_stats", "pkv_sched_batch_tables",
]
HOST_LIBRARY_ENV = "PKV_HOST_LIBRARY"

PKV_SCHED_CONTINUOUS, PKV_SCHED_STATIC = 0, 1


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("initial_free_order", ctypes.POINTER(ctypes.c_int32))]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("merge_counters", ctypes.c_void_p), ("merge_counter_bytes", ctypes.c_size_t),
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
    ]


class WriteArgs(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_scale_new", ctypes.c_void_p), ("v_scale_new", ctypes.c_void_p),
        ("slots", ctypes.c_void_p), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("n", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("kv_dtype", ctypes.c_int),
        ("src_dtype", ctypes.c_int),
    ]


class CopyArgs(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("pairs", ctypes.c_void_p),
        ("n", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("q_start", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32), ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
    ]


class SchedStepOut(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("n_running", ctypes.c_int32),
                ("n_admitted", ctypes.c_int32), ("n_retired", ctypes.c_int32)]


class SchedStats(ctypes.Structure):
    _fields_ = [("now", ctypes.c_int64), ("waiting", ctypes.c_int32), ("running", ctypes.c_int32),
                ("finished", ctypes.c_int64), ("wait_sum", ctypes.c_int64)]


class ServeDesc(ctypes.Structure):
    _fields_ = [
        ("sched", ctypes.c_void_p), ("max_blocks", ctypes.c_int32), ("max_prompt_tokens", ctypes.c_int32),
        ("ring", ctypes.c_int32), ("host_staging", ctypes.c_void_p), ("dev_staging", ctypes.c_void_p),
        ("decode", DecodeArgs), ("append", WriteArgs),
        ("k_prompt", ctypes.c_void_p), ("v_prompt", ctypes.c_void_p),
        ("k_prompt_scale", ctypes.c_void_p), ("v_prompt_scale", ctypes.c_void_p),
    ]


class ServeStepOut(ctypes.Structure):
    _fields_ = [("sched", SchedStepOut), ("prompt_tokens", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("slot_wait_us", ctypes.c_float)]


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class KVCacheOOM(PagedKVError):
    """The free-page list cannot cover the request (the OOMError of the
    paged-KV sketch); the pool is unchanged."""


class UnknownSequence(PagedKVError, KeyError):
    pass


class SequenceExists(PagedKVError):
    pass


class Unsupported(PagedKVError):
    pass


class WorkspaceError(PagedKVError):
    pass


class DeviceError(PagedKVError):
    pass


class SharedPage(PagedKVError):
    """The append would write into a page other sequences share; use
    append_tokens_cow and copy the page on the device."""


_EXC = {PKV_ERR_OOM: KVCacheOOM, PKV_ERR_NO_SEQ: UnknownSequence,
        PKV_ERR_SEQ_EXISTS: SequenceExists, PKV_ERR_UNSUPPORTED: Unsupported,
        PKV_ERR_WORKSPACE: WorkspaceError, PKV_ERR_DEVICE: DeviceError,
        PKV_ERR_SHARED_PAGE: SharedPage}

_lib = None


def _signatures():
    i32, i64, sz, vp, ci = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    P = ctypes.POINTER
    sig = {
        "pkv_abi_version": (i32, []),
        "pkv_status_string": (ctypes.c_char_p, [ci]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_device_count": (i32, []),
        "pkv_pool_create": (ci, [P(PoolDesc), P(vp)]),
        "pkv_pool_destroy": (None, [vp]),
        "pkv_seq_alloc": (ci, [vp, i64, i32, P(i64)]),
        "pkv_append_tokens": (ci, [vp, i64, i32, P(i64)]),
        "pkv_seq_release": (ci, [vp, i64]),
        "pkv_seq_info": (ci, [vp, i64, P(i32), P(i32)]),
        "pkv_seq_pages": (ci, [vp, i64, P(i32), i32, P(i32)]),
        "pkv_free_page_count": (i32, [vp]),
        "pkv_free_pages": (ci, [vp, P(i32), i32, P(i32)]),
        "pkv_build_block_tables": (ci, [vp, P(i64), i32, i32, P(i32), P(i32)]),
        "pkv_kv_bytes": (i64, [i32, i32, i32, i64, i32, ci]),
        "pkv_decode_workspace_bytes": (ci, [P(DecodeArgs), P(sz)]),
        "pkv_decode_counter_bytes": (ci, [P(DecodeArgs), P(sz)]),
        "pkv_decode_num_splits": (i32, [P(DecodeArgs)]),
        "pkv_decode_validate": (ci, [P(DecodeArgs)]),
        "pkv_write_kv": (ci, [P(WriteArgs), vp]),
        "pkv_seq_fork": (ci, [vp, i64, i64]),
        "pkv_append_tokens_cow": (ci, [vp, i64, i32, P(i64), P(i32), P(i32)]),
        "pkv_page_owners": (i32, [vp, i32]),
        "pkv_copy_pages": (ci, [P(CopyArgs), vp]),
        "pkv_sched_create": (ci, [vp, i32, ci, P(vp)]),
        "pkv_sched_destroy": (None, [vp]),
        "pkv_sched_submit": (ci, [vp, i64, i32, i32, i64]),
        "pkv_sched_finish": (ci, [vp, i64]),
        "pkv_sched_step": (ci, [vp, i32, P(i64), P(i64), P(i32), P(i64), P(i64), P(SchedStepOut)]),
        "pkv_paged_prefill": (ci, [P(PrefillArgs), vp]),
        "pkv_sched_batch_tables": (ci, [vp, i32, i32, P(i32), P(i32), P(i32)]),
        "pkv_sched_get_stats": (ci, [vp, P(SchedStats)]),
        "pkv_serve_slot_bytes": (ci, [P(ServeDesc), P(sz)]),
        "pkv_serve_create": (ci, [P(ServeDesc), P(vp)]),
        "pkv_serve_destroy": (None, [vp]),
        "pkv_serve_step": (ci, [vp, vp, P(ServeStepOut), P(i64)]),
    }
    for name in ("pkv_paged_attn_decode", "pkv_paged_attn_decode_partitions", "pkv_splitk_reduce",
                 "pkv_paged_attn_decode_noalloc"):
        sig[name] = (ci, [P(DecodeArgs), vp])
    return sig


def _declare(L, host_only: bool = False):
    for name, (res, args) in _signatures().items():
        if host_only and name not in HOST_EXPORTED:
            continue
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """Load libpagedkv.so (raises if it has not been built).  With
    PKV_HOST_LIBRARY set, load that host-only build instead: only the pool,
    scheduler and status entry points exist then, and any device call fails
    with AttributeError."""
    global _lib
    if _lib is None and os.environ.get(HOST_LIBRARY_ENV):
        _lib = _declare(ctypes.CDLL(os.environ[HOST_LIBRARY_ENV]), host_only=True)
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_266_amd.build` "
                "(there is no fallback path)")
        try:
            # torch first, so that the HIP runtime torch ships is the one both use
            import torch  # noqa: F401
        except ImportError:
            pass
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def check(status: int, what: str = "") -> None:
    if status != PKV_OK:
        L = lib()
        msg = L.pkv_last_error().decode() or L.pkv_status_string(status).decode()
        raise _EXC.get(status, PagedKVError)(status, f"{what}: {msg}" if what else msg)
