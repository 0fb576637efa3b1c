"""libpagedkv: single-token decode attention over a paged KV cache, MI355X.

Python face of the C library (include/pagedkv.h).  The library is loaded on
first use; if it has not been built, that first use raises -- nothing here
computes attention itself.
"""

from ._lib import (KVCacheOOM, PagedKVError, SequenceExists, SharedPage, Unsupported,  # noqa: F401
                   UnknownSequence, WorkspaceError, DeviceError, lib)
from .pool import KVPool, kv_bytes  # noqa: F401
from .sched import CONTINUOUS, STATIC, Scheduler  # noqa: F401
from .serve import ServeLoop  # noqa: F401
from .ops import (alloc_merge_counters, alloc_workspace, copy_pages, counter_bytes,  # noqa: F401
                  decode_args, paged_attn_decode, paged_prefill, release_stream_buffers,
                  workspace_bytes, write_kv)
