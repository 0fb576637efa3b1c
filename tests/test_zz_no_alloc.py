"""pkv_paged_attn_decode_noalloc -- decode with the library's static scratch
instead of a caller workspace -- against pkv_paged_attn_decode, through the C
ABI (needs a gfx950 GPU).  Both run the same kernels with the same wave
count, so their outputs must be bitwise equal; each is also compared with the
fp64 oracle.  Consecutive calls share the scratch: a large batch, then a
smaller one of another shape, then an int8 one."""

import ctypes

import numpy as np
import pytest

from gpu_helpers import compare, note, small_config
from synth import make_case
from synth.device import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_266_amd as pkv

    pkv.lib()
    yield


def _decode(case, dev, splits, noalloc):
    import torch

    import paged_kv_cache_266_amd as pkv
    from paged_kv_cache_266_amd._lib import check, lib

    out = torch.full_like(dev.q, float("nan"))
    a = pkv.decode_args(dev.q, dev.k_pool, dev.v_pool, dev.block_tables, dev.context_lens, case.scale,
                        max_context_len=case.cfg.max_context_len, out=out, k_scale=dev.k_scale,
                        v_scale=dev.v_scale, num_splits=splits)
    sh = torch.cuda.current_stream().cuda_stream
    if noalloc:
        check(lib().pkv_paged_attn_decode_noalloc(ctypes.byref(a), sh), "noalloc")
    else:
        ws = pkv.alloc_workspace(a, dev.q.device)
        ctr = pkv.alloc_merge_counters(a, dev.q.device)
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        a.merge_counters, a.merge_counter_bytes = ctr.data_ptr(), 4 * ctr.numel()
        check(lib().pkv_paged_attn_decode(ctypes.byref(a), sh), "decode")
    torch.cuda.synchronize()
    return out


def test_noalloc_equals_allocating_entry_point_on_consecutive_calls():
    import torch

    calls = [
        (small_config(32, 8, 128, "bf16", "bf16", 64, (30000, 5000, 64, 4000, 0, 1)), 51, 600),
        (small_config(8, 4, 64, "f16", "f16", 16, (700, 65, 3)), 52, 0),
        (small_config(16, 16, 128, "f16", "i8", 16, (900, 17, 2500, 64)), 53, 0),
    ]
    for cfg, seed, splits in calls:
        note(f"[noalloc] B={cfg.batch} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} D={cfg.head_dim} "
             f"kv={cfg.kv_dtype} splits={splits}")
        case = make_case(cfg, seed=seed)
        dev = upload(case, "cuda")
        ref = _decode(case, dev, splits, noalloc=False)
        got = _decode(case, dev, splits, noalloc=True)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        compare(case, got, "noalloc")
