"""Place a generated workload in device memory (torch tensors).

Plain tensor plumbing: full-size pools ``[num_pages][Hkv][PS][D]`` are filled
with zeros (or the poison value) and the used pages are copied to their
physical ids.  Nothing here computes attention.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .make import BF16_NAN, F16_NAN, FP8_NAN, I8_POISON, Case


def torch_dtype(name: str):
    import torch

    return {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
            "fp8": torch.float8_e4m3fn}[name]


@dataclass
class DeviceCase:
    q: "object"                 # [B][Hq][D] f16/bf16
    k_pool: "object"            # [num_pages][Hkv][PS][D]
    v_pool: "object"
    k_scale: Optional["object"]  # [num_pages][Hkv][PS] fp32 (int8 only)
    v_scale: Optional["object"]
    block_tables: "object"      # [B][max_blocks] int32
    context_lens: "object"      # [B] int32


def _bits_tensor(bits: np.ndarray, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype))


def upload_q(case: Case, device):
    return _bits_tensor(case.q_bits, case.cfg.q_dtype).to(device)


def upload(case: Case, device, poison: Optional[bool] = None) -> DeviceCase:
    import torch

    cfg = case.cfg
    poison = case.poison if poison is None else poison
    shape = (cfg.num_pages, cfg.num_kv_heads, cfg.page_size, cfg.head_dim)
    used = torch.from_numpy(case.used_pages.astype(np.int64)).to(device)
    if cfg.kv_dtype in ("i8", "fp8"):
        # byte codes move as raw bytes (index_copy has no fp8 kernel)
        fill = (int(I8_POISON) if cfg.kv_dtype == "i8" else int(FP8_NAN)) if poison else 0
        pools = []
        for pages in (case.k_pages, case.v_pages):
            p = torch.full(shape, fill & 0xFF, dtype=torch.uint8, device=device)
            p.index_copy_(0, used, torch.from_numpy(np.ascontiguousarray(pages).view(np.uint8)).to(device))
            pools.append(p.view(torch_dtype(cfg.kv_dtype)))
        scales = []
        for sc in (case.k_scale, case.v_scale):
            s = torch.full(shape[:3], float("nan") if poison else 0.0,
                           dtype=torch.float32, device=device)
            s.index_copy_(0, used, torch.from_numpy(sc).to(device))
            scales.append(s)
        k_scale, v_scale = scales
    else:
        nan_bits = F16_NAN if cfg.kv_dtype == "f16" else BF16_NAN
        pools = []
        for pages in (case.k_pages, case.v_pages):
            p = torch.zeros(shape, dtype=torch_dtype(cfg.kv_dtype), device=device)
            if poison:
                p.view(torch.int16).fill_(int(np.int16(nan_bits.view(np.int16))))
            p.index_copy_(0, used, _bits_tensor(pages, cfg.kv_dtype).to(device))
            pools.append(p)
        k_scale = v_scale = None
    return DeviceCase(
        q=upload_q(case, device),
        k_pool=pools[0], v_pool=pools[1], k_scale=k_scale, v_scale=v_scale,
        block_tables=torch.from_numpy(case.block_tables).to(device),
        context_lens=torch.from_numpy(case.context_lens).to(device),
    )
