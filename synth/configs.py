"""The five decode workloads.

Shapes stand in for the models the pages use as examples; nothing here is a
real model or dataset.

* ``tiny``            -- GQA 2:1, head_dim 64, fp16, 16-token pages, lengths
                         {37, 100}, 32-page pool.
* ``llama2_7b_mha``   -- Llama-2-7B attention shape (32 q = 32 KV heads,
                         head_dim 128), bf16, 64-token pages, batch 32, lengths
                         uniform in [128, 2048], 16k-page pool.
* ``llama3_8b_gqa``   -- Llama-3-8B attention shape (32 q / 8 KV heads, the
                         GQA sharing of "TensorRT-LLM加速大模型推理实战"), bf16,
                         64-token pages (the TensorRT-LLM default block size,
                         "TensorRT-LLM 推理加速实战", section 8), batch 64,
                         lengths uniform in [512, 4096].
* ``long_128k``       -- GQA 32/8, head_dim 128, bf16, 64-token pages, batch 4,
                         131072 tokens each (">128k tokens" of
                         "TensorRT-LLM 核心架构解析", section 1.2).
* ``qwen_1p8b_int8``  -- Qwen-1.8B attention shape (16 = 16 heads, head_dim
                         128), fp16 q, int8 K/V with one fp32 scale per token
                         per KV head, 16-token pages (the vLLM block size the
                         same section 8 compares against), 256 sequences with
                         lognormal lengths (median 512, clipped to [1, 4096]).
* ``llama3_8b_gqa_fp8`` -- the Llama-3-8B GQA workload with its K/V stored as
                         FP8 E4M3 with one fp32 scale per token per KV head
                         (the FP8 KV cache of "TensorRT-LLM 推理加速实战",
                         section 8).

Where the workload statement leaves a value open (pool sizes of the last three
configs, the lognormal sigma, the softmax scale) the plainest reading is used:
pools of 16384 / 16384 / 32768 pages, sigma = 1.0, scale = 1/sqrt(head_dim).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str          # "f16" | "bf16"
    kv_dtype: str         # "f16" | "bf16" | "i8" | "fp8" (OCP E4M3)
    page_size: int
    num_pages: int
    seed: int
    lens_kind: str        # "fixed" | "uniform" | "lognormal"
    lens_args: Tuple      # fixed: the lengths; uniform: (lo, hi) inclusive;
                          # lognormal: (median, sigma, lo, hi)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_context_len(self) -> int:
        if self.lens_kind == "fixed":
            return max(self.lens_args)
        if self.lens_kind == "uniform":
            return self.lens_args[1]
        return self.lens_args[3]

    @property
    def max_blocks(self) -> int:
        return -(-self.max_context_len // self.page_size)


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config("tiny", 2, 4, 2, 64, "f16", "f16", 16, 32, 2661,
               "fixed", (37, 100)),
        Config("llama2_7b_mha", 32, 32, 32, 128, "bf16", "bf16", 64, 16384, 2662,
               "uniform", (128, 2048)),
        Config("llama3_8b_gqa", 64, 32, 8, 128, "bf16", "bf16", 64, 16384, 2663,
               "uniform", (512, 4096)),
        Config("long_128k", 4, 32, 8, 128, "bf16", "bf16", 64, 16384, 2664,
               "fixed", (131072, 131072, 131072, 131072)),
        Config("qwen_1p8b_int8", 256, 16, 16, 128, "f16", "i8", 16, 32768, 2665,
               "lognormal", (512, 1.0, 1, 4096)),
        # the GQA workload with an FP8 (E4M3) KV cache
        Config("llama3_8b_gqa_fp8", 64, 32, 8, 128, "bf16", "fp8", 64, 16384, 2666,
               "uniform", (512, 4096)),
    ]
}

# Order used by the parity suite and documentation.
ORDER = ["tiny", "llama2_7b_mha", "llama3_8b_gqa", "long_128k", "qwen_1p8b_int8"]


def get_config(name: str, **overrides) -> Config:
    base = CONFIGS[name]
    if not overrides:
        return base
    fields = dict(base.__dict__)
    fields.update(overrides)
    return Config(**fields)
