"""KV-cache size formula.

TEST INFRASTRUCTURE (see the package docstring).

"TensorRT-LLM 推理加速实战", section 8.1, gives the per-token size as
2 x layers x kv_heads x head_dim x element bytes (the 2 is K and V); the
aiqz.cc TensorRT-LLM explainer, section "KV缓存管理", gives the whole cache as
M_kv = 2 x n_layers x n_heads x d_head x n_tokens x b x bytes, with 2 bytes
for FP16, 1 for FP8 and half a byte for INT4.  Element sizes are taken here in
bits so that INT4 stays an integer computation.
"""

from __future__ import annotations


def kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, batch: int,
             elem_bits: int) -> int:
    bits = 2 * layers * kv_heads * head_dim * tokens * batch * elem_bits
    if bits % 8:
        raise ValueError("size is not a whole number of bytes")
    return bits // 8


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bits: int) -> int:
    return kv_bytes(layers, kv_heads, head_dim, 1, 1, elem_bits)
