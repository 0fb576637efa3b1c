"""Pure-Python contiguous attention, for tiny inputs only.

TEST INFRASTRUCTURE (see the package docstring).  No pages, no block table,
no numpy arithmetic: the textbook definition from the fused attention kernel
of "TensorRT-LLM 深度实战", section 3.3 -- scores = scale * q.k, subtract the
max, exponentiate, normalise, weight V -- written with Python floats (fp64)
and ``math.exp``.
"""

from __future__ import annotations

import math
from typing import List, Sequence


def attention(q: Sequence[float], keys: Sequence[Sequence[float]],
              values: Sequence[Sequence[float]], scale: float) -> List[float]:
    n = len(keys)
    D = len(q)
    if n == 0:
        return [0.0] * D
    s = []
    for k in keys:
        dot = 0.0
        for d in range(D):
            dot += q[d] * k[d]
        s.append(scale * dot)
    M = max(s)
    w = [math.exp(x - M) for x in s]
    Z = 0.0
    for x in w:
        Z += x
    out = []
    for d in range(D):
        acc = 0.0
        for t in range(n):
            acc += w[t] * values[t][d]
        out.append(acc / Z)
    return out


def decode_batch(q, keys, values, scale, group: int):
    """q: [B][Hq][D]; keys/values: per sequence [n][Hkv][D] (nested lists of
    floats).  Query head h reads KV head h // group."""
    out = []
    for b in range(len(q)):
        per_head = []
        for h in range(len(q[b])):
            g = h // group
            ks = [tok[g] for tok in keys[b]]
            vs = [tok[g] for tok in values[b]]
            per_head.append(attention(q[b][h], ks, vs, scale))
        out.append(per_head)
    return out
