"""Seeded input generation for the decode workloads.

Recipe (numpy PCG64 ``default_rng(seed)``), in draw order:

1. context lengths -- fixed / ``integers(lo, hi + 1)`` /
   ``clip(rint(lognormal(ln median, sigma)), lo, hi)``;
2. ``perm = permutation(num_pages)``: the initial free-page list;
3. ``q ~ N(0, 1)`` as float32 ``[B][Hq][D]``;
4. for each sequence in order, K then V ~ N(0, 1) as float32 ``[n][Hkv][D]``.

Physical pages are handed out the way the free list of
"TensorRT-LLM 深度实战", section 3.1 hands them out: sequences in order
b = 0..B-1 each take ``ceil(n_b / page_size)`` pages, each page taken from the
END of the list.  A pool created with ``perm`` as its initial free list and
the same allocation order therefore reproduces these block tables exactly.

Storage encodings (the inputs both sides consume bit-for-bit):

* f16 / bf16: round-to-nearest-even from float32;
* int8 (symmetric, one scale per token per KV head):
  ``s = max(max_d |x_d|, 1e-5) / 127`` in float32 and
  ``x8 = clip(rint(x / s), -127, 127)``;
* fp8 (OCP E4M3, one scale per token per KV head):
  ``s = max(max_d |x_d|, 1e-5) / 448`` in float32 and ``x8 = e4m3(x / s)``,
  rounded to nearest even by torch's float8_e4m3fn cast (|x / s| <= 448, so
  nothing saturates).

This module draws and lays out inputs only; no attention arithmetic lives here.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .configs import Config

F16_NAN = np.uint16(0x7E00)
BF16_NAN = np.uint16(0x7FC0)
I8_POISON = np.int8(-128)
FP8_NAN = np.uint8(0x7F)


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> raw uint16 bits of f16 / bf16, round-to-nearest-even."""
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def quantize_fp8(x: np.ndarray):
    """Per-row OCP E4M3 encoding over the last axis: (codes uint8, scales fp32)."""
    import torch

    amax = np.max(np.abs(x), axis=-1)
    s = (np.maximum(amax, np.float32(1e-5)) / np.float32(448.0)).astype(np.float32)
    y = torch.from_numpy(np.ascontiguousarray(x / s[..., None], dtype=np.float32))
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, s


def quantize_int8(x: np.ndarray):
    """Symmetric per-row int8 encoding over the last axis (float32 math)."""
    amax = np.max(np.abs(x), axis=-1)
    s = (np.maximum(amax, np.float32(1e-5)) / np.float32(127.0)).astype(np.float32)
    q = np.rint(x / s[..., None])
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def draw_context_lens(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.lens_kind == "fixed":
        lens = np.asarray(cfg.lens_args, dtype=np.int64)
        assert lens.shape[0] == cfg.batch
    elif cfg.lens_kind == "uniform":
        lo, hi = cfg.lens_args
        lens = rng.integers(lo, hi + 1, size=cfg.batch)
    elif cfg.lens_kind == "lognormal":
        median, sigma, lo, hi = cfg.lens_args
        lens = np.rint(rng.lognormal(np.log(median), sigma, size=cfg.batch))
        lens = np.clip(lens, lo, hi)
    else:
        raise ValueError(cfg.lens_kind)
    return lens.astype(np.int32)


@dataclass
class Case:
    cfg: Config
    seed: int
    context_lens: np.ndarray            # int32 [B]
    free_order: np.ndarray              # int32 [num_pages], the initial free list
    block_tables: np.ndarray            # int32 [B][max_blocks], -1 past the end
    q_bits: np.ndarray                  # uint16 [B][Hq][D]
    used_pages: np.ndarray              # int32 [n_used] physical id of host row i
    page_index: np.ndarray              # int32 [num_pages] physical id -> host row, -1
    k_pages: np.ndarray                 # [n_used][Hkv][PS][D] uint16 bits or int8
    v_pages: np.ndarray
    k_scale: Optional[np.ndarray]       # float32 [n_used][Hkv][PS] (int8 only)
    v_scale: Optional[np.ndarray]
    scale: float                        # softmax scale, exactly representable in fp32
    poison: bool = False
    logical_k: Optional[List[np.ndarray]] = field(default=None, repr=False)
    logical_v: Optional[List[np.ndarray]] = field(default=None, repr=False)

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def bytes_alg(self) -> int:
        """Bytes the decode step must move per layer: valid K/V (+ scales),
        q in, out, the used block-table entries and the context lengths."""
        c = self.cfg
        e_kv = 1 if c.kv_dtype in ("i8", "fp8") else 2
        n = self.context_lens.astype(np.int64)
        kv = int(n.sum()) * c.num_kv_heads * c.head_dim * 2 * e_kv
        if c.kv_dtype in ("i8", "fp8"):
            kv += int(n.sum()) * c.num_kv_heads * 2 * 4
        qo = c.batch * c.num_q_heads * c.head_dim * (2 + 2)
        pages = -(-n // c.page_size)
        bt = int(pages.sum()) * 4 + c.batch * 4
        return kv + qo + bt


def make_case(cfg: Config, seed: Optional[int] = None, poison: bool = False,
              keep_logical: bool = False, context_lens=None) -> Case:
    """Draw one workload.  ``context_lens`` overrides step 1 (edge-case tests);
    the rest of the draw order is unchanged."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = draw_context_lens(cfg, rng)
    if context_lens is not None:
        lens = np.asarray(context_lens, dtype=np.int32)
        assert lens.shape == (cfg.batch,)
    assert (lens >= 0).all() and (lens <= cfg.max_context_len).all()
    perm = rng.permutation(cfg.num_pages).astype(np.int32)

    B, Hq, Hkv, D, PS = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    q_bits = _to_bits(q, cfg.q_dtype)
    del q

    n_pages = [-(-int(n) // PS) for n in lens]
    n_used = sum(n_pages)
    if n_used > cfg.num_pages:
        raise ValueError(f"workload needs {n_used} pages, pool has {cfg.num_pages}")
    stack = perm[::-1]                   # pop order of the free list
    block_tables = np.full((B, cfg.max_blocks), -1, dtype=np.int32)
    used_pages = stack[:n_used].astype(np.int32).copy()
    page_index = np.full(cfg.num_pages, -1, dtype=np.int32)
    page_index[used_pages] = np.arange(n_used, dtype=np.int32)

    is_i8 = cfg.kv_dtype == "i8"
    is_fp8 = cfg.kv_dtype == "fp8"
    shape = (n_used, Hkv, PS, D)
    if is_i8 or is_fp8:
        if is_i8:
            k_pages = np.full(shape, I8_POISON if poison else 0, dtype=np.int8)
            v_pages = np.full(shape, I8_POISON if poison else 0, dtype=np.int8)
        else:
            k_pages = np.full(shape, FP8_NAN if poison else 0, dtype=np.uint8)
            v_pages = np.full(shape, FP8_NAN if poison else 0, dtype=np.uint8)
        sfill = np.float32(np.nan) if poison else np.float32(0)
        k_scale = np.full(shape[:3], sfill, dtype=np.float32)
        v_scale = np.full(shape[:3], sfill, dtype=np.float32)
    else:
        fill = (F16_NAN if cfg.kv_dtype == "f16" else BF16_NAN) if poison else np.uint16(0)
        k_pages = np.full(shape, fill, dtype=np.uint16)
        v_pages = np.full(shape, fill, dtype=np.uint16)
        k_scale = v_scale = None

    logical_k, logical_v = ([], []) if keep_logical else (None, None)
    row = 0
    for b in range(B):
        n, npg = int(lens[b]), n_pages[b]
        block_tables[b, :npg] = used_pages[row:row + npg]
        kf = rng.standard_normal((n, Hkv, D), dtype=np.float32)
        vf = rng.standard_normal((n, Hkv, D), dtype=np.float32)
        for src, dst, sdst, keep in ((kf, k_pages, k_scale, logical_k),
                                     (vf, v_pages, v_scale, logical_v)):
            if is_i8:
                enc, sc = quantize_int8(src)
            elif is_fp8:
                enc, sc = quantize_fp8(src)
            else:
                enc, sc = _to_bits(src, cfg.kv_dtype), None
            if keep is not None:
                keep.append((enc, sc))
            # token t of sequence b -> host row (row + t // PS), slot t % PS
            t = np.arange(n)
            rows = row + t // PS
            slots = t % PS
            dst[rows, :, slots, :] = enc
            if sc is not None:
                sdst[rows, :, slots] = sc
        row += npg
        del kf, vf

    return Case(cfg=cfg, seed=seed, context_lens=lens, free_order=perm,
                block_tables=block_tables, q_bits=q_bits, used_pages=used_pages,
                page_index=page_index, k_pages=k_pages, v_pages=v_pages,
                k_scale=k_scale, v_scale=v_scale,
                scale=float(np.float32(cfg.scale)), poison=poison,
                logical_k=logical_k, logical_v=logical_v)


def logical_kv(case: Case, b: int):
    """The stored (encoded) K and V of sequence ``b`` in logical token order:
    ``((k_enc, k_scale|None), (v_enc, v_scale|None))`` with shapes
    ``[n][Hkv][D]`` and ``[n][Hkv]``.  Requires ``keep_logical=True``."""
    if case.logical_k is None:
        raise ValueError("case was made without keep_logical=True")
    return case.logical_k[b], case.logical_v[b]


def repermute(case: Case, seed: int) -> Case:
    """The same workload with every used physical page moved to a new random
    physical id: page contents move with it and the block tables are rewritten.
    Attention outputs must not change."""
    rng = np.random.default_rng(seed)
    new_ids = rng.permutation(case.cfg.num_pages).astype(np.int32)
    mapping = new_ids  # old physical id p -> new physical id mapping[p]
    bt = case.block_tables.copy()
    valid = bt >= 0
    bt[valid] = mapping[bt[valid]]
    used = mapping[case.used_pages]
    page_index = np.full(case.cfg.num_pages, -1, dtype=np.int32)
    page_index[used] = np.arange(used.shape[0], dtype=np.int32)
    out = Case(**{**case.__dict__})
    out.block_tables = bt
    out.used_pages = used.astype(np.int32)
    out.page_index = page_index
    return out
