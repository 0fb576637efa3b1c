"""GPU parity of the chunked-prefill kernel (needs a gfx950 GPU).

Each sequence's last nq tokens are the chunk: their K/V are in the paged
cache (the generator's layout), their queries are new rows, and each query
attends causally.  Every output row is compared with the fp64 oracle's
chunked prefill; the large case compares the first and last rows of every
chunk (the oracle, which recomputes each row from scratch, would take
minutes for all of them), exploiting that a row depends only on keys up to
its position."""

import dataclasses
import itertools

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, note, small_config, to_f64
from synth import make_case
from synth.device import torch_dtype, upload
from synth.make import _to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_266_amd as pkv

    pkv.lib()
    yield


def queries(cfg, chunks, seed):
    rng = np.random.default_rng(seed)
    n_q = int(sum(chunks))
    q = rng.standard_normal((n_q, cfg.num_q_heads, cfg.head_dim)).astype(np.float32)
    return _to_bits(q, cfg.q_dtype), np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)


def gpu_prefill(case, q_bits, q_start, dev=None, max_q_len=None, context_lens=None):
    import torch

    import paged_kv_cache_266_amd as pkv

    cfg = case.cfg
    dev = dev or upload(case, "cuda")
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch_dtype(cfg.q_dtype)).cuda()
    qs = torch.from_numpy(q_start).cuda()
    ctx = dev.context_lens if context_lens is None else torch.from_numpy(context_lens).cuda()
    mq = int(np.diff(q_start).max()) if max_q_len is None else max_q_len
    out = pkv.paged_prefill(q, dev.k_pool, dev.v_pool, dev.block_tables, qs, ctx, case.scale,
                            max_context_len=cfg.max_context_len, max_q_len=max(mq, 1),
                            k_scale=dev.k_scale, v_scale=dev.v_scale)
    torch.cuda.synchronize()
    return to_f64(out)


def check(case, got, ref, label):
    err = np.abs(got - ref)
    tol = TOL[case.cfg.kv_dtype]
    note(f"  {label}: max|err| {err.max():.3e} (tol {tol})")
    assert np.isfinite(got).all(), label
    assert err.max() <= tol, f"{label}: {err.max()} > {tol}"


LENS = (1, 63, 64, 65, 300, 777)
CHUNKS = (1, 63, 20, 65, 100, 130)


@pytest.mark.parametrize("D,PS,G,qd,kvd", [(d, ps, g, qd, kvd)
                                           for d, ps, g, qd in itertools.product((64, 128), (16, 64), (1, 2, 4, 8),
                                                                                 ("f16", "bf16"))
                                           for kvd in (qd, "i8", "fp8")])
def test_prefill_every_instantiation(D, PS, G, qd, kvd):
    """Ragged chunks: a whole 1-token sequence, a whole 63-token one, parts
    of longer ones, chunks spanning several query blocks (256/G tokens each)
    and key tiles; head_dim 64 and 128; 16-bit, int8 and E4M3 caches."""
    Hkv = 2
    cfg = small_config(G * Hkv, Hkv, D, qd, kvd, PS, LENS)
    note(f"[prefill] D={D} PS={PS} G={G} q={qd} kv={kvd}")
    case = make_case(cfg, seed=300 + PS + G + D)
    qb, qs = queries(cfg, CHUNKS, seed=PS + G)
    got = gpu_prefill(case, qb, qs)
    ref = oracle.paged_prefill(case, qb, qs)
    check(case, got, ref, "all rows")


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 1.0, 4.0])
def test_prefill_scales(scale):
    """A negative scale, a zero scale (uniform weights over the visible keys),
    and scales large enough that rows' running maxima rise by many powers of
    two after the first key tile, so the kernel's deferred rescaling runs
    mid-sequence."""
    cfg = small_config(8, 2, 128, "f16", "f16", 64, (300, 777, 1000))
    case = dataclasses.replace(make_case(cfg, seed=21), scale=scale)
    qb, qs = queries(cfg, (100, 200, 130), seed=22)
    note(f"[prefill scale] {scale}")
    got = gpu_prefill(case, qb, qs)
    ref = oracle.paged_prefill(case, qb, qs)
    check(case, got, ref, f"scale {scale}")


def test_prefill_empty_chunks_and_invalid_lengths():
    """A sequence with no new tokens is skipped; a context length shorter
    than the chunk gives NaN rows for that sequence only."""
    cfg = small_config(8, 2, 128, "bf16", "bf16", 16, (40, 90, 33))
    case = make_case(cfg, seed=5)
    qb, qs = queries(cfg, (0, 30, 10), seed=2)
    got = gpu_prefill(case, qb, qs)
    ref = oracle.paged_prefill(case, qb, qs)
    check(case, got, ref, "empty chunk")
    bad_ctx = case.context_lens.copy()
    bad_ctx[2] = 5                                  # shorter than its 10-token chunk
    got = gpu_prefill(case, qb, qs, context_lens=bad_ctx)
    assert np.isnan(got[qs[2]:qs[3]]).all()
    assert np.abs(got[qs[1]:qs[2]] - ref[qs[1]:qs[2]]).max() <= TOL["bf16"]


def test_prefill_out_of_pool_page_gives_nan_rows():
    cfg = small_config(8, 2, 128, "f16", "f16", 16, (100, 100))
    case = make_case(cfg, seed=6)
    qb, qs = queries(cfg, (40, 40), seed=3)
    ref = oracle.paged_prefill(case, qb, qs)
    bt = case.block_tables.copy()
    bt[1, 2] = cfg.num_pages + 3                    # keys 32..47 of sequence 1
    got = gpu_prefill(dataclasses.replace(case, block_tables=bt), qb, qs)
    assert np.isnan(got[qs[1]:qs[2]]).all()
    check(case, got[qs[0]:qs[1]], ref[qs[0]:qs[1]], "other sequence")


@pytest.mark.parametrize("G,qd,kvd", [(4, "bf16", "bf16"), (1, "f16", "f16"), (4, "bf16", "fp8"), (1, "f16", "i8")])
def test_prefill_large_chunks_sampled_rows(G, qd, kvd):
    """16 sequences with 512-token chunks after contexts of up to 3.5k tokens
    (the chunked-context step of a long prompt): the first and last 8 rows of
    every chunk against the oracle, computed as 8-row chunks at the same
    positions."""
    rng = np.random.default_rng(11)
    chunk = 512
    lens = tuple(int(x) for x in rng.integers(chunk, 4097, size=16))
    Hkv = 8 if G == 4 else 16
    cfg = small_config(G * Hkv, Hkv, 128, qd, kvd, 64, lens)
    case = make_case(cfg, seed=12)
    qb, qs = queries(cfg, (chunk,) * len(lens), seed=13)
    note(f"[prefill large] G={G} q={qd} kv={kvd} chunks 16 x {chunk}")
    got = gpu_prefill(case, qb, qs)
    last = np.concatenate([qb[qs[b + 1] - 8:qs[b + 1]] for b in range(len(lens))])
    qs8 = np.arange(0, 8 * len(lens) + 1, 8, dtype=np.int32)
    ref_last = oracle.paged_prefill(case, last, qs8)
    got_last = np.concatenate([got[qs[b + 1] - 8:qs[b + 1]] for b in range(len(lens))])
    check(case, got_last, ref_last, "last 8 rows")
    first = np.concatenate([qb[qs[b]:qs[b] + 8] for b in range(len(lens))])
    early = dataclasses.replace(case, context_lens=(case.context_lens - (chunk - 8)).astype(np.int32))
    ref_first = oracle.paged_prefill(early, first, qs8)
    got_first = np.concatenate([got[qs[b]:qs[b] + 8] for b in range(len(lens))])
    check(case, got_first, ref_first, "first 8 rows")


def test_prefill_random_sweep_against_oracle():
    """A seeded random sweep: head_dim, page size, group, dtype pair, KV
    heads, ragged context lengths (page and tile boundaries among them) and
    chunks (whole sequences, single tokens, parts), every row compared with
    the oracle; stops at the first mismatch, naming the case."""
    rng = np.random.default_rng(2028)
    for i in range(40):
        D = int(rng.choice([64, 128]))
        PS = int(rng.choice([16, 64]))
        G = int(rng.choice([1, 2, 4, 8]))
        qd = ["f16", "bf16"][int(rng.integers(2))]
        kvd = [qd, "i8", "fp8"][int(rng.integers(3))]
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 7))
        lens = [int(rng.choice([1, 2, PS - 1, PS, PS + 1, 64, 65, 129])) if rng.random() < 0.3
                else int(rng.integers(1, 1200)) for _ in range(B)]
        chunks = [n if rng.random() < 0.2 else int(rng.integers(1, min(n, 300) + 1)) for n in lens]
        note(f"[prefill sweep {i}] D={D} PS={PS} G={G} q={qd} kv={kvd} Hkv={Hkv} lens={lens} chunks={chunks}")
        cfg = small_config(G * Hkv, Hkv, D, qd, kvd, PS, tuple(lens))
        case = make_case(cfg, seed=4000 + i)
        qb, qs = queries(cfg, chunks, seed=i)
        check(case, gpu_prefill(case, qb, qs), oracle.paged_prefill(case, qb, qs), f"prefill sweep {i}")


@pytest.mark.parametrize("n,PS,kvd,G", [(262144, 64, "bf16", 4), (131077, 16, "i8", 1), (262144, 64, "fp8", 4)])
def test_prefill_chunk_after_a_very_long_context(n, PS, kvd, G):
    """A 512-token chunk at the end of a context of 131k or 262k tokens (and
    one short sequence): the first and last 8 rows of each chunk against the
    oracle, computed as 8-row chunks at the same positions."""
    chunk = 512
    lens = (n, 700)
    Hkv = 8 if G == 4 else 16
    cfg = small_config(G * Hkv, Hkv, 128, "bf16", kvd, PS, lens, num_pages=sum(-(-x // PS) for x in lens) + 40)
    note(f"[prefill long context] n={n} PS={PS} kv={kvd} G={G}")
    case = make_case(cfg, seed=21)
    qb, qs = queries(cfg, (chunk, chunk), seed=22)
    got = gpu_prefill(case, qb, qs)
    qs8 = np.arange(0, 8 * len(lens) + 1, 8, dtype=np.int32)
    last = np.concatenate([qb[qs[b + 1] - 8:qs[b + 1]] for b in range(len(lens))])
    check(case, np.concatenate([got[qs[b + 1] - 8:qs[b + 1]] for b in range(len(lens))]),
          oracle.paged_prefill(case, last, qs8), "last 8 rows")
    first = np.concatenate([qb[qs[b]:qs[b] + 8] for b in range(len(lens))])
    early = dataclasses.replace(case, context_lens=(case.context_lens - (chunk - 8)).astype(np.int32))
    check(case, np.concatenate([got[qs[b]:qs[b] + 8] for b in range(len(lens))]),
          oracle.paged_prefill(early, first, qs8), "first 8 rows")
