"""Pins of the oracle's chunked-prefill attention (oracle_paged_prefill)
against facts that do not come from it: pure-Python causal attention on tiny
inputs, the decode oracle for a chunk's last query, causality, a sequence's
first token, and the position of a query independent of its chunk."""

import dataclasses

import numpy as np
import pytest

import oracle
from oracle import brute
from test_oracle_pins import TINY_SHAPES, decode_bits, logical_floats, tiny_case


def queries(case, chunks, seed=5):
    """q bits [sum(chunks)][Hq][D] in the case's q type, and q_start."""
    from synth.make import _to_bits

    c = case.cfg
    rng = np.random.default_rng(seed)
    n_q = int(sum(chunks))
    q = rng.standard_normal((n_q, c.num_q_heads, c.head_dim)).astype(np.float32)
    return _to_bits(q, c.q_dtype), np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)


def chunks_of(case):
    """A chunk length per sequence: all of a short one, part of a long one."""
    return [int(n) if n <= 20 else int(n) // 3 + 1 for n in case.context_lens]


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_prefill_matches_pure_python_causal_attention(shape):
    case = tiny_case(*shape)
    c = case.cfg
    ch = chunks_of(case)
    qb, qs = queries(case, ch)
    got = oracle.paged_prefill(case, qb, qs)
    qf = decode_bits(qb, c.q_dtype)
    for b in range(c.batch):
        n = int(case.context_lens[b])
        keys = logical_floats(case, b, "k")
        vals = logical_floats(case, b, "v")
        for i in range(ch[b]):
            pos = n - ch[b] + i
            row = qs[b] + i
            for h in range(c.num_q_heads):
                g = h // c.group
                ref = brute.attention(qf[row, h].tolist(), keys[:pos + 1, g].tolist(),
                                      vals[:pos + 1, g].tolist(), case.scale)
                np.testing.assert_allclose(got[row, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", TINY_SHAPES[:4])
def test_last_query_of_a_chunk_is_a_decode_step(shape):
    case = tiny_case(*shape)
    ch = chunks_of(case)
    qb, qs = queries(case, ch)
    got = oracle.paged_prefill(case, qb, qs)
    last = np.stack([qb[qs[b + 1] - 1] for b in range(case.cfg.batch)])
    dec = oracle.paged_decode(case, q_bits=last)
    for b in range(case.cfg.batch):
        np.testing.assert_allclose(got[qs[b + 1] - 1], dec[b], rtol=0, atol=1e-13)


def test_causality_later_keys_do_not_matter():
    """Changing K and V at positions after a query leaves its output as it was."""
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (40, 33))
    ch = [12, 33]
    qb, qs = queries(case, ch)
    base = oracle.paged_prefill(case, qb, qs)
    k = case.k_pages.copy()
    v = case.v_pages.copy()
    # overwrite token 39 of sequence 0 (its last), and tokens 20..32 of sequence 1
    rng = np.random.default_rng(3)
    def poke(b, t):
        row = case.page_index[case.block_tables[b, t // 16]]
        k[row, :, t % 16] = rng.integers(0, 0x3C00, size=k.shape[-2:][1:], dtype=np.uint16)
        v[row, :, t % 16] = rng.integers(0, 0x3C00, size=v.shape[-2:][1:], dtype=np.uint16)
    poke(0, 39)
    for t in range(20, 33):
        poke(1, t)
    moved = dataclasses.replace(case, k_pages=k, v_pages=v)
    got = oracle.paged_prefill(moved, qb, qs)
    # sequence 0: queries at positions 28..39; only position 39 sees token 39
    assert (got[qs[0]:qs[1] - 1] == base[qs[0]:qs[1] - 1]).all()
    assert not (got[qs[1] - 1] == base[qs[1] - 1]).all()
    # sequence 1: queries at positions 0..32; those before 20 are unchanged
    assert (got[qs[1]:qs[1] + 20] == base[qs[1]:qs[1] + 20]).all()
    assert not (got[qs[1] + 20:] == base[qs[1] + 20:]).all()


def test_first_token_of_a_sequence_returns_its_value():
    """A chunk holding a whole sequence: query 0 sees only key 0, so its
    output is V[0] whatever q is."""
    case = tiny_case(2, 1, 64, "bf16", "bf16", 16, (9, 30))
    qb, qs = queries(case, [9, 30])
    got = oracle.paged_prefill(case, qb, qs)
    for b in range(2):
        v0 = logical_floats(case, b, "v")[0, 0]
        for h in range(2):
            assert (got[qs[b], h] == v0).all()


def test_a_query_depends_on_its_position_not_on_its_chunk():
    """The same query vector at the same position gives the same output
    whether its chunk is long or short (the context length counts the whole
    chunk, so the position of row i is n - chunk + i)."""
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (50, 50))
    qb, qs = queries(case, [20, 5])
    got = oracle.paged_prefill(case, qb, qs)
    # sequence 0's row 15 sits at position 50 - 20 + 15 = 45; sequence 1's
    # row 0 at 50 - 5 + 0 = 45: give both the same query vector
    qb2 = qb.copy()
    qb2[qs[1]] = qb[qs[0] + 15]
    both = dataclasses.replace(case, block_tables=np.stack([case.block_tables[0]] * 2),
                               context_lens=np.array([50, 50], dtype=np.int32))
    got2 = oracle.paged_prefill(both, qb2, qs)
    assert (got2[qs[1]] == got2[qs[0] + 15]).all()


def test_chunk_longer_than_context_is_rejected():
    case = tiny_case(4, 2, 64, "f16", "f16", 16, (10, 20))
    qb, qs = queries(case, [11, 3])
    with pytest.raises(oracle.OracleError):
        oracle.paged_prefill(case, qb, qs)
