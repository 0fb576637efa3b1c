"""Pins of the allocator model and the KV-size formula (CPU only).

The model is fixed to: a trace worked out by hand from the free-list rules of
"TensorRT-LLM 深度实战", section 3.1 (pop from the end, push on release);
the closed form ceil(n / page_size) computed with exact rationals; invariants
that hold after any sequence of operations; and the numbers the pages print
for the KV-cache size formula.
"""

import math
import os
from fractions import Fraction

import pytest
from hypothesis import given, settings, strategies as st

from oracle.kvsize import kv_bytes, kv_bytes_per_token
from oracle.pool_model import (OutOfPages, PagePoolModel, SequenceExists, SharedLastPage,
                               UnknownSequence, pages_needed)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = float(v) if "." in v else int(v)
    return vals


def test_hand_worked_trace():
    # 6 pages of 4 tokens; free list [0, 1, 2, 3, 4, 5], popped from the end.
    m = PagePoolModel(page_size=4, num_pages=6)
    assert m.allocate(10, 9) == [5 * 4 + 0, 5 * 4 + 1, 5 * 4 + 2, 5 * 4 + 3,
                                 4 * 4 + 0, 4 * 4 + 1, 4 * 4 + 2, 4 * 4 + 3, 3 * 4 + 0]
    assert m.page_table[10] == [5, 4, 3]
    assert m.allocate(11, 4) == [8, 9, 10, 11]          # page 2
    # 9 tokens use 3 pages of capacity 12: appending 3 fits, a 4th needs page 1
    assert m.append_tokens(10, 3) == [13, 14, 15]
    assert m.page_table[10] == [5, 4, 3]
    assert m.append_tokens(10, 1) == [1 * 4 + 0]
    assert m.page_table[10] == [5, 4, 3, 1]
    assert m.free_pages == [0]
    with pytest.raises(OutOfPages):
        m.allocate(12, 5)                                # needs 2 pages, 1 free
    assert m.free_pages == [0] and 12 not in m.page_table
    m.release(10)                                        # pushed back in page order
    assert m.free_pages == [0, 5, 4, 3, 1]
    assert m.allocate(12, 5) == [4, 5, 6, 7, 12]         # pages 1 then 3
    with pytest.raises(SequenceExists):
        m.allocate(12, 1)
    with pytest.raises(UnknownSequence):
        m.release(99)
    with pytest.raises(UnknownSequence):
        m.append_tokens(99, 1)


def test_append_oom_leaves_state_unchanged():
    m = PagePoolModel(page_size=16, num_pages=3)
    m.allocate(0, 16)
    before = (list(m.free_pages), {k: list(v) for k, v in m.page_table.items()}, dict(m.token_count))
    with pytest.raises(OutOfPages):
        m.append_tokens(0, 33)                           # needs 3 more pages, 2 free
    assert (m.free_pages, m.page_table, m.token_count) == before


@given(st.integers(0, 10 ** 6), st.integers(1, 4096))
def test_pages_needed_is_exact_ceiling(n, ps):
    assert pages_needed(n, ps) == math.ceil(Fraction(n, ps))


ops = st.lists(st.tuples(st.sampled_from(["alloc", "append", "release"]),
                         st.integers(0, 7), st.integers(0, 70)), max_size=60)


@settings(max_examples=300, deadline=None)
@given(st.sampled_from([1, 4, 16]), st.integers(1, 24), st.randoms(use_true_random=False), ops)
def test_invariants_hold_after_any_operation_sequence(ps, num_pages, rnd, seq):
    order = list(range(num_pages))
    rnd.shuffle(order)
    m = PagePoolModel(ps, num_pages, initial_free_order=order)
    for op, sid, n in seq:
        free_before = list(m.free_pages)
        try:
            if op == "alloc":
                m.allocate(sid, n)
                # taken from the end of the free list, in pop order
                k = len(m.page_table[sid])
                assert m.page_table[sid] == free_before[::-1][:k]
            elif op == "append":
                had = list(m.page_table.get(sid, []))
                m.append_tokens(sid, n)
                new = m.page_table[sid][len(had):]
                assert new == free_before[::-1][:len(new)]
            else:
                pages = list(m.page_table.get(sid, []))
                m.release(sid)
                assert m.free_pages == free_before + pages
        except (OutOfPages, SequenceExists, UnknownSequence):
            assert m.free_pages == free_before
        owned = [p for pages in m.page_table.values() for p in pages]
        # conservation and unique ownership
        assert sorted(owned + m.free_pages) == list(range(num_pages))
        for s, pages in m.page_table.items():
            assert len(pages) == math.ceil(Fraction(m.token_count[s], ps))


def test_block_tables_and_slots():
    m = PagePoolModel(page_size=16, num_pages=8, initial_free_order=[3, 1, 7, 0, 2, 6, 5, 4])
    m.allocate(1, 20)
    m.allocate(2, 1)
    bt, lens = m.block_tables([2, 1], max_blocks=3)
    assert bt.tolist() == [[6, -1, -1], [4, 5, -1]]
    assert lens.tolist() == [1, 20]


# --------------------------------------------------------------------------
# KV-size formula against the numbers printed on the pages.

def test_kv_bytes_worked_example():
    g = read_golden("kv_size_llama31_70b.txt")
    L, H, D = g["layers"], g["kv_heads"], g["head_dim"]
    assert kv_bytes_per_token(L, H, D, 16) == g["fp16_bytes_per_token"]
    assert kv_bytes_per_token(L, H, D, 8) == g["fp8_bytes_per_token"]
    for bits, approx in ((16, g["fp16_tokens_approx"]), (8, g["fp8_tokens_approx"])):
        tokens = g["kv_budget_bytes"] / kv_bytes_per_token(L, H, D, bits)
        assert abs(tokens - approx) / approx < 0.10


def test_kv_bytes_formula_is_linear_in_every_factor():
    base = kv_bytes(2, 8, 128, 100, 3, 16)
    assert base == 2 * 2 * 8 * 128 * 100 * 3 * 2
    assert kv_bytes(4, 8, 128, 100, 3, 16) == 2 * base
    assert kv_bytes(2, 8, 128, 100, 3, 4) == base // 4      # INT4: half a byte
    with pytest.raises(ValueError):
        kv_bytes(1, 1, 1, 1, 1, 3)                           # 6 bits in total


def test_prealloc_waste_figure():
    g = read_golden("prealloc_waste.txt")
    used = kv_bytes(1, 8, 128, g["avg_len"], 1, 16)
    reserved = kv_bytes(1, 8, 128, g["max_seq_len"], 1, 16)
    assert 100.0 * (1 - Fraction(used, reserved)) == Fraction(g["waste_percent"]).limit_denominator()


def test_gqa_saving_figure():
    g = read_golden("gqa_saving.txt")
    mha = kv_bytes(32, g["num_q_heads"], 128, 4096, 1, 16)
    gqa = kv_bytes(32, g["num_kv_heads"], 128, 4096, 1, 16)
    assert 100 * (1 - Fraction(gqa, mha)) == g["saving_percent"]


def test_long_context_config_is_about_2p1_gb_per_layer():
    # batch 4 x 131072 tokens, 8 KV heads, head_dim 128, bf16, one layer
    assert kv_bytes(1, 8, 128, 131072, 4, 16) == 2_147_483_648


# --------------------------------------------------------------------------
# Block reuse: shared pages, owner counts, copy-on-write of a partly filled
# shared last page.

def test_fork_and_copy_on_write_trace():

    m = PagePoolModel(16, 6)                      # free list [0..5], pop from the end
    assert m.allocate(0, 20)[:2] == [5 * 16, 5 * 16 + 1]
    assert m.page_table[0] == [5, 4]
    m.fork(0, 1)
    assert m.page_table[1] == [5, 4] and m.refcount == {5: 2, 4: 2}
    # the last page holds 4 of 16 tokens and is shared: the plain append refuses
    with pytest.raises(SharedLastPage):
        m.append_tokens(1, 1)
    slots, copy = m.append_tokens_cow(1, 1)
    assert copy == (4, 3)                          # page 4 copied to the next free page, 3
    assert m.page_table[1] == [5, 3] and slots == [3 * 16 + 4]
    assert m.refcount == {5: 2, 4: 1, 3: 1}
    # the parent is now the last page's only owner: it writes in place
    assert m.append_tokens_cow(0, 1) == ([4 * 16 + 4], None)
    # 12 more tokens fill page 3 exactly; the next append needs a new page, no copy
    m.append_tokens_cow(1, 11)
    assert m.token_count[1] == 32
    m.fork(1, 2)
    assert m.append_tokens_cow(2, 1) == ([2 * 16], None)   # full shared last page: no copy
    assert m.page_table[2] == [5, 3, 2]
    assert m.free_pages == [0, 1]
    m.release(0)
    assert m.free_pages == [0, 1, 4]               # page 5 still owned by 1 and 2
    m.release(1)
    assert m.free_pages == [0, 1, 4]               # pages 5 and 3 still owned by 2
    m.release(2)
    assert m.free_pages == [0, 1, 4, 5, 3, 2]
    assert m.refcount == {}


def test_copy_page_is_taken_before_overflow_pages():
    """An append that both copies a shared, partly filled last page and
    overflows: the copy gets the first page popped, the overflow the next."""
    m = PagePoolModel(4, 10)                      # pops 9, 8, 7, ...
    m.allocate(0, 6)                              # pages [9, 8], 2 tokens in page 8
    m.fork(0, 1)
    slots, copy = m.append_tokens_cow(1, 5)       # tokens 6..10
    assert copy == (8, 7)
    assert m.page_table[1] == [9, 7, 6] and m.page_table[0] == [9, 8]
    assert slots == [7 * 4 + 2, 7 * 4 + 3, 6 * 4 + 0, 6 * 4 + 1, 6 * 4 + 2]
    assert m.refcount == {9: 2, 8: 1, 7: 1, 6: 1}


def test_copy_on_write_is_all_or_nothing():
    m = PagePoolModel(4, 3)
    m.allocate(0, 6)                               # pages [2, 1], one free
    m.fork(0, 1)
    with pytest.raises(OutOfPages):
        m.append_tokens_cow(1, 3)                  # copy (1 page) + overflow (1 page) > 1 free
    assert m.page_table[1] == [2, 1] and m.free_pages == [0] and m.refcount == {2: 2, 1: 2}


fork_ops = st.lists(st.tuples(st.sampled_from(["alloc", "append", "append_cow", "release", "fork"]),
                              st.integers(0, 4), st.integers(0, 40), st.integers(0, 4)),
                    max_size=50)


@settings(max_examples=300, deadline=None)
@given(st.sampled_from([1, 4, 16]), st.integers(1, 24), fork_ops)
def test_owner_counts_hold_after_any_operation_sequence(ps, num_pages, seq):

    m = PagePoolModel(ps, num_pages)
    for op, sid, n, other in seq:
        before = (list(m.free_pages), {k: list(v) for k, v in m.page_table.items()}, dict(m.refcount))
        try:
            if op == "alloc":
                m.allocate(sid, n)
            elif op == "append":
                m.append_tokens(sid, n)
            elif op == "append_cow":
                last_shared = (sid in m.page_table and m.token_count[sid] % ps != 0 and n > 0
                               and m.refcount[m.page_table[sid][-1]] > 1)
                old_last = m.page_table[sid][-1] if sid in m.page_table and m.page_table[sid] else None
                _, copy = m.append_tokens_cow(sid, n)
                assert (copy is not None) == last_shared
                if copy is not None:
                    assert copy[0] == old_last and copy[1] == before[0][-1]   # next free page
            elif op == "fork":
                m.fork(other, sid)
            else:
                m.release(sid)
        except (OutOfPages, SequenceExists, UnknownSequence, SharedLastPage):
            assert (m.free_pages, m.page_table, m.refcount) == before
        owners = {}
        for pages in m.page_table.values():
            assert len(set(pages)) == len(pages)
            for p in pages:
                owners[p] = owners.get(p, 0) + 1
        assert owners == m.refcount
        assert sorted(list(owners) + m.free_pages) == list(range(num_pages))
        for s, pages in m.page_table.items():
            assert len(pages) == math.ceil(Fraction(m.token_count[s], ps))
