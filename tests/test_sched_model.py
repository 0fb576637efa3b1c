"""Pins of the continuous-batching scheduler model (oracle/sched_model.py).

The worked example is the request simulator of the aiqz.cc TensorRT-LLM
explainer ("Python 演示"): three requests arriving at steps 0, 1, 2 that
need 10, 2 and 2 decode steps.  Traced by hand from that page's loop:

* continuous: step 0 runs {0}; step 1 {0, 1}; step 2 {0, 1, 2} (1 finishes,
  waited 2 - 1 = 1); step 3 {0, 2} (2 finishes, 3 - 2 = 1); steps 4..9 {0}
  (0 finishes at 9, waited 9).  The clock ends at 10, the waits sum to 11.
* static: {0} runs alone for steps 0..9 (finishes at 9, waited 9); only
  then are 1 and 2 admitted, running at steps 10 and 11 (finishing at 11,
  waits 10 and 9).  The clock ends at 12, the waits sum to 28.

So the page's program would print wall 10 / 12 and mean waits 3.67 / 9.33,
speed-up 1.2.
"""

import numpy as np
import pytest

from oracle.pool_model import PagePoolModel
from oracle.sched_model import CONTINUOUS, STATIC, SchedError, SchedulerModel, run_to_completion


def simulator_example(policy):
    pool = PagePoolModel(page_size=16, num_pages=64)
    m = SchedulerModel(pool, max_batch=64, policy=policy)
    for rid, arrive, tokens in [(0, 0, 10), (1, 1, 2), (2, 2, 2)]:
        m.submit(rid, prompt_len=0, max_new=tokens, arrive=arrive)
    steps = run_to_completion(m)
    return m, steps


def test_simulator_example_continuous():
    m, steps = simulator_example(CONTINUOUS)
    assert m.now == 10 and m.wait_sum == 11 and m.finished == 3
    batches = [(s.step, s.seq_ids) for s in steps if s.seq_ids]
    assert batches == [(0, [0]), (1, [0, 1]), (2, [0, 1, 2]), (3, [0, 2])] + [(t, [0]) for t in range(4, 10)]


def test_simulator_example_static():
    m, steps = simulator_example(STATIC)
    assert m.now == 12 and m.wait_sum == 28 and m.finished == 3
    batches = [(s.step, s.seq_ids) for s in steps if s.seq_ids]
    assert batches == [(t, [0]) for t in range(10)] + [(10, [1, 2]), (11, [1, 2])]
    assert m.now / 10 == pytest.approx(1.2)


def test_idle_clock_jumps_to_next_arrival():
    pool = PagePoolModel(page_size=16, num_pages=8)
    m = SchedulerModel(pool, max_batch=4)
    m.submit(7, prompt_len=3, max_new=2, arrive=5)
    s = m.step()
    assert s.step == 5 and s.seq_ids == [7] and s.admitted == [7]
    assert s.context_lens == [4]


def test_batch_limit_and_slot_reuse():
    """P1's step: at most max_batch run; a finished sequence's place is
    taken by the head of the queue at the very next step."""
    pool = PagePoolModel(page_size=4, num_pages=200)
    m = SchedulerModel(pool, max_batch=3)
    lens = [2, 5, 3, 4, 1, 6]
    for i, n in enumerate(lens):
        m.submit(i, prompt_len=i, max_new=n, arrive=0)
    steps = run_to_completion(m)
    for s in steps:
        assert len(s.seq_ids) <= 3
    # sequence 0 (2 steps) retires at step 2, and 3 joins in that step
    assert steps[2].retired == [0] and steps[2].admitted == [3]
    assert steps[2].seq_ids == [1, 2, 3]
    # every request ran exactly max_new steps
    runs = {}
    for s in steps:
        for sid in s.seq_ids:
            runs[sid] = runs.get(sid, 0) + 1
    assert runs == dict(enumerate(lens))


def test_slots_and_lengths_follow_the_pool():
    """The appended token's slot is the one the pool model gives token
    context_len - 1 of that sequence: page[(n-1) // ps] * ps + (n-1) % ps."""
    pool = PagePoolModel(page_size=4, num_pages=64, initial_free_order=np.random.default_rng(1).permutation(64))
    m = SchedulerModel(pool, max_batch=2)
    m.submit(10, prompt_len=5, max_new=6, arrive=0)
    m.submit(11, prompt_len=0, max_new=3, arrive=1)
    m.submit(12, prompt_len=9, max_new=2, arrive=1)
    seen = {}
    while not m.done():
        s = m.step()
        for sid, slot, n in zip(s.seq_ids, s.new_slots, s.context_lens):
            pages = pool.page_table[sid]
            assert slot == pages[(n - 1) // 4] * 4 + (n - 1) % 4
            assert n == seen.get(sid, {10: 5, 11: 0, 12: 9}[sid]) + 1
            seen[sid] = n
    assert seen == {10: 11, 11: 3, 12: 11}
    assert pool.free_page_count() == 64


def test_page_reservation_blocks_the_queue_in_order():
    """A request waits until the pages of its whole life are free beyond
    what running sequences are still owed; nothing overtakes it."""
    pool = PagePoolModel(page_size=4, num_pages=10)
    m = SchedulerModel(pool, max_batch=8)
    m.submit(1, prompt_len=8, max_new=8, arrive=0)     # reserves 4 pages
    m.submit(2, prompt_len=16, max_new=12, arrive=0)   # reserves 7: 10 - 4 < 7
    m.submit(3, prompt_len=0, max_new=1, arrive=0)     # would fit, but waits behind 2
    s = m.step()
    assert s.admitted == [1] and s.seq_ids == [1]
    for _ in range(7):                                 # 1 runs its 8 steps alone
        s = m.step()
        assert s.seq_ids == [1] and not s.admitted
        assert pool.free_page_count() - m._owed() >= 0
    s = m.step()                                       # 1 retires; 2, then 3, join
    assert s.retired == [1] and s.admitted == [2, 3] and s.seq_ids == [2, 3]
    run_to_completion(m)
    assert pool.free_page_count() == 10 and m.finished == 3


def test_pages_conserved_under_random_traffic():
    rng = np.random.default_rng(5)
    pool = PagePoolModel(page_size=16, num_pages=300)
    for policy in (CONTINUOUS, STATIC):
        pool = PagePoolModel(page_size=16, num_pages=300)
        m = SchedulerModel(pool, max_batch=6, policy=policy)
        arrive = 0
        for i in range(40):
            arrive += int(rng.integers(0, 3))
            m.submit(i, prompt_len=int(rng.integers(0, 200)), max_new=int(rng.integers(1, 60)), arrive=arrive)
        while not m.done():
            s = m.step()
            held = sum(len(v) for v in pool.page_table.values())
            assert held + pool.free_page_count() == 300
            assert pool.free_page_count() - m._owed() >= 0
            assert len(s.seq_ids) <= 6
            if policy == STATIC and s.admitted:
                # static batching only admits into an empty batch
                assert s.seq_ids == s.admitted
        assert m.finished == 40 and pool.free_page_count() == 300


def test_finish_early_and_cancel():
    pool = PagePoolModel(page_size=8, num_pages=20)
    m = SchedulerModel(pool, max_batch=1)
    m.submit(1, prompt_len=3, max_new=100, arrive=0)
    m.submit(2, prompt_len=3, max_new=100, arrive=0)
    m.submit(3, prompt_len=3, max_new=2, arrive=0)
    m.step()
    m.step()
    m.finish(1)             # an end token: retires at the next step
    m.finish(2)             # still waiting: cancelled
    s = m.step()
    assert s.retired == [1] and s.admitted == [3] and s.seq_ids == [3]
    assert m.wait_sum == 1  # 1 generated its last token at step 1
    run_to_completion(m)
    assert m.finished == 2 and pool.free_page_count() == 20


def test_submit_validation():
    pool = PagePoolModel(page_size=4, num_pages=4)
    m = SchedulerModel(pool, max_batch=2)
    m.submit(1, prompt_len=4, max_new=4, arrive=3)
    with pytest.raises(ValueError):
        m.submit(2, prompt_len=1, max_new=1, arrive=2)      # arrival goes back
    with pytest.raises(SchedError):
        m.submit(1, prompt_len=1, max_new=1, arrive=3)      # id in use
    with pytest.raises(SchedError):
        m.submit(3, prompt_len=10, max_new=10, arrive=3)    # 5 pages > 4
    with pytest.raises(ValueError):
        m.submit(4, prompt_len=1, max_new=0, arrive=3)
