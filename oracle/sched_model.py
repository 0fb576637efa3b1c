"""Python model of the continuous-batching step driver over the page pool.

TEST INFRASTRUCTURE (see the package docstring).

What one step does follows "TensorRT-LLM 深度实战：从 Blackwell 架构到 INT4
量化的 LLM 推理性能革命", section 3.2 (continuous batching): finished
sequences leave the batch and give their KV pages back, waiting sequences
join while the batch has room (getting their KV pages), then every running
sequence advances by one token.  The clock, the arrival times, the
static-batching alternative and the two figures of merit (the time the last
request finishes, and the mean over requests of finish step minus arrival
step) follow the request simulator of the aiqz.cc TensorRT-LLM explainer,
sections "连续批处理" and "Python 演示".

Readings where the pages leave a step open:

* the waiting queue is first-come first-served in submission order, and
  arrival steps must not decrease along it (the simulator only ever looks at
  the head of its queue);
* a request is ``prompt_len`` tokens already in the cache when it is
  admitted (their pages are taken then) and finishes after ``max_new``
  decode steps, each of which appends one token; it may also be finished
  early from outside (an end token), which retires it at the next step;
* admission also needs pages: a request reserves the pages of its whole
  life, ceil((prompt_len + max_new) / page_size), so a running sequence
  never runs out of pages mid-generation; the head of the queue is admitted
  only if the free pages minus the pages still owed to running sequences
  cover its reservation, and nothing behind it is admitted before it;
* static batching admits only into an empty batch (the simulator's
  alternative); continuous batching admits whenever there is room;
* with nothing running and the head of the queue not yet arrived, the clock
  jumps to its arrival (the simulator's idle jump);
* the clock advances by one per step that ran at least one sequence;
* a step's sequences are listed in admission order, which is also the order
  of the batch handed to decode.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

from .pool_model import PagePoolModel, UnknownSequence, pages_needed

CONTINUOUS, STATIC = 0, 1


class SchedError(Exception):
    pass


@dataclass
class Request:
    seq_id: int
    prompt_len: int
    max_new: int
    arrive: int
    generated: int = 0
    stop: bool = False          # finished early from outside
    last_step: int = -1         # step of the last generated token


@dataclass
class StepResult:
    step: int                   # clock of this step (after any idle jump)
    seq_ids: List[int]          # the batch, admission order
    new_slots: List[int]        # slot of each sequence's appended token
    context_lens: List[int]     # tokens of each sequence after the append
    admitted: List[int]
    retired: List[int]


class SchedulerModel:
    def __init__(self, pool: PagePoolModel, max_batch: int, policy: int = CONTINUOUS):
        if max_batch <= 0 or policy not in (CONTINUOUS, STATIC):
            raise ValueError("bad scheduler parameters")
        self.pool = pool
        self.max_batch = max_batch
        self.policy = policy
        self.now = 0
        self.waiting: List[Request] = []
        self.running: List[Request] = []
        self.finished = 0
        self.wait_sum = 0

    def _reserve(self, r: Request) -> int:
        return pages_needed(r.prompt_len + r.max_new, self.pool.page_size)

    def submit(self, seq_id: int, prompt_len: int, max_new: int, arrive: int) -> None:
        if prompt_len < 0 or max_new <= 0 or arrive < 0:
            raise ValueError("bad request")
        if self.waiting and arrive < self.waiting[-1].arrive:
            raise ValueError("arrival steps must not decrease along the queue")
        if any(r.seq_id == seq_id for r in self.waiting + self.running) or seq_id in self.pool.page_table:
            raise SchedError(f"sequence {seq_id} exists")
        r = Request(seq_id, prompt_len, max_new, arrive)
        if self._reserve(r) > self.pool.num_pages:
            raise SchedError("request can never fit the pool")
        self.waiting.append(r)

    def finish(self, seq_id: int) -> None:
        for r in self.running:
            if r.seq_id == seq_id:
                r.stop = True
                return
        for i, r in enumerate(self.waiting):
            if r.seq_id == seq_id:
                del self.waiting[i]
                return
        raise UnknownSequence(seq_id)

    def _owed(self) -> int:
        return sum(self._reserve(r) - len(self.pool.page_table[r.seq_id]) for r in self.running)

    def step(self) -> StepResult:
        # 1. retire: sequences done in an earlier step leave and free their pages
        retired = []
        for r in list(self.running):
            if r.generated >= r.max_new or r.stop:
                self.running.remove(r)
                self.pool.release(r.seq_id)
                retired.append(r.seq_id)
                self.finished += 1
                self.wait_sum += r.last_step - r.arrive if r.last_step >= 0 else 0
        # idle: the clock jumps to the next arrival
        if not self.running and self.waiting and self.waiting[0].arrive > self.now:
            self.now = self.waiting[0].arrive
        # 2. admit, first come first served, while the batch has room and the pages fit
        admitted = []
        may_admit = self.policy == CONTINUOUS or not self.running
        while may_admit and len(self.running) < self.max_batch and self.waiting:
            r = self.waiting[0]
            if r.arrive > self.now:
                break
            if self.pool.free_page_count() - self._owed() < self._reserve(r):
                break
            self.waiting.pop(0)
            self.pool.allocate(r.seq_id, r.prompt_len)
            self.running.append(r)
            admitted.append(r.seq_id)
        # 3. one decode step: every running sequence appends one token
        res = StepResult(self.now, [], [], [], admitted, retired)
        if not self.running:
            return res
        for r in self.running:
            (slot,) = self.pool.append_tokens(r.seq_id, 1)
            r.generated += 1
            r.last_step = self.now
            res.seq_ids.append(r.seq_id)
            res.new_slots.append(slot)
            res.context_lens.append(self.pool.token_count[r.seq_id])
        self.now += 1
        return res

    def done(self) -> bool:
        return not self.waiting and not self.running

    def stats(self) -> Dict[str, int]:
        return {"now": self.now, "waiting": len(self.waiting), "running": len(self.running),
                "finished": self.finished, "wait_sum": self.wait_sum}


def run_to_completion(model: SchedulerModel, max_steps: int = 1 << 20) -> List[StepResult]:
    """Steps until every request has retired (the last step runs nothing and
    only retires)."""
    out = []
    for _ in range(max_steps):
        if model.done():
            break
        out.append(model.step())
    return out
