"""The pins of the allocator and scheduler models are strong enough: each
plausible slip in either model fails at least one of them.

Each mutant is the model's source with one deliberate mistake, loaded as a
separate module on the CPU; the names the pin modules use are pointed at it
while the pins run, then restored.  The unmodified sources pass (the pin
modules themselves).
"""

import importlib.util
import os
import sys
import types

import pytest

import test_pool_model as pool_pins
import test_sched_model as sched_pins

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

POOL_MUTANTS = {
    "free_list_fifo": ("[self.free_pages.pop() for _ in range(need)]",
                       "[self.free_pages.pop(0) for _ in range(need)]"),
    "pages_floor": ("return (num_tokens + page_size - 1) // page_size", "return num_tokens // page_size"),
    "release_reversed": ("for page in self.page_table.pop(seq_id):", "for page in reversed(self.page_table.pop(seq_id)):"),
    "copy_even_when_full": ("return n_new > 0 and usage % self.page_size != 0 and self.refcount[pages[-1]] > 1",
                            "return n_new > 0 and self.refcount[pages[-1]] > 1"),
    "shared_page_freed_early": ("            if self.refcount[page] == 0:", "            if True:"),
    "append_overflow_off_by_one": ("if usage + n_new > capacity else 0", "if usage + n_new >= capacity + 1 + 1 else 0"),
    "cow_page_taken_after_overflow": (
        "        copy = None\n        if copy_needed:\n            old, new = pages[-1], self.free_pages.pop()",
        "        copy = None\n        tail = [self.free_pages.pop() for _ in range(over)]\n"
        "        self.free_pages.extend(reversed(tail))\n"
        "        if copy_needed:\n            old, new = pages[-1], self.free_pages.pop(-1 - len(tail)) if tail else self.free_pages.pop()"),
}

SCHED_MUTANTS = {
    "retires_one_token_early": ("if r.generated >= r.max_new or r.stop:", "if r.generated >= r.max_new - 1 or r.stop:"),
    "no_idle_clock_jump": ("            self.now = self.waiting[0].arrive", "            pass"),
    "static_admits_like_continuous": ("may_admit = self.policy == CONTINUOUS or not self.running", "may_admit = True"),
    "no_page_reservation": ("if self.pool.free_page_count() - self._owed() < self._reserve(r):",
                            "if self.pool.free_page_count() < 0:"),
    "wait_off_by_one": ("self.wait_sum += r.last_step - r.arrive if", "self.wait_sum += r.last_step - r.arrive + 1 if"),
    "clock_ticks_when_idle": ("        if not self.running:\n            return res", "        if False:\n            return res"),
    "batch_in_reverse_order": ("            self.running.append(r)\n            admitted.append(r.seq_id)",
                               "            self.running.insert(0, r)\n            admitted.append(r.seq_id)"),
    "batch_limit_off_by_one": ("len(self.running) < self.max_batch", "len(self.running) <= self.max_batch"),
    "reservation_ignores_new_tokens": ("return pages_needed(r.prompt_len + r.max_new, self.pool.page_size)",
                                       "return pages_needed(r.prompt_len, self.pool.page_size)"),
}


def _load(name, src):
    mod = types.ModuleType(f"oracle.{name}")
    mod.__package__ = "oracle"
    sys.modules[mod.__name__] = mod
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _pins(module):
    return [getattr(module, n) for n in dir(module) if n.startswith("test_") and callable(getattr(module, n))]


def _run_pins(modules, patches):
    """True if some pin fails with the patched names."""
    saved = [(m, k, getattr(m, k)) for m, kv in patches.items() for k in kv]
    try:
        for m, kv in patches.items():
            for k, v in kv.items():
                setattr(m, k, v)
        for mod in modules:
            for fn in _pins(mod):
                try:
                    fn()
                except Exception:
                    return True
        return False
    finally:
        for m, k, v in saved:
            setattr(m, k, v)


def _mutant_source(path, old, new):
    src = open(path).read()
    assert src.count(old) == 1, f"mutation anchor not unique / missing: {old[:60]!r}"
    return src.replace(old, new)


POOL_NAMES = ("PagePoolModel", "pages_needed", "OutOfPages", "SequenceExists", "UnknownSequence",
              "SharedLastPage")
SCHED_NAMES = ("SchedulerModel", "run_to_completion", "CONTINUOUS", "STATIC", "SchedError")


def _pool_patches(mod):
    return {pool_pins: {n: getattr(mod, n) for n in POOL_NAMES if hasattr(pool_pins, n)}}


def _sched_patches(mod):
    return {sched_pins: {n: getattr(mod, n) for n in SCHED_NAMES if hasattr(sched_pins, n)}}


def _pool_source(old=None, new=None):
    path = os.path.join(ORACLE, "pool_model.py")
    return open(path).read() if old is None else _mutant_source(path, old, new)


def _sched_source(old=None, new=None):
    path = os.path.join(ORACLE, "sched_model.py")
    return open(path).read() if old is None else _mutant_source(path, old, new)


@pytest.mark.parametrize("name", sorted(POOL_MUTANTS))
def test_pool_model_mutant_is_caught(name):
    mod = _load(f"_mut_pool_{name}", _pool_source(*POOL_MUTANTS[name]))
    assert _run_pins([pool_pins], _pool_patches(mod)), f"pool mutant {name} survived every pin"


@pytest.mark.parametrize("name", sorted(SCHED_MUTANTS))
def test_scheduler_model_mutant_is_caught(name):
    mod = _load(f"_mut_sched_{name}", _sched_source(*SCHED_MUTANTS[name]))
    assert _run_pins([sched_pins], _sched_patches(mod)), f"scheduler mutant {name} survived every pin"


def test_unmodified_models_pass_the_pins():
    """The same loading and patching with the unmodified sources: every pin
    passes, so a caught mutant is caught by its mutation."""
    pool = _load("_mut_pool_none", _pool_source())
    sched = _load("_mut_sched_none", _sched_source())
    assert not _run_pins([pool_pins], _pool_patches(pool))
    assert not _run_pins([sched_pins], _sched_patches(sched))
