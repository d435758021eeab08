"""The scheduler reference's pins must reject plausible mistakes.

Each case plants one mistake into a copy of oracle/scheduler.py, loads it
as a fresh module and runs the hand-worked traces and the invariant checks
against it: at least one has to fail.
"""
import os
import types

import pytest

import decode_inputs as di
import oracle.scheduler as ref
import tests.test_scheduler as ts

SRC = open(ref.__file__).read()

# Dropping phase 1's reserve of one token per later running request is not
# listed: under these rules a request still computing its prompt is always
# the last running one (admission gives a request all the budget left, so a
# later admission only happens once the earlier prompt is done), so the
# reserve never binds and that change is an equivalent program.
MUTANTS = {
    "free_list_lifo": ("r.blocks.append(self.free.pop(0))", "r.blocks.append(self.free.pop())"),
    "preempt_oldest": ("victim = self.running.pop()", "victim = self.running.pop(0)"),
    "preempted_to_back_of_queue": ("self.waiting.insert(0, victim)", "self.waiting.append(victim)"),
    "preemption_keeps_cached_count": ("victim.computed = 0\n", "\n"),
    "generate_before_prompt_done": ("            if r.computed == r.known:\n",
                                    "            if r.computed >= 0:\n"),
    "context_excludes_new_tokens": ('out["context_lens"].append(r.computed + r.step_tokens)',
                                    'out["context_lens"].append(r.computed)'),
    "slot_offset_wrong": ("r.blocks[pos // bs] * bs + pos % bs", "r.blocks[pos // bs] * bs + pos % 2"),
    "admission_ignores_seq_limit": ("while self.waiting and len(batch) < self.max_seqs and budget > 0:",
                                    "while self.waiting and budget > 0:"),
    "finish_keeps_blocks": ("                    self.free.extend(r.blocks)\n                    r.blocks = []\n",
                            "                    r.blocks = []\n"),
}


def _suite(mod):
    failures = []
    saved = ts.OracleScheduler
    ts.OracleScheduler = mod.OracleScheduler
    ts.FINISHED = mod.FINISHED
    try:
        for idx in (0, 1):
            try:
                ts.test_reference_matches_hand_worked_traces(idx)
            except Exception as e:  # noqa: BLE001
                failures.append(f"golden {idx}: {type(e).__name__}")
        for name in ("tight", "chunked"):
            try:
                tc = di.TRACES[name]
                s = mod.OracleScheduler(**tc.sched_config())
                steps = ts.run_trace(s, di.make_request_trace(tc), max_steps=20000)
                ts.check_invariants(tc, steps, s)
            except Exception as e:  # noqa: BLE001
                failures.append(f"invariants {name}: {type(e).__name__}")
    finally:
        ts.OracleScheduler = saved
        ts.FINISHED = ref.FINISHED
    return failures


def _load(text, tag):
    mod = types.ModuleType(f"sched_mutant_{tag}")
    exec(compile(text, f"<sched mutant {tag}>", "exec"), mod.__dict__)
    return mod


def test_unmodified_reference_passes():
    assert _suite(_load(SRC, "clean")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_scheduler_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"anchor for {name} not found once"
    assert _suite(_load(SRC.replace(old, new), name)), f"no pin rejects the '{name}' mutant"
