"""Block manager and two-phase scheduler: reference pins and native parity (CPU).

The reference (oracle/scheduler.py) is pinned to two traces worked out by
hand from the scheduler rules (tests/golden/sched_two_traces.json) and to
invariants that must hold on any trace.  The native scheduler
(csrc/scheduler.cpp through the C ABI) must then match the reference step
by step, bit for bit, on seeded request traces.
"""
import json
import os

import numpy as np
import pytest

import decode_inputs as di
from oracle.scheduler import FINISHED, OracleScheduler
from paged_attention_decode_photon_amd import PhotonError
from paged_attention_decode_photon_amd.sched import Scheduler

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sched_two_traces.json")
KEYS = ("request_ids", "query_start", "context_lens", "block_tables", "slot_mapping", "positions",
        "preempted")


def as_lists(out):
    return {k: np.asarray(out[k]).tolist() for k in KEYS}


def run_trace(sched, trace, max_steps=100000):
    """Drive ``sched`` over a request trace; returns the per-step records."""
    steps, i, total, done = [], 0, len(trace), 0
    for step in range(max_steps):
        while i < total and trace[i][0] <= step:
            _, rid, p, n = trace[i]
            sched.add_request(rid, p, n)
            i += 1
        out = as_lists(sched.schedule())
        out["finished"] = np.asarray(sched.update()).tolist()
        steps.append(out)
        done += len(out["finished"])
        if done == total:
            return steps
    raise AssertionError("trace did not finish")


# ------------------------------------------------------------- reference pins

def golden_traces():
    return json.load(open(GOLDEN))["traces"]


@pytest.mark.parametrize("idx", [0, 1])
def test_reference_matches_hand_worked_traces(idx):
    tr = golden_traces()[idx]
    s = OracleScheduler(**tr["config"])
    for _, rid, p, n in tr["requests"]:
        s.add_request(rid, p, n)
    for k, exp in enumerate(tr["steps"]):
        out = as_lists(s.schedule())
        out["finished"] = s.update()
        assert out == exp, f"{tr['name']} step {k}"
    assert s.free == tr["final_free_blocks"]
    assert {str(r): q.preemptions for r, q in s.requests.items()} == tr["preemptions"]


def check_invariants(tc, steps, sched):
    """Facts any correct run must satisfy, whatever the scheduling choices."""
    bs, cfg = tc.block_size, tc.sched_config()
    trace = {rid: (a, p, n) for a, rid, p, n in di.make_request_trace(tc)}
    held = {}      # request -> blocks it held at its last scheduled step
    prev_running = []
    generated = {rid: 0 for rid in trace}
    first_step = {}
    for k, st in enumerate(steps):
        ids, qs = st["request_ids"], st["query_start"]
        assert len(ids) <= cfg["max_seqs"] and qs[-1] <= cfg["max_tokens_per_step"]
        assert len(set(ids)) == len(ids)
        # running requests are never skipped unless preempted
        for rid in prev_running:
            assert rid in ids or rid in st["preempted"], f"step {k}: running {rid} skipped"
        slots = st["slot_mapping"]
        assert len(set(slots)) == len(slots), f"step {k}: slot written twice"
        live_blocks = []
        for b, rid in enumerate(ids):
            table = [x for x in st["block_tables"][b] if x >= 0]
            pos = st["positions"][qs[b]:qs[b + 1]]
            assert len(pos) >= 1
            assert pos == list(range(pos[0], pos[0] + len(pos))), "positions not contiguous"
            assert st["context_lens"][b] == pos[-1] + 1
            assert len(table) == -(-st["context_lens"][b] // bs), "table not minimal"
            for j, p in enumerate(pos):
                assert slots[qs[b] + j] == table[p // bs] * bs + p % bs
            live_blocks += table
            held[rid] = table
            first_step.setdefault(rid, k)
        assert len(set(live_blocks)) == len(live_blocks), f"step {k}: a block is shared"
        assert all(0 <= x < cfg["num_blocks"] for x in live_blocks)
        for rid in st["finished"]:
            generated[rid] = trace[rid][2]
        prev_running = [r for r in ids if r not in st["finished"]]
    # every request ran to its length and nothing is left allocated
    assert all(sched.requests[r].state == FINISHED for r in trace)
    assert all(sched.requests[r].generated == trace[r][2] for r in trace)
    assert sorted(sched.free) == list(range(cfg["num_blocks"]))
    # first admissions follow arrival order (first come, first served)
    order = sorted(first_step, key=lambda r: (first_step[r], steps[first_step[r]]["request_ids"].index(r)))
    assert order == sorted(order, key=lambda r: (trace[r][0], r))


@pytest.mark.parametrize("name", ["tight", "chunked"])
def test_reference_invariants_on_traces(name):
    tc = di.TRACES[name]
    s = OracleScheduler(**tc.sched_config())
    steps = run_trace(s, di.make_request_trace(tc))
    check_invariants(tc, steps, s)
    if name == "tight":
        assert sum(len(st["preempted"]) for st in steps) > 0, "trace meant to exercise preemption"


def test_reference_decode_only_steps_have_one_token_per_request():
    # Once every admitted prompt is computed, each step is pure decode: one
    # token per running request, at position context_len - 1.
    s = OracleScheduler(num_blocks=64, block_size=16, max_seqs=4, max_tokens_per_step=64,
                        max_blocks_per_seq=8)
    for rid in range(4):
        s.add_request(rid, 10 + rid, 20)
    s.schedule(); s.update()
    for _ in range(19):
        out = s.schedule()
        assert out["query_start"] == [0, 1, 2, 3, 4]
        assert out["positions"] == [c - 1 for c in out["context_lens"]]
        s.update()


# ------------------------------------------------------------- native parity

@pytest.mark.parametrize("idx", [0, 1])
def test_native_matches_hand_worked_traces(idx):
    tr = golden_traces()[idx]
    s = Scheduler(**tr["config"])
    for _, rid, p, n in tr["requests"]:
        s.add_request(rid, p, n)
    for k, exp in enumerate(tr["steps"]):
        out = as_lists(s.schedule())
        out["finished"] = s.update().tolist()
        assert out == exp, f"{tr['name']} step {k}"
    assert s.counts()["free_blocks"] == len(tr["final_free_blocks"])
    for r, n in tr["preemptions"].items():
        assert s.request(int(r))["num_preemptions"] == n


@pytest.mark.parametrize("name", ["tight", "chunked", "serving"])
def test_native_matches_reference_step_by_step(name):
    tc = di.TRACES[name]
    trace = di.make_request_trace(tc)
    ref = run_trace(OracleScheduler(**tc.sched_config()), trace)
    nat_s = Scheduler(**tc.sched_config())
    nat = run_trace(nat_s, trace)
    assert len(nat) == len(ref)
    for k, (a, b) in enumerate(zip(nat, ref)):
        assert a == b, f"{name}: step {k} differs"
    c = nat_s.counts()
    assert c == {"waiting": 0, "running": 0, "finished": len(trace), "free_blocks": tc.num_blocks}


def test_native_request_info_tracks_resume_point():
    s = Scheduler(num_blocks=3, block_size=2, max_seqs=3, max_tokens_per_step=4, max_blocks_per_seq=3)
    for rid, p, n in [(0, 2, 3), (1, 2, 3), (2, 1, 2)]:
        s.add_request(rid, p, n)
    s.schedule(); s.update()
    s.schedule()      # request 1 is preempted here
    info = s.request(1)
    assert info["state"] == 0 and info["num_computed"] == 0 and info["num_known"] == 3
    assert info["num_blocks"] == 0 and info["num_preemptions"] == 1
    s.update()


# ----------------------------------------------------------- argument checks

@pytest.mark.parametrize("cfg", [
    dict(num_blocks=0, block_size=16, max_seqs=4, max_tokens_per_step=64, max_blocks_per_seq=8),
    dict(num_blocks=8, block_size=0, max_seqs=4, max_tokens_per_step=64, max_blocks_per_seq=8),
    dict(num_blocks=8, block_size=16, max_seqs=0, max_tokens_per_step=64, max_blocks_per_seq=8),
    dict(num_blocks=8, block_size=16, max_seqs=8, max_tokens_per_step=4, max_blocks_per_seq=8),
    dict(num_blocks=8, block_size=16, max_seqs=4, max_tokens_per_step=64, max_blocks_per_seq=0),
    dict(num_blocks=1 << 28, block_size=16, max_seqs=4, max_tokens_per_step=64, max_blocks_per_seq=8),
])
def test_native_rejects_bad_configuration(cfg):
    with pytest.raises(PhotonError):
        Scheduler(**cfg)


def test_native_rejects_bad_requests_and_call_order():
    s = Scheduler(num_blocks=8, block_size=16, max_seqs=4, max_tokens_per_step=64, max_blocks_per_seq=4)
    for args in [(0, 0, 5), (0, 5, 0), (0, 60, 6), (0, 120, 20)]:   # empty, or can never fit
        with pytest.raises(PhotonError):
            s.add_request(*args)
    s.add_request(7, 60, 5)   # 64 cached tokens at most: 4 blocks
    with pytest.raises(PhotonError):
        s.add_request(7, 3, 3)  # duplicate id
    with pytest.raises(PhotonError):
        s.update()              # nothing scheduled
    s.schedule()
    with pytest.raises(PhotonError):
        s.schedule()            # schedule twice
    s.update()
    with pytest.raises(PhotonError):
        s.request(99)
