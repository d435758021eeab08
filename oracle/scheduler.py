"""Reference continuous-batching scheduler (TEST INFRASTRUCTURE ONLY).

Plain Python, written from the PhotonInfer README ("Technical details ->
Continuous-batching scheduler": phase 1 continues every running request,
phase 2 admits waiting requests into the remaining capacity; waiting ->
running -> finished with preemption; num_computed_tokens marks the resume
point.  "Technical details -> Paged attention": block-level KV cache and
per-sequence block tables).  Where the page is silent the reading is:

* capacity per step is max_seqs requests and max_tokens_per_step new tokens;
* a running request that has not computed all its known tokens takes as
  many as the budget allows while leaving one token for every running
  request after it (so none is skipped); a prompt longer than the budget
  is thus computed in chunks;
* blocks come from a first-in first-out free list; when a running request
  needs more blocks than are free, the most recently admitted running
  request is preempted (blocks freed, cached tokens forgotten, back to the
  front of the waiting queue) until enough are free;
* admission (phase 2) is first-come first-served, stops at the first
  request whose blocks do not fit, and never preempts;
* after a step, a request whose known tokens are all computed generates one
  token; after max_new_tokens it finishes and frees its blocks.

The product implementation is C++ (csrc/scheduler.cpp); the tests compare
the two step by step on seeded request traces.
"""
from __future__ import annotations

import math

WAITING, RUNNING, FINISHED = 0, 1, 2


class OracleRequest:
    def __init__(self, rid: int, prompt_len: int, max_new: int):
        self.rid = rid
        self.prompt_len = prompt_len
        self.max_new = max_new
        self.known = prompt_len        # prompt + generated
        self.computed = 0              # known tokens whose K/V are cached
        self.generated = 0
        self.preemptions = 0
        self.state = WAITING
        self.blocks: list[int] = []
        self.step_tokens = 0


class OracleScheduler:
    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_tokens_per_step: int,
                 max_blocks_per_seq: int):
        if min(num_blocks, block_size, max_seqs, max_blocks_per_seq) <= 0 \
                or max_tokens_per_step < max_seqs:
            raise ValueError("bad scheduler configuration")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_tokens = max_tokens_per_step
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks))
        self.requests: dict[int, OracleRequest] = {}
        self.waiting: list[OracleRequest] = []
        self.running: list[OracleRequest] = []
        self.scheduled: list[OracleRequest] | None = None
        self.finished = 0

    def add_request(self, rid: int, prompt_len: int, max_new: int) -> None:
        if prompt_len < 1 or max_new < 1 or rid in self.requests:
            raise ValueError("bad request")
        most = math.ceil((prompt_len + max_new - 1) / self.block_size)
        if most > self.max_blocks_per_seq or most > self.num_blocks:
            raise ValueError("request can never fit")
        r = OracleRequest(rid, prompt_len, max_new)
        self.requests[rid] = r
        self.waiting.append(r)

    def _blocks_missing(self, r: OracleRequest, n: int) -> int:
        return math.ceil((r.computed + n) / self.block_size) - len(r.blocks)

    def _give_blocks(self, r: OracleRequest, count: int) -> None:
        for _ in range(count):
            r.blocks.append(self.free.pop(0))

    def schedule(self) -> dict:
        if self.scheduled is not None:
            raise RuntimeError("schedule twice without update")
        budget = self.max_tokens
        batch: list[OracleRequest] = []
        preempted: list[int] = []

        # phase 1: every running request continues
        i = 0
        while i < len(self.running):
            r = self.running[i]
            later = len(self.running) - 1 - i
            n = min(r.known - r.computed, budget - later)
            dropped_self = False
            while len(self.free) < self._blocks_missing(r, n):
                victim = self.running.pop()
                self.free.extend(victim.blocks)
                victim.blocks = []
                victim.computed = 0
                victim.state = WAITING
                victim.preemptions += 1
                self.waiting.insert(0, victim)
                preempted.append(victim.rid)
                if victim is r:
                    dropped_self = True
                    break
            if dropped_self:
                break
            self._give_blocks(r, self._blocks_missing(r, n))
            r.step_tokens = n
            budget -= n
            batch.append(r)
            i += 1

        # phase 2: admit waiting requests, first come first served
        while self.waiting and len(batch) < self.max_seqs and budget > 0:
            r = self.waiting[0]
            n = min(r.known - r.computed, budget)
            need = self._blocks_missing(r, n)
            if need > len(self.free):
                break
            self.waiting.pop(0)
            self._give_blocks(r, need)
            r.state = RUNNING
            self.running.append(r)
            r.step_tokens = n
            budget -= n
            batch.append(r)

        self.scheduled = batch
        bs = self.block_size
        out = {"request_ids": [], "query_start": [0], "context_lens": [], "block_tables": [],
               "slot_mapping": [], "positions": [], "preempted": preempted}
        for r in batch:
            out["request_ids"].append(r.rid)
            for pos in range(r.computed, r.computed + r.step_tokens):
                out["positions"].append(pos)
                out["slot_mapping"].append(r.blocks[pos // bs] * bs + pos % bs)
            out["query_start"].append(len(out["positions"]))
            out["context_lens"].append(r.computed + r.step_tokens)
            out["block_tables"].append(r.blocks + [-1] * (self.max_blocks_per_seq - len(r.blocks)))
        return out

    def update(self) -> list[int]:
        if self.scheduled is None:
            raise RuntimeError("update without schedule")
        done = []
        for r in self.scheduled:
            r.computed += r.step_tokens
            r.step_tokens = 0
            if r.computed == r.known:
                r.generated += 1
                r.known += 1
                if r.generated == r.max_new:
                    self.free.extend(r.blocks)
                    r.blocks = []
                    r.state = FINISHED
                    self.running.remove(r)
                    self.finished += 1
                    done.append(r.rid)
        self.scheduled = None
        return done
