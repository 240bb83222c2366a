"""Oracle of one continuous-batching scheduler step (test infrastructure only: tests,
the smoke check and the benchmark's CPU baseline may use it; the product never does).

The policy is the engine loop of "Continuous Batching" (infra.pidoku inference
notes), section "4. Tiny example" (the Go `Engine.Step` with `preempt`), with
the lifecycle of its section "1. What is it?" and the recompute preemption of
"5. Technical explanation":

  1. admit from the head of the waiting queue while fewer than max_running run and
     the head's blocks can be allocated; stop at the first that does not fit;
  2. one forward pass over every running request (prefill rows for the newly
     admitted, one decode row for the others);
  3. in running order: append one output token; a request that reached its output
     count frees its blocks at once; one that needs a new block for its next token
     allocates one, and if that fails it is preempted: its blocks are freed and it
     goes to the FRONT of the waiting queue, to be re-prefilled later.

Readings taken where the page leaves a step open (each listed with the others):
  * blocks needed at admission = ceil((prompt + outputs so far) / block_size): a
    preempted request re-prefills its prompt and the outputs it already has;
  * the prefill row of a request holds prompt + outputs-so-far new tokens at
    positions 0.. ; a decode row is the last output token at position
    prompt + outputs - 1 (its K/V is written by that step), seeing all positions up to
    it;
  * a request finishes when its output count reaches max_tokens (no EOS: no model);
  * arrivals: the requests whose arrival step is <= the current step join the back of
    the waiting queue in (arrival, id) order at the start of the step;
  * a step with nothing running emits no rows (the loop returns before the forward);
  * chunked prefill (the mixed batching of "5. Technical explanation", off unless a
    budget or a chunk size is given): a step carries at most max_batched_tokens new
    tokens. Decode rows are never cut (one token each, even past the budget); what the
    budget leaves goes to prefill rows in running order, each taking the least of its
    uncomputed context, chunk_tokens and the budget left, so a request can get no row
    in a step. A chunk holds positions done..done+q-1 and sees every position below
    done+q; the request's first output comes at the step of its last chunk; its blocks
    are still all reserved at admission, and its prompt pages enter the prefix cache
    only once the prefill is complete;
  * preemption by swap (the SWAP strategy of "5. Technical explanation", off unless a
    host swap space is given): the victim's blocks are copied, in table order, into
    host blocks taken from a host free list (LIFO, like the device pool) and its device
    blocks are freed; it goes to the front of the queue as with recompute. When the host
    space lacks blocks for the whole table the request is preempted by recompute instead.
    A swapped request is admitted like any other (blocks for prompt + outputs, strict
    FCFS, no prefix lookup); its host blocks are copied back into the first blocks of
    its new table and returned to the host free list in table order, and it resumes where
    it stopped (no prefill of what it had: its decode row, or with victim policies below
    possibly its next prefill chunk). The copies are listed per step: swap-outs by the update
    (to run before the next step's kernels), swap-ins by the schedule (before the step's
    attention);
  * victim policies (the victim selection of "5. Technical explanation": LIFO keeps the
    progress of long-running requests; the pure-Python engine's preemption takes the
    running request with the fewest generated tokens): with victim "lifo" or "fewest"
    the update first appends every row's output and frees finished requests (running
    order), then walks the running requests in order; one that needs a block for its
    next token and finds none preempts victims until it gets one: "lifo" takes the
    running request admitted last, "fewest" the one with the fewest outputs (the earliest
    admitted on ties), each among the least important priority class present; when the
    victim is the request itself it stops there. The default "self" is the Go loop's
    one-pass update, where the request that cannot grow preempts itself;
  * priority admission (the Priority admission policy of "5. Technical explanation";
    the priority classes of the serving project's extensions): given a class per
    request (0 most important), the waiting queue is kept in (class, arrival step, id)
    order, preempted requests included (they take their place by that key rather than
    the front); admission still stops at the first head that does not fit;
  * static batching (the baseline of "1. What is it?" and "2. Why does it exist?": a batch
    is decided, run to completion, then the next one is decided): admission happens
    only at steps that start with nothing running; finished requests still free their
    blocks at once, but their slots stay empty until the whole batch is done.

Parity unpinned beyond invariants and hand-worked traces: the pages print no trace of
this loop, so the tests pin it with small traces worked out by hand from the page's
loop and with invariants (conservation of blocks, strict first-come-first-served
admission, exact output counts, no leak) on random and full-size traces.
"""
from __future__ import annotations

import collections
import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import allocator as oa
from . import prefix as opx
from .metadata import build_block_table

PREFILL, DECODE = 0, 1


@dataclasses.dataclass
class Req:
    rid: int
    arrival: int
    prompt: int
    max_tokens: int
    n_out: int = 0
    stage: int = PREFILL
    preempted: int = 0
    finished_step: int = -1
    prio: int = 0                              # priority class (0: most important)
    host: Optional[List[int]] = None           # host blocks holding its swapped-out K/V
    tokens: Optional[Tuple[int, ...]] = None   # prompt token ids (prefix caching)
    cached: int = 0                            # prompt tokens of this prefill found in the cache
    done: int = 0                              # context tokens of the current prefill computed so far
    q_step: int = 0                            # new tokens of this request's row in the current step


@dataclasses.dataclass
class StepPlan:
    """What one step hands to the device: rows in running order and their metadata."""
    step: int
    ids: np.ndarray          # int64 [n] request ids
    stages: np.ndarray       # int32 [n] PREFILL / DECODE
    q_lens: np.ndarray       # int32 [n] new tokens of each row
    seq_lens: np.ndarray     # int32 [n] context including the new tokens
    block_tables: np.ndarray  # int32 [n][width], -1 padded
    cu_seqlens_q: np.ndarray  # int32 [n + 1]
    slot_mapping: np.ndarray  # int64 [sum q]
    counters: Dict[str, int]
    swap_in: List[Tuple[int, int]] = dataclasses.field(default_factory=list)   # (host block, device block)


class Scheduler:
    def __init__(self, arrival, prompt, max_tokens, num_blocks: int, free_order, block_size: int,
                 max_running: int, admission_check: bool = True,
                 prompt_tokens: Optional[Sequence[Sequence[int]]] = None, max_batched_tokens: int = 0,
                 chunk_tokens: int = 0, swap_blocks: int = 0, victim: str = "self",
                 priority: Optional[Sequence[int]] = None, static: bool = False):
        self.reqs = [Req(i, int(a), int(p), int(m)) for i, (a, p, m) in enumerate(zip(arrival, prompt, max_tokens))]
        # prompt_tokens given: prefix caching over shared blocks (oracle/prefix.py)
        self.pcache = None
        self.arrival_order = sorted(range(len(self.reqs)), key=lambda i: (self.reqs[i].arrival, i))
        self.next_arrival = 0
        self.pool = oa.BlockPool(num_blocks, free_order)
        self.tables = oa.SeqTables(self.pool, block_size)
        if prompt_tokens is not None:
            self.tables = opx.SharedTables(self.pool, block_size)
            self.pcache = opx.PrefixCache(self.tables)
            for r, tok in zip(self.reqs, prompt_tokens):
                if len(tok) != r.prompt:
                    raise ValueError(f"request {r.rid}: {len(tok)} tokens for a prompt of {r.prompt}")
                r.tokens = tuple(int(x) for x in tok)
        self.cached_tokens = 0
        self.bs = block_size
        for r in self.reqs:                     # a request that cannot fit alone would stall the queue
            if -(-(r.prompt + r.max_tokens - 1) // block_size) > num_blocks:
                raise ValueError(f"request {r.rid} needs more than the pool's {num_blocks} blocks")
        self.max_running = max_running
        # admission_check=False is the sabotage of the "Break It" experiment of "Project 17"
        # (its admission loop pops the head and prefills it with no memory check): the head
        # is taken off the queue and its allocation may raise OutOfBlocks out of the step
        self.admission_check = admission_check
        # chunked prefill ([CB] "5. Technical explanation", mixed batching): at most
        # max_batched_tokens new tokens per step (0: no limit), decode rows first, then
        # prefill chunks of at most chunk_tokens (0: no limit) in running order
        self.max_batched_tokens = int(max_batched_tokens)
        self.chunk_tokens = int(chunk_tokens)
        if self.max_batched_tokens < 0 or self.chunk_tokens < 0:
            raise ValueError("token budget and chunk size must be >= 0")
        # preemption by swap into a host space of swap_blocks blocks (0: recompute only)
        if swap_blocks < 0:
            raise ValueError("swap_blocks must be >= 0")
        self.host = oa.BlockPool(swap_blocks) if swap_blocks > 0 else None
        self.swap_out: List[Tuple[int, int]] = []   # (device block, host block) of the last update
        self.swapped_out = self.blocks_out = self.blocks_in = 0
        if victim not in ("self", "lifo", "fewest"):
            raise ValueError(f"unknown victim policy {victim!r}")
        self.victim = victim
        self.static = bool(static)                # admit only when the batch has drained
        self.by_priority = priority is not None
        if priority is not None:
            if len(priority) != len(self.reqs) or min(priority, default=0) < 0:
                raise ValueError("one priority class >= 0 per request")
            for r, c in zip(self.reqs, priority):
                r.prio = int(c)
        self.waiting: collections.deque = collections.deque()
        self.running: List[Req] = []
        self.step_no = 0
        self.preemptions = 0
        self.finished = 0

    # -- counters -------------------------------------------------------------------
    def counters(self) -> Dict[str, int]:
        c = {"free": self.pool.num_free, "running": len(self.running), "waiting": len(self.waiting),
             "preempted": self.preemptions, "finished": self.finished}
        if self.pcache is not None:
            c["cached_tokens"] = self.cached_tokens
        if self.host is not None:
            c.update(swapped_out=self.swapped_out, blocks_out=self.blocks_out, blocks_in=self.blocks_in)
        return c

    def done(self) -> bool:
        return self.finished == len(self.reqs)

    # -- one step, first half: arrivals, admission, the rows of the forward pass -------
    def schedule(self, width: int) -> StepPlan:
        s = self.step_no
        while self.next_arrival < len(self.arrival_order):
            r = self.reqs[self.arrival_order[self.next_arrival]]
            if r.arrival > s:
                break
            self._enqueue(r, front=False)
            self.next_arrival += 1
        swap_in = []
        admit = not (self.static and self.running)
        while admit and self.waiting and len(self.running) < self.max_running:
            r = self.waiting[0]
            ctx = r.prompt + r.n_out
            if r.host is not None:                                  # swapped out: copy back
                if self.admission_check and self.tables.blocks_for(ctx) > self.pool.num_free:
                    break
                self.waiting.popleft()
                self.tables.reserve(r.rid, ctx)
                swap_in += list(zip(r.host, self.tables.tables[r.rid]))
                self.blocks_in += len(r.host)
                self.host.release(r.host)
                r.host = None                                       # resumes in its stage
                self.running.append(r)
                continue
            n_hit, pages = 0, []
            if self.pcache is not None:                             # longest cached prefix
                n_hit, pages = self.pcache.lookup(r.tokens, min(r.prompt, ctx - 1))
            if not self.admission_check:
                self.waiting.popleft()
            elif self.tables.blocks_for(ctx) - len(pages) > self.pool.num_free:
                break                                               # strict FCFS: stop here
            else:
                self.waiting.popleft()
            if pages:
                self.tables.share(r.rid, pages)
            self.tables.reserve(r.rid, ctx)                         # all-or-nothing; unchecked: may raise
            r.stage = PREFILL
            r.cached = n_hit
            r.done = n_hit
            self.cached_tokens += n_hit
            self.running.append(r)
        # this step's new tokens per running request: decode rows first, then prefill
        # chunks in running order within what the budget leaves
        budget = None
        if self.max_batched_tokens > 0:
            budget = max(0, self.max_batched_tokens - sum(r.stage == DECODE for r in self.running))
        for r in self.running:
            if r.stage == DECODE:
                r.q_step = 1
                continue
            q = r.prompt + r.n_out - r.done
            if self.chunk_tokens > 0:
                q = min(q, self.chunk_tokens)
            if budget is not None:
                q = min(q, budget)
                budget -= q
            r.q_step = q
        ids, stages, q, L = [], [], [], []
        for r in self.running:
            if r.q_step == 0:
                continue                                            # no row this step
            ids.append(r.rid)
            stages.append(r.stage)
            q.append(r.q_step)
            L.append(r.done + r.q_step if r.stage == PREFILL else r.prompt + r.n_out)
        tabs = [self.tables.tables[i] for i in ids]
        bt, cu, slots = build_block_table(tabs, q, L, self.bs, width)
        return StepPlan(s, np.asarray(ids, np.int64), np.asarray(stages, np.int32), np.asarray(q, np.int32),
                        np.asarray(L, np.int32), bt, cu, slots, self.counters(), swap_in)

    # -- queue and preemption helpers ---------------------------------------------------
    def _enqueue(self, r: Req, front: bool) -> None:
        if not self.by_priority:
            (self.waiting.appendleft if front else self.waiting.append)(r)
            return
        key = (r.prio, r.arrival, r.rid)
        k = 0
        while k < len(self.waiting) and (self.waiting[k].prio, self.waiting[k].arrival, self.waiting[k].rid) < key:
            k += 1
        self.waiting.insert(k, r)

    def _preempt(self, r: Req) -> None:
        table = self.tables.tables[r.rid]
        if self.host is not None and self.host.num_free >= len(table):
            r.host = self.host.alloc(len(table))                    # by swap
            self.swap_out += list(zip(table, r.host))
            self.swapped_out += 1
            self.blocks_out += len(table)
        self.tables.release(r.rid)                                  # (else by recompute)
        r.preempted += 1
        self.preemptions += 1
        self._enqueue(r, front=True)

    def _pick_victim(self, alive: List[Req]) -> Req:
        worst = max(c.prio for c in alive)
        pool = [c for c in alive if c.prio == worst]
        if self.victim == "lifo":
            return pool[-1]
        return min(pool, key=lambda c: c.n_out)                     # first minimum: earliest admitted

    # -- second half: one output token per row, retire, grow or preempt --------------
    def update(self) -> None:
        self.swap_out = []
        for r in self.running:
            if r.stage == PREFILL:
                r.done += r.q_step
        if self.pcache is not None:                                 # prefills completed: their pages
            for r in self.running:
                if r.stage == PREFILL and r.done == r.prompt + r.n_out:
                    self.pcache.insert(r.tokens, self.tables.tables[r.rid], r.prompt)
        if self.victim != "self":
            self._update_with_victims()
            return
        still = []
        for r in self.running:
            had_row = r.q_step > 0
            r.q_step = 0
            if not had_row or (r.stage == PREFILL and r.done < r.prompt + r.n_out):
                still.append(r)                                     # no output this step
                continue
            r.cached = 0
            r.n_out += 1
            r.stage = DECODE
            if r.n_out >= r.max_tokens:
                self.tables.release(r.rid)                          # freed at once
                r.finished_step = self.step_no
                self.finished += 1
                continue
            need = r.prompt + r.n_out                               # tokens its next row writes up to
            if need > len(self.tables.tables[r.rid]) * self.bs:
                try:
                    self.tables.reserve(r.rid, need)                # one more block
                except oa.OutOfBlocks:
                    self._preempt(r)                                # the request preempts itself
                    continue
            still.append(r)
        self.running = still
        self.step_no += 1

    def _update_with_victims(self) -> None:
        # outputs and retirements first, in running order
        alive, grew = [], set()
        for r in self.running:
            had_row = r.q_step > 0
            r.q_step = 0
            if not had_row or (r.stage == PREFILL and r.done < r.prompt + r.n_out):
                alive.append(r)
                continue
            r.cached = 0
            r.n_out += 1
            r.stage = DECODE
            if r.n_out >= r.max_tokens:
                self.tables.release(r.rid)
                r.finished_step = self.step_no
                self.finished += 1
                continue
            alive.append(r)
            grew.add(r.rid)
        # then the blocks for the next tokens, victims chosen by the policy
        k = 0
        while k < len(alive):
            r = alive[k]
            need = r.prompt + r.n_out
            if r.rid in grew and need > len(self.tables.tables[r.rid]) * self.bs:
                while True:
                    try:
                        self.tables.reserve(r.rid, need)
                        break
                    except oa.OutOfBlocks:
                        v = self._pick_victim(alive)
                        if alive.index(v) < k:
                            k -= 1
                        alive.remove(v)
                        self._preempt(v)
                        if v is r:
                            break
                if r not in alive:
                    continue
            k += 1
        self.running = alive
        self.step_no += 1


def run(sched: Scheduler, width: int, max_steps: int = 1 << 30):
    """Yield (plan, counters after the update) for every step until all requests finish."""
    while not sched.done() and sched.step_no < max_steps:
        plan = sched.schedule(width)
        sched.update()
        yield plan, sched.counters()
