"""The scheduler oracle against traces worked out by hand from the engine loop of
"Continuous Batching" ("4. Tiny example", the Go Engine.Step and preempt), and
against invariants on random and full-size traces. Beyond these the scheduler is
parity unpinned: the pages print no trace of the loop."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import scheduler as osch

P, D = osch.PREFILL, osch.DECODE


def _rows(plan):
    return [(int(i), int(s), int(q), int(L)) for i, s, q, L in zip(plan.ids, plan.stages, plan.q_lens,
                                                                    plan.seq_lens)]


def test_hand_worked_trace_without_preemption():
    # block 4, pool 6, at most 2 running; A(arrive 0, prompt 5, 3 outputs),
    # B(0, 6, 4), C(1, 2, 2). Worked by hand:
    #  step 0: admit A (2 blocks) and B (2 blocks), free 2; both prefill. A: 6 <= 8, B: 7 <= 8
    #  step 1: C arrives, running is full; A decode L6, B decode L7
    #  step 2: A decode L7 -> 3rd output, finished, frees 2 (free 4); B decode L8 -> needs
    #          9 > 8 tokens, grows to 3 blocks (free 3)
    #  step 3: admit C (1 block, free 2); B decode L9 -> finished, frees 3 (free 5);
    #          C prefill q2 L2
    #  step 4: C decode L3 -> finished (free 6)
    s = osch.Scheduler([0, 0, 1], [5, 6, 2], [3, 4, 2], 6, None, 4, 2)
    got = list(osch.run(s, width=4))
    want_rows = [
        [(0, P, 5, 5), (1, P, 6, 6)],
        [(0, D, 1, 6), (1, D, 1, 7)],
        [(0, D, 1, 7), (1, D, 1, 8)],
        [(1, D, 1, 9), (2, P, 2, 2)],
        [(2, D, 1, 3)],
    ]
    want_after = [  # (free, running, waiting, preempted, finished) after each step's update
        (2, 2, 0, 0, 0), (2, 2, 1, 0, 0), (3, 1, 1, 0, 1), (5, 1, 0, 0, 2), (6, 0, 0, 0, 3)]
    assert [_rows(p) for p, _ in got] == want_rows
    assert [tuple(c.values()) for _, c in got] == want_after
    assert [r.finished_step for r in s.reqs] == [2, 3, 4]


def test_hand_worked_trace_with_preemption_and_block_ids():
    # block 4, pool 3 (free list 0,1,2: pops from the end), up to 4 running;
    # A(0, prompt 4, 3 outputs), B(0, 4, 3), C(0, 3, 1). Worked by hand:
    #  step 0: admit A [2], B [1], C [0]; free 0. Update in order: A needs 5 > 4 tokens,
    #          no block -> preempted: frees [2], goes to the front of the queue; B needs a
    #          block -> gets 2 -> [1, 2]; C reaches 1 output -> finished, frees [0].
    #  step 1: A needs ceil(5/4) = 2 blocks, 1 free -> not admitted; B decode L5
    #  step 2: A still waits; B decode L6 -> finished, frees [1, 2] (free list 0, 1, 2)
    #  step 3: admit A: pops 2, 1 -> table [2, 1]; prefill of prompt + 1 output = 5 tokens
    #          at slots 8, 9, 10, 11 (block 2) and 4 (block 1)
    #  step 4: A decode L6 at position 5 -> slot 5; 3rd output -> finished
    s = osch.Scheduler([0, 0, 0], [4, 4, 3], [3, 3, 1], 3, [0, 1, 2], 4, 4)
    got = list(osch.run(s, width=2))
    assert [_rows(p) for p, _ in got] == [
        [(0, P, 4, 4), (1, P, 4, 4), (2, P, 3, 3)],
        [(1, D, 1, 5)],
        [(1, D, 1, 6)],
        [(0, P, 5, 5)],
        [(0, D, 1, 6)],
    ]
    assert [tuple(c.values()) for _, c in got] == [
        (1, 1, 1, 1, 1), (1, 1, 1, 1, 1), (3, 0, 1, 1, 2), (1, 1, 0, 1, 2), (3, 0, 0, 1, 3)]
    p0 = got[0][0]
    assert p0.block_tables.tolist() == [[2, -1], [1, -1], [0, -1]]
    assert p0.slot_mapping.tolist() == [8, 9, 10, 11, 4, 5, 6, 7, 0, 1, 2]
    p1 = got[1][0]
    assert p1.block_tables.tolist() == [[1, 2]] and p1.slot_mapping.tolist() == [8]
    p3 = got[3][0]
    assert p3.block_tables.tolist() == [[2, 1]] and p3.slot_mapping.tolist() == [8, 9, 10, 11, 4]
    assert got[4][0].slot_mapping.tolist() == [5]
    assert s.reqs[0].preempted == 1


def test_preempted_requests_go_to_the_front_last_one_first():
    # pool 3 (free list 0,1,2), block 4; three requests of prompt 4 fill it. Update:
    # request 0 cannot grow -> preempted (frees [2]); request 1 grows into block 2;
    # request 2 cannot grow -> preempted (frees [0]) and pushed in front of request 0.
    s = osch.Scheduler([0, 0, 0, 1], [4, 4, 4, 1], [5, 5, 5, 1], 3, [0, 1, 2], 4, 4)
    plan = s.schedule(4)
    assert _rows(plan) == [(0, P, 4, 4), (1, P, 4, 4), (2, P, 4, 4)]
    s.update()
    assert [r.rid for r in s.waiting] == [2, 0]
    assert s.tables.tables == {1: [1, 2]}
    assert s.counters() == {"free": 1, "running": 1, "waiting": 2, "preempted": 2, "finished": 0}
    plan = s.schedule(4)   # request 3 arrives behind them; the head (2) needs 2 blocks, 1 free
    assert _rows(plan) == [(1, D, 1, 5)] and [r.rid for r in s.waiting] == [2, 0, 3]


def _check_invariants(tr, max_steps=200000):
    s = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                       tr.max_running)
    width = -(-int((tr.prompt + tr.max_tokens).max()) // tr.block_size)
    admitted_fresh = []
    seen_pending = False
    for plan, after in osch.run(s, width, max_steps):
        s.tables.check()                                          # conservation + uniqueness
        assert after["running"] <= tr.max_running
        assert len(plan.ids) <= tr.max_running
        used = sum(len(t) for t in s.tables.tables.values())
        assert after["free"] + used == tr.num_blocks
        for i, st_, q, L in _rows(plan):
            r = s.reqs[i]
            if st_ == P:
                assert q == L and q >= r.prompt                   # re-prefill includes outputs
                if q == r.prompt:
                    admitted_fresh.append(i)
            else:
                assert q == 1
        assert len(np.unique(plan.slot_mapping)) == len(plan.slot_mapping)
        assert (plan.slot_mapping >= 0).all() and (plan.slot_mapping < tr.num_blocks * tr.block_size).all()
        seen_pending |= after["waiting"] > 0
    assert s.done()
    assert all(r.n_out == r.max_tokens for r in s.reqs)           # exact output counts
    assert s.pool.num_free == tr.num_blocks and not s.tables.tables   # nothing leaked
    # first admissions follow arrival order (preempted requests re-enter at the front,
    # which never lets a later arrival start before an earlier one)
    assert admitted_fresh == sorted(admitted_fresh, key=lambda i: (tr.arrival[i], i))
    return s, seen_pending


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(3, 40), st.integers(1, 8))
def test_invariants_on_random_small_traces(seed, pool, max_running):
    tr = workloads.small_trace(seed, 25, max(pool, 20), block_size=4, max_running=max_running,
                               prompt_max=40, out_max=30, rate=2.0)
    _check_invariants(tr)


def test_small_pool_leaves_requests_waiting_and_still_completes_all():
    # the tiny-pool behaviours of the pure-Python engine's tests ("Running and Testing It"):
    # with too few blocks requests wait; an undersized pool still completes every request
    tr = workloads.small_trace(7, 10, 20, block_size=4, max_running=8, prompt_max=30, out_max=40, rate=5.0)
    s, pending = _check_invariants(tr)
    assert pending and s.preemptions > 0


def test_config5_trace_preempts_and_finishes_every_request():
    tr = workloads.config5()
    s, pending = _check_invariants(tr)
    assert s.preemptions > 0 and pending
    assert s.finished == 2000
