"""Scheduler policy variants in the oracle ("Continuous Batching", "5. Technical
explanation": LIFO victim selection and priority admission; the pure-Python engine's
preemption of the request with the fewest generated tokens): traces worked out by hand
where each policy picks a different victim, priority order in the queue, a regression
(equal classes on an ample pool change nothing), and the tag simulation of the cache
with every combination of victim policy, swap, chunked prefill and priorities."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import scheduler as osch
from test_oracle_swap import _simulate

P, D = osch.PREFILL, osch.DECODE


def _rows(plan):
    return [(int(i), int(s), int(q), int(L)) for i, s, q, L in zip(plan.ids, plan.stages, plan.q_lens,
                                                                    plan.seq_lens)]


def _three(victim, **kw):
    # block 4, pool 4 (free list 0..3 popped from the end), up to 4 running;
    # A(0, prompt 4, 3 outputs), B(0, 4, 3), C(0, 3, 5)
    return osch.Scheduler([0, 0, 0], [4, 4, 3], [3, 3, 5], 4, [0, 1, 2, 3], 4, 4, victim=victim, **kw)


def test_hand_worked_victims_differ():
    # step 0: A [3], B [2], C [1] admitted, free [0]; every row yields its first output.
    #  self (one pass): A grows into 0; B finds no block and preempts itself (frees 2);
    #        C needs 4 <= 4 tokens: running A, C; waiting B
    #  lifo: A grows into 0; B finds no block: the last admitted (C) is preempted (frees
    #        1) and B grows into 1: running A, B; waiting C
    #  fewest: all have one output; the earliest admitted (A, already grown) is
    #        preempted (frees 3, 0) and B grows into 0: running B, C; waiting A
    want = {"self": ([0, 2], [1], {0: [3, 0], 2: [1]}), "lifo": ([0, 1], [2], {0: [3, 0], 1: [2, 1]}),
            "fewest": ([1, 2], [0], {1: [2, 0], 2: [1]})}
    for victim, (run_ids, wait_ids, tables) in want.items():
        s = _three(victim)
        assert _rows(s.schedule(2)) == [(0, P, 4, 4), (1, P, 4, 4), (2, P, 3, 3)]
        s.update()
        assert [r.rid for r in s.running] == run_ids, victim
        assert [r.rid for r in s.waiting] == wait_ids, victim
        assert s.tables.tables == tables, victim
        assert s.preemptions == 1
        while not s.done():                     # and the trace still completes
            s.schedule(3)
            s.update()
        assert all(r.n_out == r.max_tokens for r in s.reqs)


def test_lifo_victims_are_the_last_admitted_oldest_ends_in_front():
    # block 4, pool 5; A(0, prompt 8, 3), B(0, 4, 3), C(0, 4, 3), D(0, 1, 9) fill it.
    # Step 0: A [4, 3], B [2], C [1], D [0]. Update: A needs 9 > 8 tokens, no block: the
    # last admitted, D, is preempted and A takes its block 0; B needs 5 > 4: C (now the
    # last) is preempted and B takes block 1. Each victim goes to the front: queue C, D.
    s = osch.Scheduler([0, 0, 0, 0], [8, 4, 4, 1], [3, 3, 3, 9], 5, [0, 1, 2, 3, 4], 4, 4, victim="lifo")
    s.schedule(2)
    s.update()
    assert [r.rid for r in s.running] == [0, 1] and [r.rid for r in s.waiting] == [2, 3]
    assert s.tables.tables == {0: [4, 3, 0], 1: [2, 1]} and s.preemptions == 2


def test_priority_queue_order_and_premium_preempts_bulk():
    # A(0, class 1), B(1, class 1), C(2, class 0) with one running slot: C overtakes B
    s = osch.Scheduler([0, 1, 2], [2, 2, 2], [4, 1, 1], 16, None, 4, 1, priority=[1, 1, 0])
    order = []
    while not s.done():
        p = s.schedule(2)
        order += [int(i) for i, st_ in zip(p.ids, p.stages) if st_ == P]
        s.update()
    assert order == [0, 2, 1]
    # the same without classes keeps arrival order
    s = osch.Scheduler([0, 1, 2], [2, 2, 2], [4, 1, 1], 16, None, 4, 1)
    order = []
    while not s.done():
        p = s.schedule(2)
        order += [int(i) for i, st_ in zip(p.ids, p.stages) if st_ == P]
        s.update()
    assert order == [0, 1, 2]
    # pool 2, block 4: bulk A(0, prompt 4, 5 outputs) and premium B(0, 4, 5) each hold a
    # block; both need a second one. lifo among the least important class: A (bulk) is
    # the victim even though B was admitted last
    s = osch.Scheduler([0, 0], [4, 4], [5, 5], 2, [0, 1], 4, 2, victim="lifo", priority=[1, 0])
    s.schedule(2)
    s.update()
    assert [r.rid for r in s.running] == [1] and [r.rid for r in s.waiting] == [0]


def test_preempted_request_takes_its_place_by_key():
    # pool 2 (free list 0, 1), block 4: A(0, prompt 4, 3 outputs, class 1) [1] and
    # B(0, 4, 3, class 1) [0]. Update: A cannot grow and preempts itself (frees 1), B
    # grows into 1. Step 1: C(1, prompt 4, class 0) arrives and is queued ahead of A; it
    # does not fit (no free block), so the queue stays C, A. Without classes A would be
    # at the front, C behind it.
    for prio, want in (([1, 1, 0], [2, 0]), (None, [0, 2])):
        s = osch.Scheduler([0, 0, 1], [4, 4, 4], [3, 3, 1], 2, [0, 1], 4, 4, priority=prio)
        s.schedule(2)
        s.update()
        assert s.tables.tables == {1: [0, 1]}
        p = s.schedule(2)
        assert _rows(p) == [(1, D, 1, 5)]
        assert [r.rid for r in s.waiting] == want


def test_equal_classes_on_an_ample_pool_change_nothing():
    tr = workloads.small_trace(3, 25, 400, block_size=4, max_running=4, prompt_max=40, out_max=30, rate=2.0)
    args = (tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size, tr.max_running)
    a = [(_rows(p), c) for p, c in osch.run(osch.Scheduler(*args), 20)]
    for kw in ({"priority": [0] * 25}, {"victim": "lifo"}, {"victim": "fewest", "priority": [0] * 25}):
        b = [(_rows(p), c) for p, c in osch.run(osch.Scheduler(*args, **kw), 20)]
        assert a == b, kw


def test_bad_policy_arguments():
    with pytest.raises(ValueError):
        osch.Scheduler([0], [1], [1], 4, None, 4, 1, victim="oldest")
    with pytest.raises(ValueError):
        osch.Scheduler([0, 0], [1, 1], [1, 1], 4, None, 4, 1, priority=[0])
    with pytest.raises(ValueError):
        osch.Scheduler([0], [1], [1], 4, None, 4, 1, priority=[-1])


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10_000), st.integers(3, 40), st.integers(1, 8), st.sampled_from(["self", "lifo", "fewest"]),
       st.sampled_from([0, 16, 200]), st.sampled_from([(0, 0), (8, 4)]), st.booleans())
def test_tag_simulation_with_policies(seed, pool, max_running, victim, swap_blocks, budget, prio):
    tr = workloads.small_trace(seed, 25, max(pool, 20), block_size=4, max_running=max_running, prompt_max=40,
                               out_max=30, rate=2.0)
    classes = list(np.random.default_rng(seed).integers(0, 3, 25)) if prio else None
    _simulate(tr, victim=victim, swap_blocks=swap_blocks, max_batched_tokens=budget[0], chunk_tokens=budget[1],
              priority=classes)


@pytest.mark.parametrize("victim", ["lifo", "fewest"])
def test_config5_trace_with_victim_policy(victim):
    tr = workloads.config5()
    s, pre = _simulate(tr, victim=victim, check_every=16)
    assert s.preemptions > 0 and s.finished == 2000
