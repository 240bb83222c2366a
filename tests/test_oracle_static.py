"""Static batching in the scheduler oracle, the baseline continuous batching is measured
against ("Continuous Batching", "1. What is it?" and "2. Why does it exist?": finished
sequences hold their slots until the longest one finishes, new requests wait for the
whole batch). Pinned by a hand-worked trace and invariants on random and full traces."""
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


def test_hand_worked_static_batch_waits_for_its_longest_member():
    # ample pool, block 4, 2 slots; A(0, prompt 2, 1 output), B(0, 2, 3), C(1, 3, 1)
    #  continuous: step 0 A, B prefill (A finishes); step 1 C joins B's decode
    #  static: C waits until B has finished (step 2), then runs alone
    s = osch.Scheduler([0, 0, 1], [2, 2, 3], [1, 3, 1], 16, None, 4, 2)
    assert [_rows(p) for p, _ in osch.run(s, 2)] == [
        [(0, P, 2, 2), (1, P, 2, 2)],
        [(1, D, 1, 3), (2, P, 3, 3)],
        [(1, D, 1, 4)],
    ]
    s = osch.Scheduler([0, 0, 1], [2, 2, 3], [1, 3, 1], 16, None, 4, 2, static=True)
    assert [_rows(p) for p, _ in osch.run(s, 2)] == [
        [(0, P, 2, 2), (1, P, 2, 2)],
        [(1, D, 1, 3)],
        [(1, D, 1, 4)],
        [(2, P, 3, 3)],
    ]


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(3, 40), st.integers(1, 8), st.booleans())
def test_static_invariants_on_random_small_traces(seed, pool, max_running, swap):
    tr = workloads.small_trace(seed, 25, max(pool, 20), block_size=4, max_running=max_running, prompt_max=40,
                               out_max=30, rate=2.0)
    s = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                       tr.max_running, static=True, swap_blocks=16 if swap else 0)
    width = -(-int((tr.prompt + tr.max_tokens).max()) // tr.block_size)
    while not s.done():
        before = {r.rid for r in s.running}
        plan = s.schedule(width)
        joined = {r.rid for r in s.running} - before
        assert not joined or not before               # admission only into an empty batch
        s.update()
    assert all(r.n_out == r.max_tokens for r in s.reqs)
    _simulate(tr, static=True, swap_blocks=16 if swap else 0)     # every row reads its own K/V


def test_config5_static_runs_longer_with_a_smaller_batch():
    tr = workloads.config5()
    cont = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                          tr.max_running)
    stat = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                          tr.max_running, static=True)
    rows_c = [len(p.ids) for p, _ in osch.run(cont, 512)]
    rows_s = [len(p.ids) for p, _ in osch.run(stat, 512)]
    assert stat.finished == cont.finished == 2000
    assert len(rows_s) > len(rows_c) and np.mean(rows_s) < np.mean(rows_c)

