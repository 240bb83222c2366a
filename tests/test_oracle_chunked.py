"""Chunked prefill under a per-step token budget in the scheduler oracle ("Continuous
Batching", "5. Technical explanation": mixed batching, where a long prompt is split into
chunks that ride along with the decode rows of a step, and the serving setting that caps
the tokens batched per iteration). Pinned by a trace worked out by hand, by the
no-budget regression (a budget that never binds changes nothing) and by invariants on
random traces: the budget, the chunk bound, greedy running-order allocation,
contiguous chunks, one output per completed row, exact output counts, no leak."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import scheduler as osch

P, D = osch.PREFILL, osch.DECODE


def _rows(plan):
    return [(int(i), int(s), int(q), int(L)) for i, s, q, L in zip(plan.ids, plan.stages, plan.q_lens,
                                                                    plan.seq_lens)]


def test_hand_worked_trace_budget_6_chunk_4():
    # block 4, pool 16 (free list 0..15 popped from the end), up to 4 running, at most 6
    # new tokens per step in chunks of at most 4; A(arrive 0, prompt 10, 2 outputs),
    # B(0, 3, 3), C(1, 5, 1). Worked by hand:
    #  step 0: admit A (blocks 15 14 13) and B (12); budget 6: A 4 (0..3), B 2 (0..1)
    #  step 1: admit C (11 10); budget 6: A 4 (4..7), B 1 (2; completes: 1st output),
    #          C 1 (0)
    #  step 2: B decodes; budget 5: A 2 (8..9; completes), C 3 (1..3). B's 2nd output
    #          needs 5 tokens: grows into block 9
    #  step 3: A and B decode (both finish); budget 4: C 1 (4; completes and finishes)
    s = osch.Scheduler([0, 0, 1], [10, 3, 5], [2, 3, 1], 16, None, 4, 4, max_batched_tokens=6, chunk_tokens=4)
    got = list(osch.run(s, width=3))
    assert [_rows(p) for p, _ in got] == [
        [(0, P, 4, 4), (1, P, 2, 2)],
        [(0, P, 4, 8), (1, P, 1, 3), (2, P, 1, 1)],
        [(0, P, 2, 10), (1, D, 1, 4), (2, P, 3, 4)],
        [(0, D, 1, 11), (1, D, 1, 5), (2, P, 1, 5)],
    ]
    assert [p.slot_mapping.tolist() for p, _ in got] == [
        [60, 61, 62, 63, 48, 49],
        [56, 57, 58, 59, 50, 44],
        [52, 53, 51, 45, 46, 47],
        [54, 36, 40],
    ]
    # a row's table lists the blocks its seq_len covers: C's second block is not yet in use
    assert got[2][0].block_tables.tolist() == [[15, 14, 13], [12, -1, -1], [11, -1, -1]]
    assert [tuple(c.values()) for _, c in got] == [
        (12, 2, 0, 0, 0), (10, 3, 0, 0, 0), (9, 3, 0, 0, 0), (16, 0, 0, 0, 3)]
    assert [r.finished_step for r in s.reqs] == [3, 3, 3]


def test_request_without_budget_gets_no_row_and_waits_its_turn():
    # budget 4, two decoding requests take 2; the prefill of the third gets 2 tokens a step
    s = osch.Scheduler([0, 0, 1], [1, 1, 6], [4, 4, 1], 8, None, 4, 4, max_batched_tokens=4)
    got = [_rows(p) for p, _ in osch.run(s, width=2)]
    assert got[0] == [(0, P, 1, 1), (1, P, 1, 1)]
    assert got[1] == [(0, D, 1, 2), (1, D, 1, 2), (2, P, 2, 2)]
    assert got[2] == [(0, D, 1, 3), (1, D, 1, 3), (2, P, 2, 4)]
    assert got[3] == [(0, D, 1, 4), (1, D, 1, 4), (2, P, 2, 6)]
    assert len(got) == 4 and s.done()


def test_more_decode_rows_than_budget_still_all_decode():
    # decode rows are never cut: three decoding requests and a budget of 2 leave the
    # waiting prefill without a row until a decode finishes
    s = osch.Scheduler([0, 0, 0, 1], [1, 1, 1, 3], [3, 3, 3, 1], 8, None, 4, 4, max_batched_tokens=2)
    got = [_rows(p) for p, _ in osch.run(s, width=1)]
    assert got[0] == [(0, P, 1, 1), (1, P, 1, 1)]                  # budget 2: the third waits
    assert got[1] == [(0, D, 1, 2), (1, D, 1, 2)]                  # 2 decodes use the budget
    assert got[2] == [(0, D, 1, 3), (1, D, 1, 3)]                  # both finish here
    assert got[3] == [(2, P, 1, 1), (3, P, 1, 1)]                  # budget 2 again: 1 + 1
    assert got[4] == [(2, D, 1, 2), (3, P, 1, 2)]
    assert got[5] == [(2, D, 1, 3), (3, P, 1, 3)]
    assert len(got) == 6 and s.done()


def _plans(s, width, steps=200000):
    return [(_rows(p), p.slot_mapping.tolist(), p.block_tables.tolist(), tuple(c.items()))
            for p, c in osch.run(s, width, steps)]


def _sched(tr, prefix=False, **kw):
    toks = [tr.prompt_tokens(i) for i in range(len(tr.prompt))] if prefix else None
    return osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                          tr.max_running, prompt_tokens=toks, **kw)


def _width(tr):
    return -(-int((tr.prompt + tr.max_tokens).max()) // tr.block_size)


@settings(max_examples=20, deadline=None)
@given(st.integers(0, 10_000), st.integers(20, 40), st.integers(1, 8), st.booleans())
def test_budget_that_never_binds_changes_nothing(seed, pool, max_running, prefix):
    tr = workloads.small_trace(seed, 20, pool, block_size=4, max_running=max_running, prompt_max=40,
                               out_max=20, rate=2.0, groups=3 if prefix else 0)
    big = int(tr.prompt.max() + tr.max_tokens.max()) * (max_running + 1)
    plain = _plans(_sched(tr, prefix), _width(tr))
    assert _plans(_sched(tr, prefix, max_batched_tokens=big), _width(tr)) == plain
    assert _plans(_sched(tr, prefix, chunk_tokens=big), _width(tr)) == plain


def _check_chunked(tr, budget, chunk, prefix=False, max_steps=200000):
    s = _sched(tr, prefix, max_batched_tokens=budget, chunk_tokens=chunk)
    width = _width(tr)
    nxt = {}                                    # request -> next prefill position
    outputs = 0
    while not s.done():
        assert s.step_no < max_steps
        n_out_before = {r.rid: r.n_out for r in s.reqs}
        plan = s.schedule(width)
        run_ids = [r.rid for r in s.running]
        rows = _rows(plan)
        by_id = {i: (st_, q, L) for i, st_, q, L in rows}
        # every decoding request has its row; rows keep running order
        decoding = [r.rid for r in s.running if r.stage == D]
        assert [i for i, st_, _, _ in rows if st_ == D] == decoding
        assert [i for i, _, _, _ in rows] == [i for i in run_ids if i in by_id]
        # the budget, the chunk bound, and greedy allocation in running order
        pre = [(i, q, L) for i, st_, q, L in rows if st_ == P]
        left = None if budget == 0 else max(0, budget - len(decoding))
        if left is not None:
            assert sum(q for _, q, _ in pre) <= left
        cut = False
        for r in s.running:
            if r.stage != P:
                continue
            want = r.prompt + r.n_out - (nxt[r.rid] if r.rid in nxt else r.cached)
            if chunk:
                want = min(want, chunk)
            got = by_id[r.rid][1] if r.rid in by_id else 0
            assert 0 <= got <= want
            if cut:
                assert got == 0                 # once one prefill is cut, later ones get nothing
            if got < want:
                cut = True
                assert left is not None and sum(q for _, q, _ in pre) == left   # budget used up
        # chunks are contiguous: a fresh prefill starts at its cached prefix
        for i, q, L in pre:
            start = L - q
            assert start == nxt.get(i, s.reqs[i].cached)
            nxt[i] = L
        assert len(np.unique(plan.slot_mapping)) == len(plan.slot_mapping)
        s.update()
        s.tables.check()
        gained = [i for i in n_out_before if s.reqs[i].n_out != n_out_before[i]]
        for i in gained:
            assert s.reqs[i].n_out == n_out_before[i] + 1 and i in by_id
            st_, q, L = by_id[i]
            if st_ == P:                          # an output only when the prefill is complete
                assert L == s.reqs[i].prompt + n_out_before[i]
                del nxt[i]
        for i, (st_, q, L) in by_id.items():
            if st_ == P and i not in gained:
                assert L < s.reqs[i].prompt + n_out_before[i]
        outputs += len(gained)
    assert all(r.n_out == r.max_tokens for r in s.reqs)
    assert outputs == int(tr.max_tokens.sum())
    assert s.pool.num_free == tr.num_blocks and not s.tables.tables
    return s


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(3, 40), st.integers(1, 8), st.sampled_from([0, 1, 3, 8, 24]),
       st.sampled_from([0, 1, 4, 16]), st.booleans())
def test_invariants_on_random_small_traces(seed, pool, max_running, budget, chunk, prefix):
    tr = workloads.small_trace(seed, 25, max(pool, 20), block_size=4, max_running=max_running, prompt_max=40,
                               out_max=30, rate=2.0, groups=3 if prefix else 0)
    _check_chunked(tr, budget, chunk, prefix)


def test_config5_trace_with_budget_2048_chunk_512():
    s = _check_chunked(workloads.config5(), 2048, 512)
    assert s.finished == 2000 and s.preemptions > 0


def test_negative_budget_rejected():
    with pytest.raises(ValueError):
        osch.Scheduler([0], [1], [1], 4, None, 4, 1, max_batched_tokens=-1)
    with pytest.raises(ValueError):
        osch.Scheduler([0], [1], [1], 4, None, 4, 1, chunk_tokens=-2)
