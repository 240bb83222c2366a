"""Preemption by swap in the oracle ("Continuous Batching", "5. Technical explanation",
Preemption, the SWAP strategy): the block copies (oracle/swap.py) against a hand-worked
layout, a round trip and untouched blocks; the scheduler against a trace worked out by
hand, the fall-back to recompute when the host space is short, and a simulation of the
cache with position tags on random and full traces, which checks that every row finds,
through its block table, exactly its own K/V for every earlier position after any
number of swap-outs and swap-ins (freed blocks are poisoned every step)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import scheduler as osch
from oracle import swap as osw

P, D = osch.PREFILL, osch.DECODE


def _rows(plan):
    return [(int(i), int(s), int(q), int(L)) for i, s, q, L in zip(plan.ids, plan.stages, plan.q_lens,
                                                                    plan.seq_lens)]


def test_host_layout_hand_worked():
    # 2 layers, 3 blocks of 1 token, 1 head of 2 elements: K[l, b] = (100 l + 10 b, +1),
    # V = K + 1000; host block h holds layer 0 K, layer 0 V, layer 1 K, layer 1 V
    k = np.zeros((2, 3, 1, 1, 2), np.int64)
    for l in range(2):
        for b in range(3):
            k[l, b, 0, 0] = [100 * l + 10 * b, 100 * l + 10 * b + 1]
    v = k + 1000
    host = np.full(osw.host_shape(2, k), -1, np.int64)
    osw.swap_out(k, v, [(2, 0), (0, 1)], host)
    assert host[0].ravel().tolist() == [20, 21, 1020, 1021, 120, 121, 1120, 1121]
    assert host[1].ravel().tolist() == [0, 1, 1000, 1001, 100, 101, 1100, 1101]


def test_round_trip_through_other_blocks_and_untouched_blocks():
    rng = np.random.default_rng(3)
    k = rng.integers(0, 256, (3, 8, 4, 2, 16), dtype=np.uint8)
    v = rng.integers(0, 256, k.shape, dtype=np.uint8)
    k0, v0 = k.copy(), v.copy()
    host = rng.integers(0, 256, osw.host_shape(5, k), dtype=np.uint8)
    h0 = host.copy()
    osw.swap_out(k, v, [(6, 4), (1, 0), (3, 2)], host)
    assert (k == k0).all() and (v == v0).all()                     # a swap-out reads only
    assert (host[[1, 3]] == h0[[1, 3]]).all()                        # host blocks no pair names
    osw.swap_in(host, [(4, 0), (0, 7), (2, 5)], k, v)
    for src, dst in ((6, 0), (1, 7), (3, 5)):
        assert (k[:, dst] == k0[:, src]).all() and (v[:, dst] == v0[:, src]).all()
    others = [b for b in range(8) if b not in (0, 7, 5)]
    assert (k[:, others] == k0[:, others]).all() and (v[:, others] == v0[:, others]).all()


def test_hand_worked_trace_with_swap():
    # the recompute trace of the scheduler tests with a host space of 4 blocks: block 4,
    # pool 3 (free list 0,1,2), up to 4 running; A(0, prompt 4, 3 outputs), B(0, 4, 3),
    # C(0, 3, 1).
    #  step 0: admit A [2], B [1], C [0]. Update: A cannot grow -> swapped out: device 2 to
    #          host 3 (host free list 0..3 popped from the end), frees [2]; B grows into 2;
    #          C finishes, frees [0]
    #  step 1-2: A needs 2 blocks, 1 free; B decodes and finishes at step 2 (frees 1, 2)
    #  step 3: A admitted: table [2, 1]; host 3 -> device 2; host 3 freed; A resumes with a
    #          decode row at position 4 (slot 4, block 1), no prefill
    #  step 4: A decodes position 5 and finishes
    s = osch.Scheduler([0, 0, 0], [4, 4, 3], [3, 3, 1], 3, [0, 1, 2], 4, 4, swap_blocks=4)
    got = []
    for plan, after in osch.run(s, width=2):
        got.append((_rows(plan), plan.swap_in, list(s.swap_out), plan.slot_mapping.tolist(), after))
    assert [g[0] for g in got] == [
        [(0, P, 4, 4), (1, P, 4, 4), (2, P, 3, 3)],
        [(1, D, 1, 5)],
        [(1, D, 1, 6)],
        [(0, D, 1, 5)],
        [(0, D, 1, 6)],
    ]
    assert [g[1] for g in got] == [[], [], [], [(3, 2)], []]
    assert [g[2] for g in got] == [[(2, 3)], [], [], [], []]
    assert got[3][3] == [4] and got[4][3] == [5]
    assert [(a["swapped_out"], a["blocks_out"], a["blocks_in"]) for *_, a in got] == [
        (1, 1, 0), (1, 1, 0), (1, 1, 0), (1, 1, 1), (1, 1, 1)]
    assert s.host.num_free == 4 and s.pool.num_free == 3


def test_short_host_space_falls_back_to_recompute():
    # A holds 2 blocks when it cannot grow; a host space of 1 block cannot take it
    s = osch.Scheduler([0, 0], [8, 4], [3, 3], 3, [0, 1, 2], 4, 4, swap_blocks=1)
    s.schedule(2)
    s.update()                                  # A: 9 > 8 tokens, no block -> preempted
    assert s.swap_out == [] and s.counters()["swapped_out"] == 0 and s.preemptions == 1
    assert s.waiting[0].rid == 0 and s.waiting[0].host is None
    for _ in range(10):
        if s.done():
            break
        plan = s.schedule(3)
        if 0 in plan.ids.tolist():
            k = plan.ids.tolist().index(0)
            assert plan.stages[k] == P and plan.q_lens[k] == 9   # re-prefill of prompt + output
            break
        s.update()


def test_negative_swap_space_rejected():
    with pytest.raises(ValueError):
        osch.Scheduler([0], [1], [1], 4, None, 4, 1, swap_blocks=-1)


def _simulate(tr, max_steps=10 ** 6, check_every=1, **kw):
    """Run the scheduler over a tag cache: every slot holds (request, position) of the
    token written there; swap copies move the tags; blocks held by no table are
    poisoned after every update. Every row must see its own tags at positions 0..L-1
    (checked at every check_every-th step for all rows, at every step for the rows of
    requests that were ever preempted)."""
    s = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                       tr.max_running, **kw)
    bs = tr.block_size
    width = -(-int((tr.prompt + tr.max_tokens).max()) // bs)
    cache = np.full((tr.num_blocks, bs, 2), -1, np.int64)
    host = None if s.host is None else np.full((s.host.num_blocks, bs, 2), -1, np.int64)
    prefill_tokens = 0
    while not s.done():
        assert s.step_no < max_steps
        plan = s.schedule(width)
        for h, b in plan.swap_in:               # before the step's attention
            cache[b] = host[h]
        cu = plan.cu_seqlens_q
        for k, (i, st_, q, L) in enumerate(_rows(plan)):
            slots = plan.slot_mapping[cu[k]:cu[k + 1]]
            cache.reshape(-1, 2)[slots] = np.stack([np.full(q, i), np.arange(L - q, L)], 1)
            if st_ == P:
                prefill_tokens += q
        full = plan.step % check_every == 0
        for k, (i, st_, q, L) in enumerate(_rows(plan)):
            if not full and s.reqs[i].preempted == 0:
                continue
            pos = np.arange(L)
            seen = cache[plan.block_tables[k][pos // bs], pos % bs]
            assert (seen[:, 0] == i).all() and (seen[:, 1] == pos).all(), f"step {plan.step} request {i}"
        s.update()
        for b, h in s.swap_out:                 # before the next step's kernels
            host[h] = cache[b]
        held = np.zeros(tr.num_blocks, bool)
        for t in s.tables.tables.values():
            held[t] = True
        cache[~held] = -7                       # freed blocks lose their contents
        if host is not None:                    # and so do free host blocks
            hheld = np.zeros(len(host), bool)
            for r in s.waiting:
                if r.host is not None:
                    hheld[r.host] = True
            assert int(hheld.sum()) + s.host.num_free == len(host)       # host blocks conserved
            host[~hheld] = -9
    assert all(r.n_out == r.max_tokens for r in s.reqs)
    assert s.pool.num_free == tr.num_blocks and not s.tables.tables
    if s.host is not None:
        assert s.host.num_free == s.host.num_blocks
    return s, prefill_tokens


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(3, 40), st.integers(1, 8), st.sampled_from([0, 1, 4, 16, 200]),
       st.sampled_from([(0, 0), (8, 4), (3, 0)]))
def test_tag_simulation_on_random_small_traces(seed, pool, max_running, swap_blocks, budget):
    tr = workloads.small_trace(seed, 25, max(pool, 20), block_size=4, max_running=max_running, prompt_max=40,
                               out_max=30, rate=2.0)
    s, pre = _simulate(tr, swap_blocks=swap_blocks, max_batched_tokens=budget[0], chunk_tokens=budget[1])
    c = s.counters()
    if swap_blocks:
        assert c["blocks_in"] == c["blocks_out"]                   # every swap-out came back
        if swap_blocks >= tr.num_blocks:
            assert c["swapped_out"] == s.preemptions               # the host always had room


def test_swap_saves_the_recompute_prefill_on_a_small_pool():
    tr = workloads.small_trace(7, 10, 20, block_size=4, max_running=8, prompt_max=30, out_max=40, rate=5.0)
    s_rc, pre_rc = _simulate(tr)
    s_sw, pre_sw = _simulate(tr, swap_blocks=64)
    assert s_rc.preemptions > 0 and s_sw.counters()["swapped_out"] == s_sw.preemptions > 0
    assert pre_sw == int(tr.prompt.sum())                          # only the first prefills
    assert pre_rc > pre_sw


def test_config5_trace_with_swap():
    tr = workloads.config5()
    s, pre = _simulate(tr, swap_blocks=4096, check_every=16)
    c = s.counters()
    assert c["swapped_out"] == s.preemptions > 0 and c["blocks_in"] == c["blocks_out"]
    assert pre == int(tr.prompt.sum())
