"""Prefix caching oracle (shared, reference-counted blocks; "Project 17", "Step 8: Prefix
caching"): a trace worked out by hand, a regression against the plain scheduler when no
prefix is shared, and invariants on random traces with shared system prompts."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import allocator as oa
from oracle import prefix as opx
from oracle import scheduler as osch


def test_hand_worked_two_requests_share_two_pages():
    # blocks of 4, pool 0..7 popped from the end; A at step 0 and B at step 1 with the same
    # 9-token prompt, two outputs each
    toks = list(range(100, 109))
    s = osch.Scheduler([0, 1], [9, 9], [2, 2], 8, list(range(8)), 4, 4, prompt_tokens=[toks, toks])
    p0 = s.schedule(4)
    assert p0.ids.tolist() == [0] and p0.q_lens.tolist() == [9] and p0.seq_lens.tolist() == [9]
    assert p0.block_tables.tolist() == [[7, 6, 5, -1]]
    s.update()                                  # A's whole prompt pages [7], [7, 6] are cached
    p1 = s.schedule(4)
    # B finds the 8-token prefix (its last prompt token must be computed): shares 7, 6 and
    # takes 4; its row is one token at position 8
    assert p1.ids.tolist() == [0, 1] and p1.q_lens.tolist() == [1, 1] and p1.seq_lens.tolist() == [10, 9]
    assert p1.block_tables.tolist() == [[7, 6, 5, -1], [7, 6, 4, -1]]
    assert p1.slot_mapping.tolist() == [5 * 4 + 1, 4 * 4 + 0]
    assert s.tables.ref[7] == 2 and s.tables.ref[6] == 2 and s.tables.ref[4] == 1
    assert p1.counters["cached_tokens"] == 8
    s.update()                                  # A finishes: only block 5 drops to zero
    assert s.pool.free == [0, 1, 2, 3, 5]
    p2 = s.schedule(4)
    assert p2.ids.tolist() == [1] and p2.slot_mapping.tolist() == [4 * 4 + 1]
    s.update()                                  # B finishes: 7, 6, 4 freed in table order
    assert s.pool.free == [0, 1, 2, 3, 5, 7, 6, 4] and s.done()
    assert s.pcache.lookup(toks, 8) == (0, [])  # freed pages invalidate the entries


def test_lookup_longest_first_and_limit():
    pool = oa.BlockPool(6)
    t = opx.SharedTables(pool, 2)
    c = opx.PrefixCache(t)
    t.reserve(1, 6)
    c.insert([1, 2, 3, 4, 5, 6], t.tables[1], 6)
    assert c.lookup([1, 2, 3, 4, 5, 6, 7], 7) == (6, t.tables[1][:3])
    assert c.lookup([1, 2, 3, 4, 5, 6, 7], 5) == (4, t.tables[1][:2])      # limit cuts to whole pages
    assert c.lookup([1, 2, 9, 4], 4) == (2, t.tables[1][:1])
    assert c.lookup([9, 2], 2) == (0, [])
    t.share(2, t.tables[1][:2])
    t.release(1)                                # page 3 freed: the 6-token entry is stale
    assert c.lookup([1, 2, 3, 4, 5, 6], 6) == (4, t.tables[2][:2])
    t.check()


def _plans(s, width, steps=10_000):
    out = []
    for plan, after in osch.run(s, width, steps):
        out.append((plan, after))
    return out


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10_000), st.integers(20, 60), st.integers(1, 8))
def test_no_shared_prefix_is_the_plain_scheduler(seed, pool, max_running):
    tr = workloads.small_trace(seed, 25, pool, block_size=4, max_running=max_running, prompt_max=30, out_max=20,
                               rate=2.0)
    toks = [[(r << 8) + i for i in range(int(p))] for r, p in enumerate(tr.prompt)]   # all distinct
    a = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, 4, max_running)
    b = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, 4, max_running,
                       prompt_tokens=toks)
    pa, pb = _plans(a, 20), _plans(b, 20)
    assert len(pa) == len(pb)
    for (x, xa), (y, ya) in zip(pa, pb):
        for f in ("ids", "stages", "q_lens", "seq_lens", "block_tables", "cu_seqlens_q", "slot_mapping"):
            assert (getattr(x, f) == getattr(y, f)).all(), f
        assert ya.pop("cached_tokens") == 0 and xa == ya


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(24, 80), st.integers(1, 8), st.integers(1, 4))
def test_shared_prefix_invariants(seed, pool, max_running, groups):
    tr = workloads.small_trace(seed, 30, pool, block_size=4, max_running=max_running, prompt_max=24, out_max=16,
                               rate=2.0, groups=groups)
    toks = [tr.prompt_tokens(r).tolist() for r in range(tr.num_requests)]
    s = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, 4, max_running,
                       prompt_tokens=toks)
    bs = 4
    for _ in range(5000):
        if s.done():
            break
        plan = s.schedule(40)
        s.tables.check()
        cu = plan.cu_seqlens_q
        for k, (rid, st_, q, L) in enumerate(zip(plan.ids, plan.stages, plan.q_lens, plan.seq_lens)):
            r = s.reqs[int(rid)]
            tab = s.tables.tables[int(rid)]
            if st_ == osch.PREFILL:
                n = L - q                                        # the cached prefix
                assert n % bs == 0 and n <= min(r.prompt, L - 1)
                for j in range(n // bs):
                    assert s.tables.ref[tab[j]] >= 1
            # every written slot lies in a block this row holds alone
            for slot in plan.slot_mapping[cu[k]:cu[k + 1]]:
                assert s.tables.ref[int(slot) // bs] == 1
        s.update()
        s.tables.check()
    assert s.done()
    assert s.pool.num_free == tr.num_blocks and all(x == 0 for x in s.tables.ref)
    assert all(r.n_out == r.max_tokens for r in s.reqs)
