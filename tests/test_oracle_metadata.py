"""Pins for the oracle's block-table / slot-mapping build."""
import numpy as np
import pytest

from oracle.allocator import BlockPool, SeqTables
from oracle.metadata import build_block_table


def append_simulation(pool: BlockPool, n_tokens: int, bs: int):
    """Token-at-a-time growth as in "Step 4: Implement the paged KV cache":
    slot_in_page = length % PAGE_SIZE, a new page at each boundary."""
    table, where = [], []
    for length in range(n_tokens):
        slot_in_page = length % bs
        if slot_in_page == 0:
            table.append(pool.alloc(1)[0])
        where.append((table[-1], slot_in_page))
    return table, where


@pytest.mark.parametrize("bs", [1, 4, 16, 32])
def test_slot_mapping_matches_append_simulation(bs):
    rng = np.random.default_rng(bs)
    lens = [int(x) for x in rng.integers(1, 150, size=7)] + [bs, bs + 1, 2 * bs]
    N = sum(-(-L // bs) for L in lens) + 3
    order = rng.permutation(N)
    # the append simulation grows one page at a time ...
    pool_a = BlockPool(N, order)
    sims = [append_simulation(pool_a, L, bs) for L in lens]
    # ... the same pages, in the same order, reserved whole
    tabs = [t for t, _ in sims]
    W = max(len(t) for t in tabs) + 2
    bt, cu, slots = build_block_table(tabs, lens, lens, bs, W)   # q = L: every token new
    expect = [page * bs + off for _, where in sims for page, off in where]
    assert slots.dtype == np.int64
    assert slots.tolist() == expect
    assert cu.tolist() == [0] + np.cumsum(lens).tolist()
    for s, t in enumerate(tabs):
        assert bt[s, :len(t)].tolist() == t
        assert (bt[s, len(t):] == -1).all()
    assert len(set(expect)) == len(expect)


def test_decode_slots_are_last_position():
    t = SeqTables(BlockPool(16), 4)
    for s, L in enumerate([5, 4, 9]):
        t.reserve(s, L)
    tabs = [t.tables[s] for s in range(3)]
    bt, cu, slots = build_block_table(tabs, [1, 1, 1], [5, 4, 9], 4, 4)
    assert cu.tolist() == [0, 1, 2, 3]
    # position L-1 lives in block (L-1)//4 at offset (L-1)%4
    assert slots.tolist() == [tabs[0][1] * 4 + 0, tabs[1][0] * 4 + 3, tabs[2][2] * 4 + 0]


def test_prefill_chunk_with_cached_prefix():
    t = SeqTables(BlockPool(16, list(range(15, -1, -1))), 4)
    t.reserve(0, 10)
    tab = t.tables[0]
    bt, cu, slots = build_block_table([tab], [3], [10], 4, 3)
    assert slots.tolist() == [tab[1] * 4 + 3, tab[2] * 4 + 0, tab[2] * 4 + 1]


def test_entries_past_context_are_minus_one_and_errors():
    bt, cu, slots = build_block_table([[3, 4, 5]], [1], [4], 4, 5)
    assert bt.tolist() == [[3, -1, -1, -1, -1]]       # only ceil(4/4) = 1 block in use
    with pytest.raises(ValueError):
        build_block_table([[3]], [2], [1], 4, 2)       # q_len > seq_len
    with pytest.raises(ValueError):
        build_block_table([[3]], [1], [5], 4, 2)       # table too short for seq_len
    with pytest.raises(ValueError):
        build_block_table([[3, 4, 5]], [1], [12], 4, 2)  # table width too small
    bt, cu, slots = build_block_table([], [], [], 4, 2)
    assert bt.shape == (0, 2) and cu.tolist() == [0] and slots.size == 0
