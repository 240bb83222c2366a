"""The pages' printed values as pins for the oracle's allocator and metadata."""
import json
import os

from oracle.allocator import BlockPool, SeqTables
from oracle.metadata import build_block_table
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


def test_config1_uses_the_printed_prompt_lengths():
    assert workloads.config1().seq_lens.tolist() == GOLD["tiny_vllm_prompt_lengths"]["value"]
    assert workloads.config1().block_size == GOLD["page_size_tokens"]["value"]


def test_table_entry_count():
    v = GOLD["tiny_vllm_block_table_entries"]["value"]
    assert v["max_sequences"] * v["layers"] * v["max_blocks_per_seq"] == v["entries"]


def test_reserved_vs_stored_tokens():
    v = GOLD["contiguous_vs_stored"]["value"]
    reserved = v["requests"] * v["max_len"]
    stored = v["requests"] * v["avg_len"]
    assert stored == v["stored_printed"]
    assert abs(reserved - v["reserved_printed"]) / v["reserved_printed"] < 0.025
    t = SeqTables(BlockPool(4096), GOLD["page_size_tokens"]["value"])
    for s in range(v["requests"]):
        t.reserve(s, v["avg_len"])
    paged_tokens = (4096 - t.pool.num_free) * 16
    assert paged_tokens - stored == 800      # vs 389,600 wasted by contiguous reservation


def test_plus_one_seq_len_reads_two_blocks():
    v = GOLD["tiny_vllm_seq_len_plus_one"]["value"]
    t = SeqTables(BlockPool(8), 16)
    t.reserve(0, v["seq_len_for_attention"])
    bt, cu, slots = build_block_table([t.tables[0]], [1], [v["seq_len_for_attention"]], 16, 4)
    assert int((bt[0] >= 0).sum()) == v["blocks_read_at_bs16"]
    # the current token (position 16) is the first slot of the second block
    assert slots.tolist() == [t.tables[0][1] * 16 + 0]


def test_leak_free_pool_differs_from_printed_prototype_stats():
    v = GOLD["prototype_stats_after_three_requests"]["value"]
    t = SeqTables(BlockPool(v["total"]), 16)
    for s in range(v["completed_requests"]):
        t.reserve(s, 40)
        t.reserve(s, 72)          # grow, as a generating request does
    for s in range(v["completed_requests"]):
        t.release(s)
    assert t.pool.num_free == v["total"] != v["free_kv_blocks"]
