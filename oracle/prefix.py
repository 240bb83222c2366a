"""Prefix caching over shared, reference-counted blocks (oracle; test infrastructure:
only tests, the smoke check and the benchmark's CPU baseline use it).

"Project 17: Production Serving: Continuous Batching and PagedAttention", "Step 8:
Prefix caching": a cache maps page-aligned token prefixes to the pages that hold their
K/V; a lookup tries the longest page-aligned prefix of the tokens first and walks down
one page at a time, and a hit takes a reference on each of its pages. Reference counts
per block follow "Build a pure-Python continuous batching LLM serving engine from
scratch", "Step 2" (a count raised on allocation, lowered on free).

Readings where the pages stop (each also listed with the other readings):
  * a block goes back to the free list when its last reference goes (the page that
    lowers the count frees the block in the same breath; with sharing that would free a
    page another table still reads, so the count decides);
  * the cache itself holds no reference: an entry is usable while every one of its
    blocks is still held by some table and has not been freed since (a generation per
    block, bumped on every free, invalidates stale entries);
  * only whole pages of prompt tokens are cached, and only after the step that wrote
    them; the first entry for a prefix stays while it is valid;
  * a lookup looks at most at `limit` tokens: a fresh request must compute at least its
    last prompt token (that row yields its first output), so limit = prompt - 1; a
    recompute after preemption also holds outputs, so limit = prompt;
  * shared pages are never written: a request's new tokens start after its cached
    prefix, which ends on a page boundary, so no copy-on-write is needed.
Pinned by hand-worked traces and invariants in tests/test_oracle_prefix.py.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

from .allocator import BlockPool, SeqTables


class SharedTables(SeqTables):
    """SeqTables whose blocks may appear in several tables, with a count per block."""

    def __init__(self, pool: BlockPool, block_size: int):
        super().__init__(pool, block_size)
        self.ref = [0] * pool.num_blocks
        self.gen = [0] * pool.num_blocks

    def reserve(self, seq: int, n_tokens: int) -> List[int]:
        t = self.tables.get(seq, [])
        need = self.blocks_for(n_tokens) - len(t)
        if need > 0:
            new = self.pool.alloc(need)          # raises OutOfBlocks, no change
            for b in new:
                self.ref[b] = 1
            t = t + new
        self.tables[seq] = t
        return t

    def share(self, seq: int, blocks: Sequence[int]) -> None:
        """Start seq's (empty) table with blocks other tables hold, one reference each."""
        if self.tables.get(seq):
            raise ValueError("share starts a table")
        for b in blocks:
            if self.ref[b] <= 0:
                raise ValueError(f"block {b} is not held")
        for b in blocks:
            self.ref[b] += 1
        self.tables[seq] = list(blocks)

    def release(self, seq: int) -> None:
        t = self.tables.pop(seq)
        freed = []
        for b in t:                              # table order
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.gen[b] += 1
                freed.append(b)
        self.pool.release(freed)

    def check(self) -> None:
        """Every block is free xor referenced, and its count = the tables holding it."""
        count = [0] * self.pool.num_blocks
        for t in self.tables.values():
            for b in t:
                count[b] += 1
        assert count == self.ref, "reference counts"
        free = set(self.pool.free)
        assert len(free) == len(self.pool.free), "duplicate free id"
        for b in range(self.pool.num_blocks):
            assert (b in free) == (self.ref[b] == 0), b


class PrefixCache:
    """Page-aligned token prefix -> [(block, generation)] of the pages holding it."""

    def __init__(self, tables: SharedTables):
        self.tables = tables
        self.bs = tables.block_size
        self.cache: Dict[Tuple[int, ...], List[Tuple[int, int]]] = {}

    def _valid(self, entry) -> bool:
        return all(self.tables.ref[b] > 0 and self.tables.gen[b] == g for b, g in entry)

    def lookup(self, tokens: Sequence[int], limit: int) -> Tuple[int, List[int]]:
        """Longest page-aligned prefix of tokens[:limit] with a valid entry: (tokens, pages)."""
        for n in range(min(limit, len(tokens)) // self.bs * self.bs, 0, -self.bs):
            e = self.cache.get(tuple(tokens[:n]))
            if e is not None and self._valid(e):
                return n, [b for b, _ in e]
        return 0, []

    def insert(self, tokens: Sequence[int], table: Sequence[int], n_tokens: int) -> None:
        """Register the whole pages of tokens[:n_tokens], held by table[:pages]."""
        for k in range(1, min(n_tokens, len(tokens)) // self.bs + 1):
            key = tuple(tokens[:k * self.bs])
            e = self.cache.get(key)
            if e is None or not self._valid(e):
                self.cache[key] = [(b, self.tables.gen[b]) for b in table[:k]]
