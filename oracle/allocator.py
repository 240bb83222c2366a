"""Block pool with a LIFO free list, and per-sequence block tables (oracle).

Follows "Project 17: Production Serving: Continuous Batching and PagedAttention",
"Step 4: Implement the paged KV cache": the free list starts as the list of
page ids, a page is taken from the end of the list and a freed page is appended;
a sequence's pages are returned in page-table order. The all-or-nothing
multi-block request and the out-of-memory error follow "Build a pure-Python
continuous batching LLM serving engine from scratch", "Step 2: Implement the
PagedAttention KV Cache Manager" (raise when fewer blocks are free than asked,
otherwise pop them one by one from the end). Double frees are rejected here;
the pages do not guard against them.

Pinned by: printed block counts and fragmentation arithmetic from "The Concept",
conservation / uniqueness / LIFO invariants, and the leak-free end state
(tests/test_oracle_allocator.py).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional


class OutOfBlocks(Exception):
    """Fewer free blocks than requested; the pool is left unchanged."""


class InvalidFree(Exception):
    """An id that is not currently allocated was freed."""


class BlockPool:
    def __init__(self, num_blocks: int, order: Optional[Iterable[int]] = None):
        self.num_blocks = int(num_blocks)
        self.free: List[int] = list(range(self.num_blocks)) if order is None else [int(x) for x in order]
        if sorted(self.free) != list(range(self.num_blocks)):
            raise ValueError("initial free order must be a permutation of 0..N-1")
        self._allocated = [False] * self.num_blocks

    def alloc(self, n: int) -> List[int]:
        """Take n ids from the END of the free list, or raise OutOfBlocks."""
        if n < 0:
            raise ValueError("negative request")
        if len(self.free) < n:
            raise OutOfBlocks(f"need {n}, free {len(self.free)}")
        out = []
        for _ in range(n):
            b = self.free.pop()
            self._allocated[b] = True
            out.append(b)
        return out

    def release(self, ids: Iterable[int]) -> None:
        """Append ids to the free list in the given order."""
        ids = [int(b) for b in ids]
        seen = set()
        for b in ids:
            if not (0 <= b < self.num_blocks) or not self._allocated[b] or b in seen:
                raise InvalidFree(b)
            seen.add(b)
        for b in ids:
            self._allocated[b] = False
            self.free.append(b)

    @property
    def num_free(self) -> int:
        return len(self.free)


class SeqTables:
    """Per-sequence block tables drawn from one pool.

    reserve(seq, n_tokens) grows seq's table to ceil(n_tokens / block_size)
    blocks (never shrinks), all-or-nothing; release(seq) frees its table in
    table order and forgets the sequence.
    """

    def __init__(self, pool: BlockPool, block_size: int):
        self.pool = pool
        self.block_size = int(block_size)
        self.tables: Dict[int, List[int]] = {}

    def blocks_for(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    def reserve(self, seq: int, n_tokens: int) -> List[int]:
        t = self.tables.get(seq, [])
        need = self.blocks_for(n_tokens) - len(t)
        if need > 0:
            new = self.pool.alloc(need)          # raises OutOfBlocks, no change
            t = t + new
        self.tables[seq] = t
        return t

    def release(self, seq: int) -> None:
        t = self.tables.pop(seq)
        self.pool.release(t)

    def check(self) -> None:
        """Conservation and uniqueness: every id is free xor in exactly one table."""
        used = [b for t in self.tables.values() for b in t]
        allids = used + self.pool.free
        assert len(allids) == self.pool.num_blocks, (len(allids), self.pool.num_blocks)
        assert len(set(allids)) == self.pool.num_blocks


def replay_history(tables: SeqTables, history, owner_base: int = 1 << 40) -> None:
    """Apply a list of ("alloc", owner, n) / ("free", owner) requests; dummy
    owners are keyed far from real sequence ids and stay live if never freed."""
    for op in history:
        if op[0] == "alloc":
            owner, n = op[1], op[2]
            key = owner_base + owner
            tables.tables[key] = tables.pool.alloc(n)
        elif op[0] == "free":
            tables.release(owner_base + op[1])
        else:
            raise ValueError(op)
