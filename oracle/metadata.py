"""Per-step metadata for one attention launch (oracle).

From "Continuous Batching", "6. Under the hood": each step builds the request
boundaries for varlen kernels (cu_seqlens), a (num_seqs, max_blocks) block table
for paged attention, and the per-sequence context lengths (seq_lens).
From "Project 17 ...", "Step 4: Implement the paged KV cache": token position p
of a sequence lives in logical page p // PAGE_SIZE at slot p % PAGE_SIZE, so its
flat cache slot is table[p // bs] * bs + p % bs. Unused table entries hold -1,
as the tiny-vllm reading ("Termination and returning blocks") resets them.
seq_lens counts this step's tokens as already written (the tiny-vllm reading,
"Uploading the active arrays to the GPU": the current token's K/V is stored
before attention reads seq_len tokens).

Pinned by a token-at-a-time append simulation of the Step 4 page-table growth
(tests/test_oracle_metadata.py).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def build_block_table(tables: Sequence[Sequence[int]], q_lens, seq_lens, block_size: int,
                      table_width: int):
    """Return (block_tables [B][W] int32, cu_seqlens_q [B+1] int32, slot_mapping [sum q] int64).

    tables[s] is sequence s's list of physical block ids (logical order);
    the new tokens of s are positions seq_lens[s]-q_lens[s] .. seq_lens[s]-1.
    """
    B = len(tables)
    bs = int(block_size)
    bt = np.full((B, table_width), -1, dtype=np.int32)
    cu = np.zeros(B + 1, dtype=np.int32)
    slots = []
    for s in range(B):
        L = int(seq_lens[s])
        q = int(q_lens[s])
        if q < 0 or q > L:
            raise ValueError(f"sequence {s}: q_len {q} outside 0..seq_len {L}")
        nblk = -(-L // bs)
        if nblk > len(tables[s]):
            raise ValueError(f"sequence {s}: table holds {len(tables[s])} blocks, needs {nblk}")
        if nblk > table_width:
            raise ValueError(f"sequence {s}: {nblk} blocks exceed table width {table_width}")
        for j in range(nblk):
            bt[s, j] = tables[s][j]
        cu[s + 1] = cu[s] + q
        for p in range(L - q, L):
            slots.append(int(tables[s][p // bs]) * bs + p % bs)
    return bt, cu, np.asarray(slots, dtype=np.int64)
