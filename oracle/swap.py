"""Swap-out and swap-in of K/V blocks between the device cache and a host swap space
(oracle; test infrastructure only: tests, the smoke check and the benchmark's CPU
baseline may use it, the product never does).

"Continuous Batching" (infra.pidoku inference notes), "5. Technical explanation",
Preemption: the SWAP strategy copies a victim's K/V blocks to CPU memory and frees the
GPU blocks, and copies them back later. What is copied is the plain definition below:
for a pair (device block b, host block h), every layer's K block b and V block b
(block_size x kv heads x head_dim elements each, the cache's own bytes: no conversion)
go to host block h, which holds, in order, layer 0 K, layer 0 V, layer 1 K, ... A swap-in
pair (host block h, device block b) copies them back.

Pinned by a hand-worked layout case, the round trip through other blocks, and the
blocks no pair names staying untouched (tests/test_oracle_swap.py).
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def host_shape(host_blocks: int, k_cache: np.ndarray) -> tuple:
    """Shape of a host swap space for caches [layers][blocks][bs][Hkv][d]:
    [host_blocks][layers][2 (K, V)][bs][Hkv][d]."""
    L, _, bs, h, d = k_cache.shape
    return (int(host_blocks), L, 2, bs, h, d)


def swap_out(k_cache: np.ndarray, v_cache: np.ndarray, pairs: Iterable[Tuple[int, int]], host: np.ndarray) -> None:
    """host[h, l, 0] = k_cache[l, b] and host[h, l, 1] = v_cache[l, b] for each (b, h)."""
    for b, h in pairs:
        for l in range(k_cache.shape[0]):
            host[h, l, 0] = k_cache[l, b]
            host[h, l, 1] = v_cache[l, b]


def swap_in(host: np.ndarray, pairs: Iterable[Tuple[int, int]], k_cache: np.ndarray, v_cache: np.ndarray) -> None:
    """k_cache[l, b] = host[h, l, 0] and v_cache[l, b] = host[h, l, 1] for each (h, b)."""
    for h, b in pairs:
        for l in range(k_cache.shape[0]):
            k_cache[l, b] = host[h, l, 0]
            v_cache[l, b] = host[h, l, 1]
