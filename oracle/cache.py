"""Cache write and exact cache decode (oracle).

Layout (a reading of "Project 17 ...", "Step 6: Implement attention over paged
storage", whose pool storage is indexed (page, slot-in-page, head, head_dim,
K-or-V)): per layer, two planes K and V, each [num_blocks][block_size][Hkv][d]
row-major, so one (token, head) row is d contiguous elements and one token's
heads are Hkv*d contiguous elements. Flat slot = block * block_size + offset.

Write ("Step 4: Implement the paged KV cache", append): for every new token i
and KV head h, plane[slot_i // bs][slot_i % bs][h][:] = enc(x[i][h][:]); nothing
else changes. enc is a bit copy for f32 and bf16, the E4M3 encoder of fp8.py
for an fp8 cache. A negative slot skips the token (padding rows).

An fp8 scale may be per KV head (an array [Hkv], see fp8.py): it then applies along the
head axis of the rows and planes.
"""
from __future__ import annotations

import numpy as np

from . import fp8


def empty_plane(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                cache_dtype: str, fill: int = 0) -> np.ndarray:
    dt = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[cache_dtype]
    return np.full((num_blocks, block_size, num_kv_heads, head_dim), fill, dtype=dt)


def _bits_in(x: np.ndarray, in_dtype: str) -> np.ndarray:
    if in_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if in_dtype == "bf16":
        return np.asarray(x, dtype=np.uint16)
    raise ValueError(in_dtype)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _along_heads(scale):
    """A per-head scale array [Hkv] as [Hkv][1], to broadcast over [..., Hkv, d]."""
    return np.asarray(scale, dtype=np.float64)[:, None] if np.ndim(scale) == 1 else scale


def write(plane: np.ndarray, x: np.ndarray, in_dtype: str, cache_dtype: str,
          slot_mapping, scale=1.0) -> None:
    """Scatter new rows x [T][Hkv][d] (float32 array or bf16 bits) into plane."""
    nb, bs = plane.shape[0], plane.shape[1]
    src = _bits_in(x, in_dtype)
    if cache_dtype == "fp8":
        xf = src.view(np.float32) if in_dtype == "f32" else _bf16_bits_to_f32(src)
        enc = fp8.encode(xf, _along_heads(scale))
    elif cache_dtype == in_dtype:
        enc = src
    else:
        raise ValueError(f"unsupported cache write {in_dtype} -> {cache_dtype}")
    seen = set()
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        slot = int(slot)
        if slot < 0:
            continue
        if slot in seen:
            raise ValueError(f"slot {slot} written twice in one step")
        seen.add(slot)
        if slot >= nb * bs:
            raise ValueError(f"slot {slot} outside the pool")
        plane[slot // bs, slot % bs] = enc[i]


def decode_plane(plane: np.ndarray, cache_dtype: str, scale=1.0) -> np.ndarray:
    """Exact float64 values of a cache plane (fp8 codes times scale)."""
    if cache_dtype == "f32":
        return plane.view(np.float32).astype(np.float64)
    if cache_dtype == "bf16":
        return _bf16_bits_to_f32(plane).astype(np.float64)
    if cache_dtype == "fp8":
        return fp8.decode(plane, _along_heads(scale))
    raise ValueError(cache_dtype)


def decode_rows(plane: np.ndarray, block_ids, n_tokens: int, cache_dtype: str,
                scale: float = 1.0) -> np.ndarray:
    """Gather the first n_tokens rows [n][Hkv][d] of one sequence through its
    block table, decoded exactly to float64."""
    bs = plane.shape[1]
    t = np.arange(int(n_tokens), dtype=np.int64)
    blocks = np.asarray(block_ids, dtype=np.int64)[t // bs]
    return decode_plane(plane[blocks, t % bs], cache_dtype, scale)
