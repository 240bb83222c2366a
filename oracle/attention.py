"""Attention over a paged KV cache (oracle), float64 on exactly decoded K/V.

Definition followed: "Project 17: Production Serving: Continuous Batching and
PagedAttention", "Step 6: Implement attention over paged storage" — for each
token of the sequence, walk the page table to the page and slot that hold its
key, score it against the query scaled by 1/sqrt(head_dim), softmax the scores,
then walk the table again and sum the values weighted by the softmax. Readings
where that sketch is garbled or silent:

* scores and softmax are per query head (the sketch sums the product over all
  heads and applies one weight to every head; per-head is the only reading that
  makes its output multi-head attention);
* head_dim, undefined in the sketch, is the query's last dimension; scale is
  1/sqrt(head_dim) unless given;
* grouped-query attention maps query head h to KV head h // (Hq / Hkv);
* a query row at absolute position p sees keys 0..p: a chunk of q new tokens of
  a sequence with seq_len L covers positions L-q..L-1 (bottom-right causal
  alignment; a decode row is the case q = 1 and sees all L keys);
* a row with no keys (seq_len 0) outputs zeros and log-sum-exp -inf.

`attend` is the plain definition over contiguous (gathered) K/V; `paged_attention`
gathers each sequence's rows through its block table and calls it;
`paged_attention_literal` evaluates the same definition token by token through the
page table, in pure Python, for tiny shapes; and
`split_merge` evaluates fixed-length context partitions and merges them by
log-sum-exp, which equals `attend` algebraically.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import cache


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale: float,
           group: int, heads: Optional[Sequence[int]] = None):
    """q [n][Hq][d], K/V [L][Hkv][d] (float64). Row i sees keys 0..positions[i].

    Returns (out [n][Hq][d], lse [n][Hq]); heads restricts which query heads
    are computed (others left zero / -inf)."""
    q = np.asarray(q, np.float64)
    n, Hq, d = q.shape
    L = K.shape[0]
    pos = np.asarray(positions, dtype=np.int64).reshape(n)
    out = np.zeros((n, Hq, d), np.float64)
    lse = np.full((n, Hq), -np.inf, np.float64)
    keys = np.arange(L)
    visible = keys[None, :] <= pos[:, None]              # [n][L]
    hs = range(Hq) if heads is None else heads
    for h in hs:
        g = h // group
        z = scale * (q[:, h, :] @ K[:, g, :].T)           # [n][L]
        z = np.where(visible, z, -np.inf)
        for i in range(n):
            if not visible[i].any():
                continue
            m = z[i].max()
            e = np.exp(z[i] - m)
            tot = e.sum()
            out[i, h] = (e / tot) @ V[:, g, :]
            lse[i, h] = m + math.log(tot)
    return out, lse


def paged_attention(q: np.ndarray, k_plane: np.ndarray, v_plane: np.ndarray, cache_dtype: str,
                    block_tables: np.ndarray, seq_lens, cu_seqlens_q, scale: float, group: int,
                    k_scale: float = 1.0, v_scale: float = 1.0,
                    seqs: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """Attention for every query row of a step. q [sum q][Hq][d] float64.

    Row r of sequence s (cu_seqlens_q[s] <= r < cu_seqlens_q[s+1]) sits at
    position seq_lens[s] - q_s + (r - cu_seqlens_q[s]). Returns (out, lse) over
    all rows; `seqs` / `heads` restrict the work (other entries stay 0 / -inf)."""
    q = np.asarray(q, np.float64)
    T, Hq, d = q.shape
    out = np.zeros((T, Hq, d), np.float64)
    lse = np.full((T, Hq), -np.inf, np.float64)
    B = len(seq_lens)
    for s in (range(B) if seqs is None else seqs):
        L = int(seq_lens[s])
        r0, r1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        nq = r1 - r0
        if nq == 0:
            continue
        K = cache.decode_rows(k_plane, block_tables[s], L, cache_dtype, k_scale)
        V = cache.decode_rows(v_plane, block_tables[s], L, cache_dtype, v_scale)
        positions = L - nq + np.arange(nq)
        o, l = attend(q[r0:r1], K, V, positions, scale, group, heads)
        out[r0:r1] = o
        lse[r0:r1] = l
    return out, lse


def paged_attention_literal(query: np.ndarray, page_table, k_plane: np.ndarray,
                            v_plane: np.ndarray, cache_dtype: str, seq_len: int,
                            group: int, scale: Optional[float] = None):
    """Decode attention of one query [Hq][d] evaluated token by token from the
    definition, reading each key and value through the page table: token t of the
    sequence is row t % block_size of physical block page_table[t // block_size]. Per
    query head h (KV head h // group): z_t = scale * q_h . K_t for every t < seq_len,
    weights w_t = exp(z_t - max z) / sum exp(z - max z), out_h = sum_t w_t V_t.

    Slow by design (pure Python arithmetic); for tiny shapes only."""
    Hq, d = query.shape
    bs = k_plane.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    where = [(int(page_table[t // bs]), t % bs) for t in range(int(seq_len))]
    out = np.zeros((Hq, d), np.float64)
    for h in range(Hq):
        g = h // group
        K = [cache.decode_plane(k_plane[blk, off, g], cache_dtype) for blk, off in where]
        V = [cache.decode_plane(v_plane[blk, off, g], cache_dtype) for blk, off in where]
        if not K:
            continue
        z = [scale * math.fsum(float(a) * float(b) for a, b in zip(query[h], k)) for k in K]
        zmax = max(z)
        e = [math.exp(zt - zmax) for zt in z]
        tot = math.fsum(e)
        for j in range(d):
            out[h, j] = math.fsum(et / tot * float(v[j]) for et, v in zip(e, V))
    return out


def split_merge(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, group: int,
                partition: int):
    """One decode row [Hq][d] over contiguous K/V [L][Hkv][d], evaluated in
    partitions [k*P, min((k+1)*P, L)) that each give (m_k, l_k, o_k) with
    o_k normalised, merged by log-sum-exp. Returns (out [Hq][d], lse [Hq])."""
    Hq, d = q_row.shape
    L = K.shape[0]
    out = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    for h in range(Hq):
        g = h // group
        z = scale * (K[:, g, :] @ q_row[h])
        ms, ls, os_ = [], [], []
        for a in range(0, L, partition):
            b = min(a + partition, L)
            zk = z[a:b]
            m = zk.max()
            e = np.exp(zk - m)
            l_k = e.sum()
            ms.append(m)
            ls.append(l_k)
            os_.append((e / l_k) @ V[a:b, g, :])
        if not ms:
            continue
        M = max(ms)
        W = np.array([l_k * math.exp(m - M) for m, l_k in zip(ms, ls)])
        out[h] = (W[:, None] * np.array(os_)).sum(0) / W.sum()
        lse[h] = M + math.log(W.sum())
    return out, lse
