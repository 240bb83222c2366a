"""Helpers for the GPU parity tests: put one workload step into device memory through
libpkv (host tables + cache-write kernel) and compute the oracle's side.

Both sides take their inputs from `workloads` (identical bits); the oracle side never
reads anything produced by the GPU path except to compare against it."""
from __future__ import annotations

import dataclasses
import functools
import json
import os
import subprocess
import sys
import tempfile
from typing import Optional

import numpy as np
import torch

import paged_kv_cache_42_amd as pkv
import workloads
import workloads.gpu as wgen
from oracle import allocator as oa
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import fp8 as ofp8
from oracle.metadata import build_block_table as oracle_build

DUMMY = 1 << 40
NAN_FILL = {"f32": 0x7FC00000, "bf16": 0x7FC0, "fp8": 0x7F}   # stale slots hold NaN
TOL = {"f32": None, "bf16": 2e-2, "fp8": 6e-2}


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[name]


def to_device(a: np.ndarray, dtype: str, dev="cuda"):
    """Storage array (float32 or bf16 bits) -> device tensor of that dtype."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(dev).view(torch.bfloat16)
    raise ValueError(dtype)


def plane_bits(t: torch.Tensor) -> np.ndarray:
    """Device cache plane -> host array of raw bits (uint32 / uint16 / uint8)."""
    h = t.cpu()
    if h.dtype == torch.float32:
        return h.numpy().view(np.uint32)
    if h.dtype == torch.bfloat16:
        return h.view(torch.int16).numpy().view(np.uint16)
    return h.numpy().view(np.uint8)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class Step:
    w: workloads.Workload
    pool: pkv.Pool
    width: int
    bt: np.ndarray
    cu: np.ndarray
    slots: np.ndarray
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    q: torch.Tensor
    bt_d: torch.Tensor
    lens_d: torch.Tensor
    cu_d: torch.Tensor
    ctx_slots: np.ndarray
    new_rows: tuple   # (k, v) storage arrays of this step's new tokens


def build_step(w: workloads.Workload, width: Optional[int] = None, fill_nan: bool = True,
               pool_order=None) -> Step:
    """Tables from libpkv's host pool, prior context written by the cache-write kernel,
    then this step's new tokens written by a second cache-write launch."""
    order = w.free_order if pool_order is None else pool_order
    pool = pkv.Pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype, free_order=order)
    for op in w.history:
        if op[0] == "alloc":
            pool.seq_reserve(DUMMY + op[1], op[2] * w.block_size)
        else:
            pool.seq_release(DUMMY + op[1])
    for s, L in enumerate(w.seq_lens):
        pool.seq_reserve(s, int(L))
    W = width or max(1, w.max_blocks_per_seq())
    ids = np.arange(w.num_seqs)
    prior = (w.seq_lens - w.q_lens).astype(np.int32)
    _, _, ctx_slots = pool.build_block_table(ids, prior, prior, W)
    bt, cu, slots = pool.build_block_table(ids, w.q_lens, w.seq_lens, W)

    cdt = torch_dtype(w.cache_dtype)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    if w.cache_dtype == "f32":
        k_cache = torch.empty(shape, dtype=torch.int32, device="cuda")
    elif w.cache_dtype == "bf16":
        k_cache = torch.empty(shape, dtype=torch.int16, device="cuda")
    else:
        k_cache = torch.empty(shape, dtype=torch.uint8, device="cuda")
    if fill_nan:
        k_cache.fill_(NAN_FILL[w.cache_dtype])
    v_cache = k_cache.clone()
    if w.cache_dtype != "fp8":
        k_cache = k_cache.view(cdt)
        v_cache = v_cache.view(cdt)

    # inputs made on the GPU by the counter-hash twin of the numpy generator
    tdt = torch_dtype(w.dtype)
    Hkv, Hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    n_ctx, n_new = int(prior.sum()), int(w.q_lens.sum())
    ctx_k = torch.empty((n_ctx, Hkv, d), dtype=tdt, device="cuda")
    ctx_v = torch.empty_like(ctx_k)
    new_k = torch.empty((n_new, Hkv, d), dtype=tdt, device="cuda")
    new_v = torch.empty_like(new_k)
    q = torch.empty((n_new, Hq, d), dtype=tdt, device="cuda")
    oc = on = 0
    for s in range(w.num_seqs):
        p, L = int(prior[s]), int(w.seq_lens[s])
        for buf_ctx, buf_new, which in ((ctx_k, new_k, "k"), (ctx_v, new_v, "v")):
            key = w.value_key(which, s)
            if p:
                wgen.fill(buf_ctx[oc:oc + p], key, 0, w.sigma)
            if L > p:
                wgen.fill(buf_new[on:on + L - p], key, p * Hkv * d, w.sigma)
        if L > p:
            wgen.fill(q[on:on + L - p], w.value_key("q", s), p * Hq * d, w.sigma)
        oc += p
        on += L - p
    if n_ctx:
        pkv.kv_cache_write(ctx_k, ctx_v, k_cache, v_cache, torch.from_numpy(ctx_slots).cuda(), w.block_size,
                           w.k_scale, w.v_scale, **heads(w))
    if n_new:
        pkv.kv_cache_write(new_k, new_v, k_cache, v_cache, torch.from_numpy(slots).cuda(), w.block_size,
                           w.k_scale, w.v_scale, **heads(w))
    del ctx_k, ctx_v
    return Step(w, pool, W, bt, cu, slots, k_cache, v_cache, q,
                torch.from_numpy(bt).cuda(), torch.from_numpy(w.seq_lens.astype(np.int32)).cuda(),
                torch.from_numpy(cu).cuda(), ctx_slots, (new_k, new_v))


def heads(w: workloads.Workload) -> dict:
    """The per-head scale factors as keyword arguments of the libpkv calls."""
    return {"k_head_scales": w.k_head_scales, "v_head_scales": w.v_head_scales}


def oracle_scales(w: workloads.Workload):
    """(K, V) scales for the oracle: per tensor, or per head (the product of the two)."""
    ks = w.k_scale if w.k_head_scales is None else ofp8.head_scales(w.k_scale, w.k_head_scales)
    vs = w.v_scale if w.v_head_scales is None else ofp8.head_scales(w.v_scale, w.v_head_scales)
    return ks, vs


def oracle_planes(st: Step):
    """The oracle's own tables and cache planes for the same step (same write order)."""
    w = st.w
    ref = oa.SeqTables(oa.BlockPool(w.num_blocks, w.free_order), w.block_size)
    oa.replay_history(ref, w.history, owner_base=DUMMY)
    for s, L in enumerate(w.seq_lens):
        ref.reserve(s, int(L))
    tabs = [ref.tables[s] for s in range(w.num_seqs)]
    prior = (w.seq_lens - w.q_lens).astype(np.int32)
    _, _, ctx_slots = oracle_build(tabs, prior, prior, w.block_size, st.width)
    bt, cu, slots = oracle_build(tabs, w.q_lens, w.seq_lens, w.block_size, st.width)
    fill = NAN_FILL[w.cache_dtype]
    kp = ocache.empty_plane(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype, fill)
    vp = kp.copy()
    ks, vs = zip(*[w.kv(s) for s in range(w.num_seqs)])
    ctx_k = np.concatenate([k[: prior[s]] for s, k in enumerate(ks)])
    ctx_v = np.concatenate([v[: prior[s]] for s, v in enumerate(vs)])
    new_k = np.concatenate([k[prior[s]:] for s, k in enumerate(ks)])
    new_v = np.concatenate([v[prior[s]:] for s, v in enumerate(vs)])
    ks, vs = oracle_scales(w)
    ocache.write(kp, ctx_k, w.dtype, w.cache_dtype, ctx_slots, ks)
    ocache.write(vp, ctx_v, w.dtype, w.cache_dtype, ctx_slots, vs)
    ocache.write(kp, new_k, w.dtype, w.cache_dtype, slots, ks)
    ocache.write(vp, new_v, w.dtype, w.cache_dtype, slots, vs)
    return tabs, bt, cu, slots, kp, vp


def oracle_attention_full(st: Step, kp, vp, bt, cu):
    w = st.w
    q = workloads.storage_to_f64(w.q_all(), w.dtype)
    ks, vs = oracle_scales(w)
    return oatt.paged_attention(q, kp, vp, w.cache_dtype, bt, w.seq_lens, cu, w.softmax_scale, w.group, ks, vs)


def run_decode(st: Step, partition_size: Optional[int] = None, lse: bool = True, max_seq_len=None,
               use_work: bool = True):
    w = st.w
    P = w.partition_size if partition_size is None else partition_size
    B, Hq, d = w.num_seqs, w.num_q_heads, w.head_dim
    msl = int(w.seq_lens.max()) if max_seq_len is None else max_seq_len
    out = torch.empty((B, Hq, d), dtype=torch_dtype(w.dtype), device="cuda")
    ws_bytes = pkv.decode_workspace_bytes(B, Hq, d, msl, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    lse_t = torch.empty((B, Hq), dtype=torch.float32, device="cuda") if lse else None
    work = torch.from_numpy(pkv.build_decode_work(w.seq_lens, P)).cuda() if use_work else None
    pkv.paged_attention_decode(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, w.num_kv_heads,
                               w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale, P, ws, lse_t, work=work,
                               **heads(w))
    torch.cuda.synchronize()
    return out, lse_t


def run_decode_split(st: Step, num_slots: Optional[int] = None, min_piece_tokens: int = 0, lse: bool = True,
                     max_seq_len=None, plan_lens=None, q=None):
    """The balanced-split decode launch; outputs start as NaN so an unwritten row shows.
    q: decode queries [B][Hq][d] (default: the step's rows, one per sequence)."""
    w = st.w
    B, Hq, d = w.num_seqs, w.num_q_heads, w.head_dim
    msl = int(w.seq_lens.max()) if max_seq_len is None else max_seq_len
    if num_slots is None:
        num_slots = pkv.decode_split_slots(pkv.FP8 if w.cache_dtype == "fp8" else pkv.BF16, w.num_kv_heads, d,
                                           w.block_size)
    split = pkv.build_decode_split(w.seq_lens if plan_lens is None else plan_lens, num_slots, min_piece_tokens)
    plan_d = torch.from_numpy(split.plan).cuda()
    out = torch.full((B, Hq, d), float("nan"), dtype=torch_dtype(w.dtype), device="cuda")
    ws = pkv.decode_split_workspace(split, Hq, d)
    lse_t = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    pkv.paged_attention_decode_split(out, st.q if q is None else q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, plan_d, split,
                                     w.num_kv_heads, w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale,
                                     ws, lse_t, **heads(w))
    torch.cuda.synchronize()
    return out, lse_t, split


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what=""):
    if dtype == "f32":
        err = np.abs(got - ref)
        bound = 1e-5 * np.abs(ref) + 1e-6
        bad = ~(err <= bound)
        assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1e-5 rel, worst {err.max():.3e}"
    else:
        tol = TOL[dtype]
        err = np.abs(got - ref)
        assert np.all(err <= tol), f"{what}: max abs err {np.nanmax(err):.3e} > {tol}"


def run_varlen(st: Step, lse: bool = True, max_seq_len=None):
    """The mixed-step launch (prefill chunks + decode rows) over the step's rows."""
    w = st.w
    T, Hq, d = w.total_q, w.num_q_heads, w.head_dim
    msl = int(w.seq_lens.max()) if max_seq_len is None else max_seq_len
    out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    work = torch.from_numpy(pkv.build_varlen_work(w.q_lens, w.seq_lens, w.num_kv_heads, w.group)).cuda()
    pkv.paged_attention_prefill_varlen(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, st.cu_d, work,
                                       w.num_kv_heads, w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale,
                                       lse=lse_t, **heads(w))
    torch.cuda.synchronize()
    return out, lse_t


def run_mixed_two_launch(st: Step, num_slots: Optional[int] = None, min_piece_tokens: int = 0, lse: bool = True,
                         chunk_slots: Optional[int] = None, min_piece_tiles: int = 0):
    """A mixed step as two launches: decode rows (one new token) by the balanced-split decode
    with the batch's row map, the other rows by the chunk kernel (blocks cut along the keys
    over chunk_slots resident workgroups, the device's count when None, 0: uncut)."""
    w = st.w
    T, Hq, d = w.total_q, w.num_q_heads, w.head_dim
    msl = int(w.seq_lens.max())
    cdt = pkv.FP8 if w.cache_dtype == "fp8" else pkv.BF16
    if num_slots is None:
        num_slots = pkv.decode_split_slots(cdt, w.num_kv_heads, d, w.block_size)
    if chunk_slots is None:
        chunk_slots = pkv.chunk_slots(cdt, d, w.block_size)
    mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, w.num_kv_heads, w.group, num_slots, min_piece_tokens,
                              chunk_slots, min_piece_tiles)
    out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    if len(mp.decode_rows):
        ws = pkv.decode_split_workspace(mp.split, Hq, d)
        pkv.paged_attention_decode_split(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d,
                                         torch.from_numpy(mp.split.plan).cuda(), mp.split, w.num_kv_heads,
                                         w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale, ws, lse_t,
                                         rows=torch.from_numpy(mp.decode_rows).cuda(), cu_seqlens_q=st.cu_d,
                                         **heads(w))
    dev = mp.chunks.to_device(d)
    if dev is not None:
        work, merges, cws = dev
        pkv.paged_attention_prefill_chunks(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, st.cu_d, work,
                                           merges, mp.chunks.num_partials, cws, w.num_kv_heads, w.block_size, msl,
                                           w.softmax_scale, w.k_scale, w.v_scale, lse=lse_t, **heads(w))
    torch.cuda.synchronize()
    return out, lse_t


def run_mixed(st: Step, num_slots: Optional[int] = None, min_piece_tokens: int = 0, lse: bool = True,
              chunk_slots: Optional[int] = None, min_piece_tiles: int = 0):
    """A mixed step through pkv_paged_attention_mixed (one launch plus the merges with 8k
    KV heads, else the two kernels in turn); decode slots from mixed_decode_slots when
    num_slots is None."""
    w = st.w
    T, Hq, d = w.total_q, w.num_q_heads, w.head_dim
    msl = int(w.seq_lens.max())
    cdt = pkv.FP8 if w.cache_dtype == "fp8" else pkv.BF16
    if num_slots is None:
        num_slots = pkv.mixed_decode_slots(w.q_lens, w.seq_lens, cdt, w.num_kv_heads, w.group, d, w.block_size)
    if chunk_slots is None:
        chunk_slots = pkv.chunk_slots(cdt, d, w.block_size)
    mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, w.num_kv_heads, w.group, num_slots, min_piece_tokens,
                              chunk_slots, min_piece_tiles)
    out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    pkv.paged_attention_mixed(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, st.cu_d, mp,
                              mp.to_device(d, Hq), w.num_kv_heads, w.block_size, msl, w.softmax_scale, w.k_scale,
                              w.v_scale, lse=lse_t, **heads(w))
    torch.cuda.synchronize()
    return out, lse_t


ORACLE_JOBS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_jobs.py")


@functools.lru_cache(maxsize=None)
def _oracle_job(job_json: str, timeout: float):
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    print(f"[oracle] {job_json} on {workers} worker processes", flush=True)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "oracle.npz")
        subprocess.run([sys.executable, ORACLE_JOBS, job_json, path, str(workers)], check=True, timeout=timeout)
        with np.load(path) as z:
            return {k: z[k] for k in z.files}


def oracle_job(job: dict, timeout: float = 900) -> dict:
    """The oracle's results for `job` (see oracle_jobs.py), computed by a child program
    with a pool of worker processes (this process holds the GPU and must not fork);
    cached for the rest of the test session."""
    return _oracle_job(json.dumps(job, sort_keys=True), timeout)


def report_error(what: str, got: np.ndarray, ref: np.ndarray, got_lse=None, ref_lse=None) -> None:
    """Print the worst absolute errors of a comparison (collected into the design notes)."""
    msg = f"[parity] {what}: max |out err| {np.nanmax(np.abs(got - ref)):.3e}"
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        e = np.abs(got_lse[fin] - ref_lse[fin])
        msg += f", max |lse err| {e.max() if e.size else 0.0:.3e}"
    print(msg, flush=True)
