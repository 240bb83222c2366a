"""Oracle outputs for the full-size GPU parity tests, computed in a separate program.

The GPU test process must neither fork nor exec itself once it holds the GPU, and the
oracle at full size (every sequence and head of the large decode batches, every row of
kept replay steps in every layer) is minutes of single-threaded float64 work. So the
tests start this file as a child program; it never touches the GPU, spreads the work
over a pool of worker processes (forked here, which is safe: this process has no GPU
state) and writes the results to an .npz file.

It reads only the seeded input generator (`workloads`) and the oracle (`oracle/`).

    python tests/oracle_jobs.py '<job json>' <out.npz> <workers>

Jobs:
  {"kind": "decode", "config": 3 | 4}
      out [B][Hq][d] and lse [B][Hq] (float64) of the batch's decode rows, by the
      oracle's attention definition over each sequence's dense K/V.
  {"kind": "replay", "trace": "config5" | "config5_prefix", "cache_dtype": "bf16" | "fp8",
   "sched": {scheduler options}, "steps": [...], "layers": [...]}
      the scheduler oracle's plan of each listed step (ids, stages, q_lens, seq_lens,
      cu_seqlens_q), and for every layer listed, out [T][Hq][d] / lse [T][Hq] (float32)
      of every query row of the step over the request's dense K/V (E4M3 caches: the
      dequantised codes the oracle's encoder gives). Scheduler options are those of
      oracle.scheduler.Scheduler (token budget, swap space, victim policy), plus
      "priority": true for the trace's priority classes; a prefix trace passes its
      prompt token ids (prefix caching on).
"""
from __future__ import annotations

import json
import multiprocessing as mp
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from oracle import attention as oatt  # noqa: E402
from oracle import fp8 as ofp8  # noqa: E402
from oracle import scheduler as osch  # noqa: E402

_W = None      # the job's workload / trace, set in each worker by the pool initialiser


def _init(job):
    global _W
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)            # one BLAS thread per worker process
    except Exception:
        pass
    _W = workloads.config(int(job["config"])) if job["kind"] == "decode" else _trace(job)


def _trace(job):
    if job.get("trace", "config5") == "config5_prefix":
        return workloads.config5_prefix(job["cache_dtype"])
    return workloads.config5(job["cache_dtype"])


def _decode_seq(s):
    w = _W
    L, G = int(w.seq_lens[s]), w.group
    k, v = w.kv_f32(s)
    q = workloads.storage_to_f64(w.q(s), w.dtype)
    out = np.zeros((w.num_q_heads, w.head_dim))
    lse = np.full(w.num_q_heads, -np.inf)
    for g in range(w.num_kv_heads):
        K = np.ascontiguousarray(k[:, g:g + 1, :], dtype=np.float64)
        V = np.ascontiguousarray(v[:, g:g + 1, :], dtype=np.float64)
        o, l_ = oatt.attend(q[:, g * G:(g + 1) * G, :], K, V, [L - 1], w.softmax_scale, G)
        out[g * G:(g + 1) * G] = o[0]
        lse[g * G:(g + 1) * G] = l_[0]
    return s, out, lse


def _dense(tr, which, layer, req, L):
    x = tr.rows_f32(which, layer, req, 0, L).astype(np.float64)
    if tr.cache_dtype == "fp8":
        scale = tr.k_scale if which == "k" else tr.v_scale
        x = ofp8.decode(ofp8.encode(x.astype(np.float32), scale), scale)
    return x


def _replay_row(task):
    """(step, layer, row index, request, q, L) -> that row's out [q][Hq][d], lse [q][Hq]."""
    step, layer, r, req, q, L = task
    tr = _W
    K = _dense(tr, "k", layer, req, L)
    V = _dense(tr, "v", layer, req, L)
    qs = tr.rows_f32("q", layer, req, L - q, L).astype(np.float64)
    o, l_ = oatt.attend(qs, K, V, np.arange(L - q, L), tr.softmax_scale, tr.group)
    return step, layer, r, o.astype(np.float32), l_.astype(np.float32)


def run_decode(job, workers):
    w = workloads.config(int(job["config"]))
    out = np.zeros((w.num_seqs, w.num_q_heads, w.head_dim))
    lse = np.zeros((w.num_seqs, w.num_q_heads))
    order = np.argsort(-w.seq_lens)                 # longest first: the pool finishes together
    with mp.get_context("fork").Pool(workers, _init, (job,)) as pool:
        for s, o, l_ in pool.imap_unordered(_decode_seq, order.tolist(), chunksize=1):
            out[s], lse[s] = o, l_
    return {"out": out, "lse": lse, "seq_lens": w.seq_lens}


def run_replay(job, workers):
    tr = _trace(job)
    steps = sorted(int(s) for s in job["steps"])
    layers = [int(x) for x in job["layers"]]
    kw = dict(job.get("sched", {}))
    if kw.pop("priority", False):
        kw["priority"] = workloads.priority_classes(tr)
    if job.get("trace") == "config5_prefix":
        kw["prompt_tokens"] = [tr.prompt_tokens(r) for r in range(tr.num_requests)]
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, **kw)
    width = -(-int((tr.prompt + tr.max_tokens - 1).max()) // tr.block_size)
    res, tasks = {}, []
    for plan, _ in osch.run(ref, width, max_steps=steps[-1] + 1):
        if plan.step not in steps:
            continue
        p = f"s{plan.step}"
        res[p + "_ids"], res[p + "_stages"] = plan.ids, plan.stages
        res[p + "_q_lens"], res[p + "_seq_lens"], res[p + "_cu"] = plan.q_lens, plan.seq_lens, plan.cu_seqlens_q
        T = int(plan.cu_seqlens_q[-1])
        for layer in layers:
            res[f"{p}_l{layer}_out"] = np.zeros((T, tr.num_q_heads, tr.head_dim), np.float32)
            res[f"{p}_l{layer}_lse"] = np.zeros((T, tr.num_q_heads), np.float32)
            for r in range(len(plan.ids)):
                tasks.append((plan.step, layer, r, int(plan.ids[r]), int(plan.q_lens[r]), int(plan.seq_lens[r])))
    tasks.sort(key=lambda t: -t[4] * t[5])          # biggest rows first
    with mp.get_context("fork").Pool(workers, _init, (job,)) as pool:
        for step, layer, r, o, l_ in pool.imap_unordered(_replay_row, tasks, chunksize=1):
            c0 = int(res[f"s{step}_cu"][r])
            res[f"s{step}_l{layer}_out"][c0:c0 + len(o)] = o
            res[f"s{step}_l{layer}_lse"][c0:c0 + len(o)] = l_
    return res


def main(argv):
    job = json.loads(argv[1])
    out_path, workers = argv[2], max(1, int(argv[3]))
    res = run_decode(job, workers) if job["kind"] == "decode" else run_replay(job, workers)
    np.savez(out_path, **res)
    print(f"[oracle_jobs] {job['kind']} done: {out_path}", flush=True)


if __name__ == "__main__":
    main(sys.argv)
