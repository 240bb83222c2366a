#!/usr/bin/env python3
"""Benchmark: one continuous-batching decode step of attention over a paged KV cache
on one MI355X, through libpkv's C ABI.

A step is the whole hot path for that batch: the cache write of the step's new K/V
(one token per sequence) followed by paged decode attention (by default the balanced
split: every resident workgroup streams an equal share of all sequences' context, then
the log-sum-exp merge of sequences split across workgroups). Inputs (cache contents,
queries, tables, the split plan) are resident in HBM before the timed region; block
tables come from libpkv's host pool.

Default workload: the large decode batch -- 256 sequences with lognormal contexts
(median 1024, sigma 1, capped at 8192), 32 query / 8 KV heads, head_dim 128, blocks
of 16 tokens, bf16, a pool 1.2x the need with shuffled block ids.

Prints one JSON line. `value` is decode HBM GB/s: algorithmic bytes of the decode
launch (K/V of every context token, queries, outputs, block-table entries, lengths)
divided by the decode time (partition pass + merge), timed with HIP events on the
launch stream around the decode call; `roofline` reports that same decode (pass +
merge) against the 8 TB/s HBM peak, and under `pass_only` the partition pass alone,
from a second run of the steps in which the library records an event between the pass
and the merge. `cpu_baseline` times the CPU oracle on a bounded prefix of the same batch
with all BLAS threads and with one, and names the host CPU.

Sub-measurements in the same line: `decode_variants` (the config-3 batch with an E4M3
cache, and config 4: 16 sequences of 32k-128k tokens, each with GB/s, fraction of peak
and the merge's share), `mixed_step` (48 decode rows + 4 prefill chunks of 512),
`swap_copy` (1 GiB of K/V to pinned host memory and back) and `sched_replay` (the
2000-request continuous-batching trace, 16 layers, with bf16 and E4M3 caches by default;
`--replays all` adds static batching, chunked prefill, swap, victim policies, priority
classes and prefix caching), each switchable off.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBS = 8000.0
METRIC = "paged-attn decode HBM GB/s (% of peak) + attention tokens/s per step"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg3", choices=["cfg3", "cfg4"])
    ap.add_argument("--no-mixed", action="store_true",
                    help="skip the mixed prefill+decode step (48 decode rows + 4 chunks of 512) sub-measurement")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-context partition (tokens; 0 = none) of the fixed-partition decode; the smallest "
                         "piece of the balanced split")
    ap.add_argument("--decode", default="split", choices=["split", "partition"],
                    help="balanced split over resident workgroup slots (default) or fixed context partitions")
    ap.add_argument("--no-replay", action="store_true",
                    help="skip the continuous-batching trace replay (2000 requests, scheduler step + 16 layers of "
                         "cache write and mixed attention per step, bf16 and E4M3 caches)")
    ap.add_argument("--replay-steps", type=int, default=None, help="replay only the first N scheduler steps")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap-copy measurement (1 GiB each way)")
    ap.add_argument("--replays", default="bf16,fp8,bf16_per_layer",
                    help="comma-separated names of the trace replays to run (default: the trace with bf16 and "
                         "E4M3 caches, layer-batched launches, and bf16 with one launch per layer; 'all' for every "
                         "variant: static batching, chunked prefill, swap, victim policies, priorities, prefix "
                         "caching)")
    ap.add_argument("--replay-batching-sweep", action="store_true",
                    help="also replay continuous vs static batching for three output-length distributions")
    ap.add_argument("--replay-budget-sweep", action="store_true",
                    help="also replay the bf16 trace under several token budgets / chunk sizes (chunked prefill)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-variants", action="store_true",
                    help="skip the config-3 E4M3-cache and config-4 (long context) decode sub-measurements")
    ap.add_argument("--probe-copy-mib", type=int, default=0,
                    help="instead of the step, time a plain device copy of this many MiB (stream bandwidth and "
                         "the known-size kernel that calibrates HBM byte counters)")
    ap.add_argument("--probe-read-mib", type=int, default=0,
                    help="instead of the step, sweep a stream-read probe over a buffer of this many MiB")
    return ap.parse_args()


def probe_read(mib: int, steps: int) -> None:
    """Achievable HBM read bandwidth: a plain streaming read at several launch shapes."""
    import torch
    import workloads.gpu as wgen
    buf = torch.empty(mib * (1 << 20), dtype=torch.uint8, device="cuda").fill_(3)
    best = None
    for blocks in (256, 512, 1024, 2048, 4096, 8192):
        for unroll in (1, 2, 4, 8):
            out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
            wgen.read_probe(buf, blocks, unroll, out)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                wgen.read_probe(buf, blocks, unroll, out)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / steps
            gbs = buf.numel() / t / 1e9
            print(json.dumps({"probe": "stream read", "bytes": buf.numel(), "blocks": blocks, "threads": 256,
                              "unroll": unroll, "us": round(t * 1e6, 2), "GBps": round(gbs, 1)}), flush=True)
            if best is None or gbs > best[0]:
                best = (gbs, blocks, unroll)
    for blocks in (256, 512, 1024, 2048):
        out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
        wgen.read_probe_stream(buf, blocks, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            wgen.read_probe_stream(buf, blocks, out)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / steps
        gbs = buf.numel() / t / 1e9
        print(json.dumps({"probe": "stream read, one share per workgroup, non-temporal", "bytes": buf.numel(),
                          "blocks": blocks, "threads": 512, "us": round(t * 1e6, 2), "GBps": round(gbs, 1)}), flush=True)
        if gbs > best[0]:
            best = (gbs, blocks, "stream")
    print(json.dumps({"probe": "stream read best", "GBps": round(best[0], 1), "blocks": best[1],
                      "unroll": best[2]}), flush=True)


def measured_read_peak() -> float:
    """Best stream-read rate of a 2 GiB buffer (GB/s) over a few launch shapes of two
    probes: a grid-stride read with plain loads, and one contiguous share per workgroup
    with non-temporal loads (the faster on MI355X): the achievable read bandwidth the
    decode rate is also compared with. The buffer is 8x the 256 MB last-level cache."""
    import torch
    import workloads.gpu as wgen
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    runs = [(lambda b=b, u=u, o=torch.empty(b * 256, dtype=torch.int32, device="cuda"): wgen.read_probe(buf, b, u, o))
            for b in (1024, 4096, 8192) for u in (4, 8)]
    runs += [(lambda b=b, o=torch.empty(b * 512, dtype=torch.int32, device="cuda"): wgen.read_probe_stream(buf, b, o))
             for b in (256, 512, 1024, 2048)]
    best = 0.0
    for run in runs:
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            run()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, buf.numel() / (e0.elapsed_time(e1) * 1e-3 / 10) / 1e9)
    del buf, runs
    torch.cuda.empty_cache()
    return best


def probe_copy(mib: int, steps: int, warmup: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    print(json.dumps({"probe": "device copy", "bytes_read": n, "bytes_written": n, "us_per_copy": round(t * 1e6, 2),
                      "read_plus_write_GBps": round(2 * n / t / 1e9, 1)}), flush=True)


def decode_bytes(w) -> int:
    """Algorithmic bytes of one decode launch (each byte the math must touch, once)."""
    import numpy as np
    e_kv = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]
    e_q = {"f32": 4, "bf16": 2}[w.dtype]
    L = w.seq_lens.astype(np.int64)
    kv = int(L.sum()) * 2 * w.num_kv_heads * w.head_dim * e_kv
    qo = w.num_seqs * w.num_q_heads * w.head_dim * 2 * e_q
    tables = int(((L + w.block_size - 1) // w.block_size).sum()) * 4
    return kv + qo + tables + w.num_seqs * 4


def write_bytes(w) -> int:
    e_in = {"f32": 4, "bf16": 2}[w.dtype]
    e_kv = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]
    T = int(w.q_lens.sum())
    return T * 2 * w.num_kv_heads * w.head_dim * (e_in + e_kv) + T * 8


def mixed_bytes_flops(w):
    """Algorithmic bytes and flops of one varlen launch over a mixed step."""
    import numpy as np
    e = 2
    L = w.seq_lens.astype(np.int64)
    q = w.q_lens.astype(np.int64)
    nbytes = int(L.sum()) * 2 * w.num_kv_heads * w.head_dim * e + int(q.sum()) * w.num_q_heads * w.head_dim * 2 * e
    nbytes += int(((L + w.block_size - 1) // w.block_size).sum()) * 4 + (2 * w.num_seqs + 1) * 4
    keys = 0
    for Ls, qs in zip(L, q):
        keys += int(qs * (Ls - qs) + qs * (qs + 1) // 2)      # row i sees L - q + i + 1 keys
    flops = keys * w.num_q_heads * w.head_dim * 4
    return nbytes, flops


def mixed_step(steps: int, warmup: int):
    """Config-2 mixed continuous-batching step: cache write of the 2096 new tokens, then the
    attention of 48 decode rows and 4 prefill chunks of 512 (causal): one launch of the
    mixed kernel (the product form: decode slots and chunk items side by side), one varlen
    launch, or split decode rows + the chunk kernel. Each timed step follows a 512 MiB cache
    flush; times are HIP events (write + attention), tokens/s = query tokens / that time."""
    import numpy as np
    import torch
    import paged_kv_cache_42_amd as pkv
    import workloads
    import workloads.gpu as wgen

    w = workloads.config2()
    pool = pkv.Pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype, free_order=w.free_order)
    for op in w.history:                       # fragment the pool with the dummy owners
        if op[0] == "alloc":
            pool.seq_reserve((1 << 40) + op[1], op[2] * w.block_size)
        else:
            pool.seq_release((1 << 40) + op[1])
    for s, L in enumerate(w.seq_lens):
        pool.seq_reserve(s, int(L))
    W = w.max_blocks_per_seq()
    ids = np.arange(w.num_seqs)
    prior = (w.seq_lens - w.q_lens).astype(np.int32)
    _, _, ctx_slots = pool.build_block_table(ids, prior, prior, W)
    bt, cu, slots = pool.build_block_table(ids, w.q_lens, w.seq_lens, W)
    Hkv, Hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    shape = (w.num_blocks, w.block_size, Hkv, d)
    kc = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    n_ctx, n_new = int(prior.sum()), int(w.q_lens.sum())
    ck = torch.empty((n_ctx, Hkv, d), dtype=torch.bfloat16, device="cuda")
    cv = torch.empty_like(ck)
    nk = torch.empty((n_new, Hkv, d), dtype=torch.bfloat16, device="cuda")
    nv = torch.empty_like(nk)
    q = torch.empty((n_new, Hq, d), dtype=torch.bfloat16, device="cuda")
    oc = on = 0
    for s in range(w.num_seqs):
        p, L = int(prior[s]), int(w.seq_lens[s])
        if p:
            wgen.fill(ck[oc:oc + p], w.value_key("k", s), 0, w.sigma)
            wgen.fill(cv[oc:oc + p], w.value_key("v", s), 0, w.sigma)
        wgen.fill(nk[on:on + L - p], w.value_key("k", s), p * Hkv * d, w.sigma)
        wgen.fill(nv[on:on + L - p], w.value_key("v", s), p * Hkv * d, w.sigma)
        wgen.fill(q[on:on + L - p], w.value_key("q", s), p * Hq * d, w.sigma)
        oc += p
        on += L - p
    pkv.kv_cache_write(ck, cv, kc, vc, torch.from_numpy(ctx_slots).cuda(), w.block_size)
    del ck, cv
    slots_d = torch.from_numpy(slots).cuda()
    bt_d = torch.from_numpy(bt).cuda()
    lens_d = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    cu_d = torch.from_numpy(cu).cuda()
    work = torch.from_numpy(pkv.build_varlen_work(w.q_lens, w.seq_lens, Hkv, w.group)).cuda()
    out = torch.empty_like(q)
    msl = int(w.seq_lens.max())
    stream = torch.cuda.current_stream()
    # the same attention as two launches: split decode rows + the chunk kernel, with the
    # chunk blocks uncut ("uncut") or cut along the keys over the resident workgroups
    dslots = pkv.decode_split_slots(pkv.BF16, Hkv, d, w.block_size)
    plans = {}
    for mode, cslots in (("uncut", 0), ("cut", pkv.chunk_slots(pkv.BF16, d, w.block_size))):
        mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, Hkv, w.group, dslots, 0, cslots)
        plans[mode] = (mp, mp.chunks.to_device(d))
    mp = plans["cut"][0]
    rows_d = torch.from_numpy(mp.decode_rows).cuda()
    plan_d = torch.from_numpy(mp.split.plan).cuda()
    ws = pkv.decode_split_workspace(mp.split, Hq, d)
    # the product form: one launch of the mixed kernel, decode slots balanced against the
    # chunk items (pkv_mixed_decode_slots), chunk blocks uncut
    mslots = pkv.mixed_decode_slots(w.q_lens, w.seq_lens, pkv.BF16, Hkv, w.group, d, w.block_size)
    mmp = pkv.build_mixed_step(w.q_lens, w.seq_lens, Hkv, w.group, mslots, 0, 0)
    mdev = mmp.to_device(d, Hq)
    mixed = pkv.paged_attention_mixed(out, q, kc, vc, bt_d, lens_d, cu_d, mmp, mdev, Hkv, w.block_size, msl,
                                      w.softmax_scale, defer=True)

    def attention(mode, emid=None):
        if mode == "one_launch":
            pkv.paged_attention_prefill_varlen(out, q, kc, vc, bt_d, lens_d, cu_d, work, Hkv, w.block_size, msl,
                                               w.softmax_scale)
            return
        if mode == "mixed":
            mixed()
            return
        pkv.paged_attention_decode_split(out, q, kc, vc, bt_d, lens_d, plan_d, mp.split, Hkv, w.block_size, msl,
                                         w.softmax_scale, 1.0, 1.0, ws, rows=rows_d, cu_seqlens_q=cu_d)
        if emid is not None:
            emid.record(stream)
        cp, (cwork, cmerges, cws) = plans[mode]
        pkv.paged_attention_prefill_chunks(out, q, kc, vc, bt_d, lens_d, cu_d, cwork, cmerges, cp.chunks.num_partials,
                                           cws, Hkv, w.block_size, msl, w.softmax_scale)

    def step(mode, e=None):
        if e is not None:
            e[0].record(stream)
        pkv.kv_cache_write(nk, nv, kc, vc, slots_d, w.block_size)
        if e is not None:
            e[1].record(stream)
        attention(mode, None if e is None else e[3])
        if e is not None:
            e[2].record(stream)

    nbytes, flops = mixed_bytes_flops(w)
    res = {"workload": f"{w.name}: 48 decode rows (context U[16,2048]) + 4 causal chunks of 512 new tokens "
                       f"after 0/512/1024/1536 cached, 32/8 heads, d 128, bs 16, bf16, fragmented pool",
           "query_tokens": n_new, "context_tokens": int(w.seq_lens.sum()),
           "attention_bytes": nbytes, "attention_flops": flops}
    names = {"mixed": "one_launch_mixed", "one_launch": "one_launch", "uncut": "split_decode_plus_chunks_uncut",
             "cut": "split_decode_plus_chunks"}
    # the step's working set (~250 MB) fits in the last-level cache: evict it before every
    # timed step (outside the events) by streaming a 512 MiB buffer through the caches. A
    # read, not a write: a written flush leaves dirty lines whose write-back the next step
    # would pay for.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    flush_out = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    for two in names:
        for _ in range(warmup):
            step(two)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            wgen.read_probe(flush, 4096, 4, flush_out)
            step(two, ev[i])
        torch.cuda.synchronize()
        wall = float(np.mean([e[0].elapsed_time(e[2]) for e in ev])) * 1e-3     # write + attention
        t_w = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
        t_a = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
        parts = {}
        if two in ("uncut", "cut"):
            parts = {"decode_rows": round(float(np.mean([e[1].elapsed_time(e[3]) for e in ev])) * 1e3, 2),
                     "chunks": round(float(np.mean([e[3].elapsed_time(e[2]) for e in ev])) * 1e3, 2)}
        res[names[two]] = {
            "ms_per_step": round(wall * 1e3, 4),
            "kernel_us": {"kv_cache_write": round(t_w * 1e6, 2), "attention": round(t_a * 1e6, 2), **parts},
            "tokens_per_s": round(n_new / wall, 1),
            "hbm_GBps": round(nbytes / t_a / 1e9, 1), "hbm_frac": round(nbytes / t_a / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_TFLOPs": round(flops / t_a / 1e12, 1), "mfma_frac": round(flops / t_a / 1e12 / 2500.0, 4)}
        if two == "mixed":
            res[names[two]]["decode_slots"] = mslots
    res["product_form"] = "one_launch_mixed"
    return res


def swap_bench(reps: int = 5):
    """Preemption by swap at the trace geometry (16 layers, 4,096 blocks of 16 tokens, 8 KV
    heads x 64, bf16): 2,048 blocks = 1 GiB of K/V out to pinned host memory and back,
    with the host blocks in one run and scattered; a plain DMA copy of 1 GiB each way
    (contiguous device buffer <-> pinned host buffer) as the link's ceiling."""
    import torch
    import numpy as np
    import paged_kv_cache_42_amd as pkv
    import workloads
    tr = workloads.config5("bf16")
    L, nb = tr.num_layers, tr.num_blocks
    k = torch.zeros((L, nb, tr.block_size, tr.num_kv_heads, tr.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    block_bytes = k[0, 0].numel() * 2
    n = 2048
    nbytes = n * L * 2 * block_bytes
    hs = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    ws = torch.empty(pkv.swap_workspace_bytes(n, L, block_bytes), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(31)
    dev = rng.permutation(nb)[:n].astype(np.int32)
    res = {"bytes_each_way": nbytes, "pages_model": "2 x KV bytes / PCIe bandwidth; 1 GB round trip ~80 ms on Gen4"}

    def timed(fn):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts[1:]))

    for name, host in (("one_run", np.arange(n, dtype=np.int32)), ("scattered", rng.permutation(n).astype(np.int32))):
        t_out = timed(lambda: pkv.swap_out(k, v, np.stack([dev, host], 1), hs, ws))
        t_in = timed(lambda: pkv.swap_in(k, v, np.stack([host, dev], 1), hs, ws))
        res[name] = {"swap_out_ms": round(t_out * 1e3, 3), "swap_in_ms": round(t_in * 1e3, 3),
                     "round_trip_ms": round((t_out + t_in) * 1e3, 3),
                     "GBps_out": round(nbytes / t_out / 1e9, 1), "GBps_in": round(nbytes / t_in / 1e9, 1)}
    d2h = timed(lambda: hs.copy_(ws[:nbytes], non_blocking=True))
    h2d = timed(lambda: ws[:nbytes].copy_(hs, non_blocking=True))
    res["dma_only"] = {"d2h_ms": round(d2h * 1e3, 3), "h2d_ms": round(h2d * 1e3, 3),
                       "GBps_d2h": round(nbytes / d2h / 1e9, 1), "GBps_h2d": round(nbytes / h2d / 1e9, 1)}
    del k, v, hs, ws
    torch.cuda.empty_cache()
    return res


# the budgets of the continuous-batching page's tuning exercise (the budget alone bounds
# the chunks), then budget / chunk pairs with a 512-token chunk cap
def replay_batching_sweep(max_steps):
    """Continuous vs static batching on the trace with three output-length distributions
    (constant, geometric, lognormal with a long tail): the gain's dependence on the
    spread of output lengths."""
    import workloads
    from workloads import replay
    out = {}
    for kind in ("constant", "geometric", "lognormal"):
        res = {}
        for mode in ("continuous", "static"):
            print(f"[bench] batching sweep {kind} {mode}", file=sys.stderr, flush=True)
            _, summ = replay.run(workloads.config5_outputs(kind), max_steps=max_steps,
                                 static_batching=mode == "static")
            res[mode] = {k: summ[k] for k in ("steps", "attention_s_total", "requests_per_s", "avg_running_batch",
                                              "ttft_ms", "tbt_ms", "preemptions")}
        c, st = res["continuous"], res["static"]
        res["gain_requests_per_s"] = round(c["requests_per_s"] / st["requests_per_s"], 2)
        res["batch_ratio"] = round(c["avg_running_batch"] / st["avg_running_batch"], 2)
        res["ttft_p50_ratio"] = round(st["ttft_ms"]["p50"] / c["ttft_ms"]["p50"], 2)
        out[kind] = res
    return out


BUDGET_SWEEP = ((512, 0), (2048, 0), (8192, 0), (32768, 0), (1024, 512), (2048, 512), (4096, 1024))


def replay_budget_sweep(max_steps):
    """The bf16 trace under per-step token budgets with chunked prefill (key-cut chunk
    work): the prefill-throughput / decode-latency trade of the budget."""
    import workloads
    from workloads import replay
    out = {}
    for budget, chunk in BUDGET_SWEEP:
        name = f"budget_{budget}_chunk_{chunk}"
        print(f"[bench] replay sweep {name}", file=sys.stderr, flush=True)
        _, summ = replay.run(workloads.config5("bf16"), max_steps=max_steps, token_budget=budget,
                             chunk_tokens=chunk, chunk_cut=True)
        out[name] = summ
    return out


def sched_replay(max_steps, only=None):
    """Continuous-batching trace replay (the 2000-request trace): per step the host
    scheduler admits/plans/updates and 16 layers run the cache write and the mixed
    attention launch; per-step attention time from HIP events (inputs generated on the
    device before each step's timed region)."""
    import workloads
    from workloads import replay
    out = {}
    runs = [("bf16", workloads.config5("bf16"), {}), ("fp8", workloads.config5("fp8"), {}),
            # steps with decode rows and prefill chunks as two launches (split decode, then
            # the chunk kernel) instead of one launch of the mixed kernel
            ("bf16_two_launches", workloads.config5("bf16"), {"one_launch": False}),
            ("fp8_two_launches", workloads.config5("fp8"), {"one_launch": False}),
            # one launch per kernel and layer, as a model running its layers in turn issues
            # them (the runs above launch each kernel once per step for all 16 layers)
            ("bf16_per_layer", workloads.config5("bf16"), {"layer_batched": False}),
            ("fp8_per_layer", workloads.config5("fp8"), {"layer_batched": False}),
            # the static-batching baseline continuous batching is measured against
            ("bf16_static_batching", workloads.config5("bf16"), {"static_batching": True}),
            # chunked prefill: at most 2048 new tokens per step, prefills in chunks of 512
            ("bf16_chunked_2048_512", workloads.config5("bf16"),
             {"token_budget": 2048, "chunk_tokens": 512, "chunk_cut": True}),
            # preemption by swap into a host space of 4096 blocks (instead of recompute)
            ("bf16_swap", workloads.config5("bf16"), {"swap_blocks": 4096}),
            ("bf16_swap_overlap", workloads.config5("bf16"), {"swap_blocks": 4096, "swap_overlap": True}),
            # victim policies (LIFO; fewest generated) and priority admission (25% premium)
            ("bf16_victim_lifo", workloads.config5("bf16"), {"victim": "lifo"}),
            ("bf16_victim_fewest", workloads.config5("bf16"), {"victim": "fewest"}),
            ("bf16_fcfs_classes", workloads.config5("bf16"), {"classes": True}),
            ("bf16_priority", workloads.config5("bf16"), {"priority": True}),
            ("bf16_priority_lifo", workloads.config5("bf16"), {"priority": True, "victim": "lifo"}),
            # shared system prompts (16 groups), with and without the prefix cache
            ("bf16_prefix_cache", workloads.config5_prefix("bf16"), {}),
            ("bf16_prefix_trace_no_cache", workloads.config5_prefix("bf16"), {"prefix_cache": False})]
    if only:
        unknown = set(only) - {r[0] for r in runs}
        if unknown:
            raise SystemExit(f"unknown replay names: {sorted(unknown)}")
        runs = [r for r in runs if r[0] in only]
    for name, tr, kw in runs:
        print(f"[bench] replay {name}: {tr.name} {kw}", file=sys.stderr, flush=True)
        args = dict(kw)
        for key in ("priority", "classes"):    # 25% premium (class 0), 75% bulk (class 1)
            if args.get(key):
                args[key] = workloads.priority_classes(tr)
        _, summ = replay.run(tr, max_steps=max_steps, **args,
                             progress=lambda n: print(f"[bench] replay {name}: {n} steps", file=sys.stderr, flush=True))
        summ.update({k: v for k, v in kw.items() if k != "prefix_cache"})
        out[name] = summ
    return out


def measured_traffic(partition: int, workload: str, decode: str):
    """HBM bytes of one decode (the split pass and its log-sum-exp merge, per launch pair)
    from the committed rocprofv3 counter record, valid only while the profiled kernel
    sources are unchanged (else None)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    rec = os.path.join(here, "profiles", f"decode_{decode}_pass__cfg3_large_decode_bf16.counters.json")
    if workload != "cfg3" or not os.path.exists(rec):
        return None
    r = json.load(open(rec))
    h = hashlib.sha256()
    for f in r.get("sources", [r.get("source", "")]):          # the kernel's file and its headers
        src = os.path.join(here, f)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if h.hexdigest() != r.get("sources_sha256", r.get("source_sha256")):
        return None
    if r.get("partition_size", 512) != partition or r.get("decode", "partition") != decode:
        return None
    return int(r["traffic_bytes"])


def setup_device(w, partition):
    """Pool + tables (libpkv host), K/V generated on the GPU, context written by the
    cache-write kernel (E4M3-encoded for an fp8 cache); returns the tensors of one
    decode step."""
    import numpy as np
    import torch
    import paged_kv_cache_42_amd as pkv
    import workloads.gpu as wgen

    pool = pkv.Pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype, free_order=w.free_order)
    for s, L in enumerate(w.seq_lens):
        pool.seq_reserve(s, int(L))
    W = w.max_blocks_per_seq()
    ids = np.arange(w.num_seqs)
    prior = (w.seq_lens - w.q_lens).astype(np.int32)
    _, _, ctx_slots = pool.build_block_table(ids, prior, prior, W)
    bt, cu, slots = pool.build_block_table(ids, w.q_lens, w.seq_lens, W)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[w.cache_dtype]
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    k_cache = torch.empty(shape, dtype=cdt, device="cuda")
    v_cache = torch.empty(shape, dtype=cdt, device="cuda")
    Hkv, Hq, d = w.num_kv_heads, w.num_q_heads, w.head_dim
    n_new = int(w.q_lens.sum())
    new_k = torch.empty((n_new, Hkv, d), dtype=dt, device="cuda")
    new_v = torch.empty_like(new_k)
    q = torch.empty((n_new, Hq, d), dtype=dt, device="cuda")
    # the context is written in chunks of sequences to bound the staging buffers
    on = 0
    chunk_tokens = 1 << 20
    s0 = 0
    slot_off = 0
    while s0 < w.num_seqs:
        s1, tok = s0, 0
        while s1 < w.num_seqs and (tok == 0 or tok + int(prior[s1]) <= chunk_tokens):
            tok += int(prior[s1])
            s1 += 1
        ck = torch.empty((tok, Hkv, d), dtype=dt, device="cuda")
        cv = torch.empty_like(ck)
        o = 0
        for s in range(s0, s1):
            p = int(prior[s])
            if p:
                wgen.fill(ck[o:o + p], w.value_key("k", s), 0, w.sigma)
                wgen.fill(cv[o:o + p], w.value_key("v", s), 0, w.sigma)
            o += p
        if tok:
            sl = torch.from_numpy(ctx_slots[slot_off:slot_off + tok].copy()).cuda()
            pkv.kv_cache_write(ck, cv, k_cache, v_cache, sl, w.block_size, w.k_scale, w.v_scale)
        slot_off += tok
        s0 = s1
        del ck, cv
    for s in range(w.num_seqs):
        p, L = int(prior[s]), int(w.seq_lens[s])
        wgen.fill(new_k[on:on + L - p], w.value_key("k", s), p * Hkv * d, w.sigma)
        wgen.fill(new_v[on:on + L - p], w.value_key("v", s), p * Hkv * d, w.sigma)
        wgen.fill(q[on:on + L - p], w.value_key("q", s), p * Hq * d, w.sigma)
        on += L - p
    msl = int(w.seq_lens.max())
    work = torch.from_numpy(pkv.build_decode_work(w.seq_lens, partition)).cuda()
    ws_bytes = pkv.decode_workspace_bytes(w.num_seqs, Hq, d, msl, partition)
    # balanced split: the plan for the slots that fill this device
    split = pkv.build_decode_split(w.seq_lens, pkv.decode_split_slots({"bf16": pkv.BF16, "fp8": pkv.FP8}.get(w.cache_dtype, pkv.BF16), Hkv,
                                                                      d, w.block_size), partition)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ws_split = pkv.decode_split_workspace(split, Hq, d)
    torch.cuda.synchronize()
    return dict(pool=pool, k_cache=k_cache, v_cache=v_cache, new_k=new_k, new_v=new_v, q=q,
                out=torch.empty_like(q), slots=torch.from_numpy(slots).cuda(), bt=torch.from_numpy(bt).cuda(),
                lens=torch.from_numpy(w.seq_lens.astype(np.int32)).cuda(), ws=ws, ws_split=ws_split,
                max_seq_len=msl, work=work,
                split=split, plan=torch.from_numpy(split.plan).cuda())


def time_decode_step(w, P, decode_kind, steps, warmup):
    """The decode step of workload w (cache write of its new tokens, then decode attention)
    timed with HIP events on the launch stream: K steps as a caller runs them, then K more
    with the library recording an event between the pass and the merge. Returns the
    per-step event times (seconds, numpy arrays), the wall time of the first run and the
    device tensors."""
    import numpy as np
    import torch
    import paged_kv_cache_42_amd as pkv

    dev = setup_device(w, P)
    stream = torch.cuda.current_stream()
    scale = w.softmax_scale

    # the calls are checked and marshalled once (as a serving loop would), so a timed step
    # waits on no host-side argument checks between its launches
    write = pkv.kv_cache_write(dev["new_k"], dev["new_v"], dev["k_cache"], dev["v_cache"], dev["slots"],
                               w.block_size, w.k_scale, w.v_scale, defer=True)
    if decode_kind == "split":
        decode = pkv.paged_attention_decode_split(dev["out"], dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"],
                                                  dev["lens"], dev["plan"], dev["split"], w.num_kv_heads,
                                                  w.block_size, dev["max_seq_len"], scale, w.k_scale, w.v_scale,
                                                  dev["ws_split"], defer=True)
    else:
        def decode():
            pkv.paged_attention_decode(dev["out"], dev["q"], dev["k_cache"], dev["v_cache"], dev["bt"], dev["lens"],
                                       w.num_kv_heads, w.block_size, dev["max_seq_len"], scale, w.k_scale,
                                       w.v_scale, P, dev["ws"], work=dev["work"])

    for _ in range(warmup):
        write()
        decode()
    torch.cuda.synchronize()

    def timed(profile: bool):
        """K steps bracketed by events (write | decode); with profile=True the library also
        records an event between the partition pass and the merge (which adds its own gap)."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in ev:        # materialise the event handles before use by the library hook
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            e0, e1, e2, e3 = ev[i]
            e0.record(stream)
            write()
            e1.record(stream)
            if profile:
                pkv.decode_set_profile_event(e2)
            decode()
            if profile:
                pkv.decode_set_profile_event(None)
            e3.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in ev]) * 1e-3
        return wall, ms(0, 1), ms(1, 3), ms(0, 3), (ms(1, 2) if profile else None), (ms(2, 3) if profile else None)

    # the step as a caller runs it, then again with the pass/merge split point
    wall, t_write, t_decode, t_step, _, _ = timed(False)
    _, _, _, _, t_part, t_merge = timed(True)
    return dict(wall=wall, write=t_write, decode=t_decode, step=t_step, part=t_part, merge=t_merge, dev=dev)


# Warmup steps of the decode sub-measurements (not the headline, which takes --warmup as
# given): after the idle setup of a workload the first few hundred microseconds of GPU
# work run slow, and the E4M3 decode (less memory-bound than bf16) reads 5-20 us high
# after 5 steps, steady after 50.
SUB_WARMUP = 50


def decode_record(w, P, decode_kind, steps, warmup):
    """A decode sub-measurement: GB/s of the decode (pass + merge), its fraction of the
    8 TB/s peak, the pass alone, and the merge's share of the decode time (at least
    SUB_WARMUP warmup steps first)."""
    import numpy as np
    import torch
    warmup = max(warmup, SUB_WARMUP)
    r = time_decode_step(w, P, decode_kind, steps, warmup)
    dbytes = decode_bytes(w)
    t_dec, t_part, t_merge = float(r["decode"].mean()), float(r["part"].mean()), float(r["merge"].mean())
    split = r["dev"]["split"]
    out = {"workload": w.name, "cache_dtype": w.cache_dtype, "num_seqs": w.num_seqs,
           "context_tokens": int(w.seq_lens.sum()), "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
           "head_dim": w.head_dim, "block_size": w.block_size, "decode": decode_kind,
           "steps": steps, "warmup": warmup, "algorithmic_bytes": dbytes,
           "decode_us": round(t_dec * 1e6, 2), "decode_GBps": round(dbytes / t_dec / 1e9, 1),
           "decode_frac_of_peak": round(dbytes / t_dec / 1e9 / PEAK_HBM_GBS, 4),
           "pass_us_profiled": round(t_part * 1e6, 2), "merge_us_profiled": round(t_merge * 1e6, 2),
           "pass_GBps": round(dbytes / t_part / 1e9, 1),
           "pass_frac_of_peak": round(dbytes / t_part / 1e9 / PEAK_HBM_GBS, 4),
           "merge_share_of_decode": round(t_merge / (t_part + t_merge), 4),
           "tokens_per_s": round(w.num_seqs / float(r["step"].mean()), 1)}
    if decode_kind == "split":
        out.update(split_slots=split.num_slots, split_tiles_per_slot=split.tiles_per_slot,
                   split_max_pieces=split.max_pieces)
    del r
    torch.cuda.empty_cache()
    return out


def scheduler_host():
    """libpkv's scheduler step on the host over the whole 2000-request trace (schedule,
    plan with block tables / cu_seqlens / slot mapping, update), driven through the
    Python binding: microseconds per step, no GPU work; at the trace's 128-request cap
    and at caps of 8 and 256 (the batch sizes of the page's scheduler-cost exercise)."""
    out = _scheduler_host_run(128)
    # cap 256 with a 4x pool, so that the cap (not the memory) bounds the batch
    out["by_max_running"] = {"8": _scheduler_host_run(8), "256 (16384-block pool)": _scheduler_host_run(256, 16384)}
    return out


def _scheduler_host_run(max_running, num_blocks=None):
    import dataclasses
    import numpy as np
    import paged_kv_cache_42_amd as pkv
    import workloads
    tr = dataclasses.replace(workloads.config5("bf16"), max_running=max_running)
    if num_blocks:
        tr = dataclasses.replace(tr, num_blocks=num_blocks,
                                 free_order=np.random.default_rng(5).permutation(num_blocks).astype(np.int32))
    pool = pkv.Pool(tr.num_blocks, tr.block_size, tr.num_kv_heads, tr.head_dim, tr.cache_dtype,
                    free_order=tr.free_order)
    sched = pkv.Scheduler(pool, tr.max_running)
    sched.add_requests(np.arange(tr.num_requests), tr.arrival, tr.prompt, tr.max_tokens)
    width = -(-int((tr.prompt + tr.max_tokens - 1).max()) // tr.block_size)
    steps = rows = 0
    t0 = time.perf_counter()
    while sched.counters()["finished"] < tr.num_requests:
        n, q, _ = sched.schedule()
        if n:
            sched.plan(n, q, width)
        sched.update()
        steps += 1
        rows += n
    dt = time.perf_counter() - t0
    return {"steps": steps, "avg_rows": round(rows / steps, 1), "us_per_step": round(dt / steps * 1e6, 1),
            "note": "C++ step through the ctypes binding (plan arrays allocated per step)"}


def scheduler_oracle(budget_s: float):
    """The scheduler oracle (plain Python) on the same trace, for at most budget_s seconds."""
    import workloads
    from oracle import scheduler as osch
    tr = workloads.config5("bf16")
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running)
    width = -(-int((tr.prompt + tr.max_tokens - 1).max()) // tr.block_size)
    steps = rows = 0
    t0 = time.perf_counter()
    for plan, _ in osch.run(ref, width):
        steps += 1
        rows += len(plan.ids)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(dt / steps * 1e6, 1), "unit": "us per scheduler step", "cores": 1, "kind": "oracle",
            "sample": f"first {steps} steps of the 2000-request trace ({rows / steps:.1f} rows per step on "
                      f"average), pure Python, one thread, {dt:.1f} s"}


def cpu_info() -> dict:
    """The host the oracle runs on: CPU model, logical CPUs, the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, budget_s: float):
    """The oracle (float64 NumPy, as it stands) on a prefix of the batch, sequence by
    sequence, until `budget_s` seconds of oracle time; inputs prepared untimed. Timed twice:
    with NumPy's BLAS on all the threads it starts with (the headline value), and with one
    BLAS thread."""
    import numpy as np
    import workloads
    from oracle import attention as oatt
    from oracle import cache as ocache
    from oracle.allocator import BlockPool, SeqTables
    from oracle.metadata import build_block_table
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1

    tabs = SeqTables(BlockPool(w.num_blocks, w.free_order), w.block_size)
    for s, L in enumerate(w.seq_lens):
        tabs.reserve(s, int(L))
    kp = np.zeros((w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim), np.uint16)
    vp = np.zeros_like(kp)
    # prepare (untimed) as many sequences as a preparation budget allows
    prep = []
    t_prep = time.perf_counter()
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        t = [tabs.tables[s]]
        _, _, slots = build_block_table(t, [L], [L], w.block_size, len(t[0]))
        k, v = w.kv(s)
        ocache.write(kp, k, w.dtype, w.cache_dtype, slots)
        ocache.write(vp, v, w.dtype, w.cache_dtype, slots)
        bt, cu, _ = build_block_table(t, [1], [L], w.block_size, len(t[0]))
        prep.append((L, bt, cu, workloads.storage_to_f64(w.q(s), w.dtype)))
        if time.perf_counter() - t_prep > 4 * budget_s:
            break
    e_kv = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]

    def timed(items, budget):
        """Whole passes of the oracle over `items` until `budget` seconds are spent."""
        spent, passes = 0.0, 0
        while spent < budget and passes < 100:
            t0 = time.perf_counter()
            for L, bt, cu, q in items:
                oatt.paged_attention(q, kp, vp, w.cache_dtype, bt, [L], cu, w.softmax_scale, w.group)
            spent += time.perf_counter() - t0
            passes += 1
        tokens = sum(p[0] for p in items)
        nbytes = tokens * 2 * w.num_kv_heads * w.head_dim * e_kv
        return nbytes * passes / spent / 1e9, tokens, nbytes, passes, spent

    gbs, tokens, nbytes, passes, spent = timed(prep, budget_s)
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"first {len(prep)} of {w.num_seqs} sequences ({tokens} context tokens, {nbytes / 1e9:.3f} GB "
                     f"of K/V), {passes} pass(es) of the float64 NumPy oracle in {spent:.1f} s; cores = BLAS threads",
           **cpu_info(), "blas_threads": int(threads)}
    if threadpool_limits is not None:
        # one thread: the longest prefix of the prepared sequences one pass of which fits
        # in the budget (the rate is per byte, so a prefix measures it)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            n = 0
            while n < len(prep) and time.perf_counter() - t0 < budget_s / 2:
                L, bt, cu, q = prep[n]
                oatt.paged_attention(q, kp, vp, w.cache_dtype, bt, [L], cu, w.softmax_scale, w.group)
                n += 1
            g1, tok1, nb1, p1, sp1 = timed(prep[:max(n, 1)], budget_s / 2)
        res["single_thread"] = {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                                "sample": f"first {max(n, 1)} sequences ({tok1} context tokens, {nb1 / 1e9:.3f} GB of "
                                          f"K/V), {p1} pass(es) in {sp1:.1f} s with one BLAS thread"}
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.probe_copy_mib:
        probe_copy(args.probe_copy_mib, args.steps, args.warmup)
        return
    if args.probe_read_mib:
        probe_read(args.probe_read_mib, args.steps)
        return
    import dataclasses
    import numpy as np
    import torch
    import workloads

    w = workloads.config3() if args.workload == "cfg3" else workloads.config4()
    P = w.partition_size if args.partition is None else args.partition
    print(f"[bench] {w.name}: B={w.num_seqs} sumL={int(w.seq_lens.sum())} P={P}; setting up", file=sys.stderr,
          flush=True)
    K = args.steps
    r = time_decode_step(w, P, args.decode, K, args.warmup)
    dev = r["dev"]
    dbytes = decode_bytes(w)
    t_dec = float(r["decode"].mean())
    gbs = dbytes / t_dec / 1e9
    part_gbs = dbytes / float(r["part"].mean()) / 1e9
    ms_step = r["wall"] / K * 1e3
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype,
        "data": "synthetic (seeded counter-hash values, Irwin-Hall(3) approximation of N(0,1), exact in bf16)",
        "config": {"workload": f"{w.name}: {w.num_seqs} decode rows, context lognormal median 1024 sigma 1 cap 8192"
                               if args.workload == "cfg3" else
                               f"{w.name}: {w.num_seqs} decode rows, context U[32k,128k]",
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "context_tokens": int(w.seq_lens.sum()),
                   "partition_size": P, "num_blocks": w.num_blocks, "decode": args.decode,
                   **({"split_slots": dev["split"].num_slots, "split_tiles_per_slot": dev["split"].tiles_per_slot}
                      if args.decode == "split" else {})},
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "pct_of_measured_read_peak": None,
        "tokens_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "context_tokens_per_s": round(float(w.seq_lens.sum()) / (ms_step * 1e-3), 1),
        "kernel_us": {"kv_cache_write": round(float(r["write"].mean()) * 1e6, 2),
                      "decode": round(t_dec * 1e6, 2),
                      "decode_median": round(float(np.median(r["decode"])) * 1e6, 2),
                      "decode_min": round(float(r["decode"].min()) * 1e6, 2),
                      "step_events": round(float(r["step"].mean()) * 1e6, 2),
                      "profiled_partition_pass": round(float(r["part"].mean()) * 1e6, 2),
                      "profiled_merge": round(float(r["merge"].mean()) * 1e6, 2)},
        # the decode as a caller runs it: the partition pass and the log-sum-exp merge
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(P, args.workload, args.decode),
                     "kernel": "decode: partition pass + log-sum-exp merge (HIP events around both launches)",
                     "algorithmic_bytes": dbytes,
                     "pass_only": {"achieved": round(part_gbs, 2), "frac": round(part_gbs / PEAK_HBM_GBS, 4),
                                   "us": round(float(r["part"].mean()) * 1e6, 2)}},
        "cpu_baseline": None,
    }
    del r, dev
    torch.cuda.empty_cache()
    rp = measured_read_peak()
    res["measured_read_peak_GBps"] = round(rp, 1)
    res["pct_of_measured_read_peak"] = round(100 * gbs / rp, 2)
    if not args.no_decode_variants:
        # the other decode shapes the workloads name: config 3 with an E4M3 cache (half the
        # bytes) and config 4 (long contexts, split context merged by log-sum-exp), bf16 and E4M3
        res["decode_variants"] = {}
        for name, wv in (("cfg3_e4m3_cache", dataclasses.replace(workloads.config3(), cache_dtype="fp8")),
                         ("cfg4_long_context_bf16", workloads.config4()),
                         ("cfg4_e4m3_cache", dataclasses.replace(workloads.config4(), cache_dtype="fp8"))):
            print(f"[bench] decode variant {name}", file=sys.stderr, flush=True)
            res["decode_variants"][name] = decode_record(wv, wv.partition_size, "split", K, args.warmup)
    if not args.no_mixed:
        print("[bench] mixed prefill+decode step", file=sys.stderr, flush=True)
        res["mixed_step"] = mixed_step(args.steps, args.warmup)
    if not args.no_swap:
        print("[bench] swap copies", file=sys.stderr, flush=True)
        res["swap_copy"] = swap_bench()
    if not args.no_replay:
        res["sched_replay"] = sched_replay(args.replay_steps,
                                           None if args.replays == "all" else args.replays.split(","))
    if args.replay_budget_sweep:
        res["replay_budget_sweep"] = replay_budget_sweep(args.replay_steps)
    if args.replay_batching_sweep:
        res["replay_batching_sweep"] = replay_batching_sweep(args.replay_steps)
    if not args.no_replay:
        res["scheduler_host"] = scheduler_host()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        if not args.no_replay:
            res["cpu_baseline"]["scheduler"] = scheduler_oracle(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
