"""Trace replay on the GPU: libpkv's scheduler step drives the cache write and the
mixed (prefill + decode) attention launch of every layer, step after step.

Benchmark and test infrastructure. Per step: the host scheduler admits, plans and
updates (C ABI); the step's metadata goes to the device once for all layers; the Q/K/V
of every new token of every layer are generated on the device by the counter-hash
generator (outside the timed region), then the cache write, the balanced-split decode
over the step's decode rows and the chunk kernel over its prefill chunks run for every
layer, bracketed by HIP events per step: by default each kernel once for all layers (the
layer-batched entry points; the layers' inputs here are independent streams), or one
launch per kernel and layer (layer_batched=False), as a model that runs its layers in
turn would issue them. A step with both decode rows and prefill chunks runs them in one
launch of the mixed kernel (one_launch, the default), decode slots beside chunk items."""
from __future__ import annotations

import dataclasses
import time
from typing import Dict, List, Optional, Sequence

import numpy as np

import paged_kv_cache_42_amd as pkv
import workloads
from workloads import gpu as wgen


@dataclasses.dataclass
class StepRecord:
    step: int
    rows: int
    q_tokens: int
    context_tokens: int
    prefill_rows: int
    attention_bytes: int         # algorithmic HBM bytes of the step's 16-layer write + attention
    ev: tuple                    # (start, end) events around the layers' write + attention
    kept: Dict[int, object]      # layer -> output tensor [T][Hq][d] (only for kept layers)
    plan: Optional[object] = None
    first_outputs: Sequence[int] = ()   # requests whose first output token this step made
    host_s: float = 0.0          # host time to enqueue the step's layers (between the events)
    swap_ev: tuple = ()          # (swap-in end event, swap-out start, swap-out end) or None entries
    swap_blocks: tuple = (0, 0)  # (blocks swapped in before the layers, swapped out after the update)
    decode_by_class: tuple = ()  # decode rows per priority class (priority replays)


class Replay:
    """One trace replay: libpkv's scheduler over a pool, 16 layers of K/V planes on the
    device, and the options of the scheduler and the launches:
      chunk_cut / min_piece_tiles: cut long chunk blocks along the keys (chunk kernel);
      prefix_cache: prefix caching for traces with shared system prompts;
      token_budget / chunk_tokens: chunked prefill under a per-step token budget;
      swap_blocks / swap_overlap: preemption by swap into pinned host memory (the DMA
        leg of swap-outs on a copy stream when overlapped);
      victim, priority, classes: victim policy, priority classes for admission, or
        classes used only to report latencies by;
      static_batching: the static-batching baseline;
      layer_batched: one launch per kernel for all layers (else one per layer);
      one_launch: a step with decode rows and prefill chunks runs both in one launch
        (pkv_paged_attention_mixed) over pkv_mixed_decode_slots decode slots."""

    def __init__(self, tr: workloads.Trace, chunk_cut: bool = False, min_piece_tiles: int = 0,
                 prefix_cache: bool = True, token_budget: int = 0, chunk_tokens: int = 0, swap_blocks: int = 0,
                 swap_overlap: bool = False, victim: str = "self", priority=None, classes=None,
                 static_batching: bool = False, layer_batched: bool = True, one_launch: bool = True):
        import torch
        self.torch = torch
        self.tr = tr
        self.pool = pkv.Pool(tr.num_blocks, tr.block_size, tr.num_kv_heads, tr.head_dim, tr.cache_dtype,
                             free_order=tr.free_order)
        self.sched = pkv.Scheduler(self.pool, tr.max_running)
        self.sched.add_requests(np.arange(tr.num_requests), tr.arrival, tr.prompt, tr.max_tokens)
        self.width = -(-int((tr.prompt + tr.max_tokens - 1).max()) // tr.block_size)
        shape = (tr.num_layers, tr.num_blocks, tr.block_size, tr.num_kv_heads, tr.head_dim)
        if tr.cache_dtype == "fp8":
            self.k_cache = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        else:
            self.k_cache = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        self.v_cache = torch.zeros_like(self.k_cache)
        # stream keys of (layer, kind, owner), kind = q, k, v; owners = requests, then groups
        groups = 0 if tr.prefix_group is None else int(tr.prefix_group.max()) + 1
        self.keys = np.zeros((tr.num_layers, 3, tr.num_requests + groups), np.uint64)
        for l in range(tr.num_layers):
            for k, which in enumerate("qkv"):
                self.keys[l, k] = [tr.value_key(which, l, o) for o in
                                   list(range(tr.num_requests)) + [workloads.GROUP_OWNER + g for g in range(groups)]]
        if prefix_cache and tr.prefix_group is not None:     # shared system prompts
            self.sched.enable_prefix_cache([tr.prompt_tokens(r) for r in range(tr.num_requests)])
        if token_budget or chunk_tokens:                       # chunked prefill
            self.sched.set_token_budget(token_budget, chunk_tokens)
        self.n_out = np.zeros(tr.num_requests, np.int64)        # outputs per request so far
        if victim != "self":
            self.sched.set_victim_policy(victim)
        if static_batching:                                    # the static-batching baseline
            self.sched.set_static_batching(True)
        self.priority = None if priority is None else np.asarray(priority, np.int32)
        if self.priority is not None:                          # priority admission
            self.sched.set_priorities(np.arange(tr.num_requests), self.priority)
        # classes to report latencies by (the priority classes, or labels only)
        self.classes = self.priority if classes is None else np.asarray(classes, np.int32)
        self.host_space = self.swap_ws = None
        if swap_blocks:                                        # preemption by swap
            self.sched.enable_swap(swap_blocks)
            block_bytes = self.k_cache[0, 0].numel() * self.k_cache.element_size()
            self.pair_bytes = tr.num_layers * 2 * block_bytes
            self.host_space = torch.empty(swap_blocks * self.pair_bytes, dtype=torch.uint8, pin_memory=True)
        # swap-outs' DMA leg on a copy stream, overlapping the next steps; any later swap
        # call waits for it (it reuses the workspace and may read those host blocks)
        self.copy_stream = torch.cuda.Stream() if swap_overlap else None
        self.heads = np.array([tr.num_q_heads, tr.num_kv_heads, tr.num_kv_heads], np.int64)
        self.buf = None
        self.e_kv = 1 if tr.cache_dtype == "fp8" else 2
        resident = pkv.decode_split_slots(pkv.FP8 if tr.cache_dtype == "fp8" else pkv.BF16, tr.num_kv_heads,
                                          tr.head_dim, tr.block_size)
        self.min_piece = 256
        # The split decode's slots: the workgroups resident at once. When the layers share
        # a launch, its grid holds every layer's slots, so each layer's plan takes its share
        # of them (fewer, longer pieces per layer: fewer partials to merge).
        self.layer_batched = layer_batched
        nl = tr.num_layers if layer_batched else 1
        self.slots = max(1, -(-resident // nl))
        # the workspace (its size depends only on the slots and the heads; one plan's
        # partials per layer when the layers share a launch)
        self.split_ws = torch.empty(pkv.decode_split_workspace_bytes(self.slots, tr.num_q_heads, tr.head_dim, 2) * nl,
                                    dtype=torch.uint8, device="cuda")
        cs = pkv.chunk_slots(pkv.FP8 if tr.cache_dtype == "fp8" else pkv.BF16, tr.head_dim, tr.block_size)
        self.chunk_slots = max(1, -(-cs // nl)) if chunk_cut else 0
        self.min_piece_tiles = min_piece_tiles
        self.one_launch = one_launch

    def _values(self, ids, q_lens, seq_lens):
        """Generate Q/K/V of the step's new tokens for every layer into one buffer; return
        per-layer views (q [T][Hq][d], k [T][Hkv][d], v [T][Hkv][d]). A row's positions may
        come from two streams (a group's shared prompt, then the request's own tokens)."""
        torch, tr = self.torch, self.tr
        T, d, NL = int(q_lens.sum()), tr.head_dim, tr.num_layers
        per_layer = T * d * int(self.heads.sum())
        if self.buf is None or self.buf.numel() < NL * per_layer:
            self.buf = torch.empty(max(NL * per_layer, 1 << 20), dtype=torch.bfloat16, device="cuda")
        # owner segments of the rows, in row order: (owner, first position, length)
        segs = [(owner, lo, hi - lo) for r, q, L in zip(ids, q_lens, seq_lens)
                for owner, lo, hi in tr.owner_segments(int(r), int(L - q), int(L))]
        owners = np.array([o for o, _, _ in segs], np.int64)
        pos0 = np.array([p for _, p, _ in segs], np.int64)
        lens = np.array([n for _, _, n in segs], np.int64)
        keys, e0s, sizes = [], [], []
        # segment order: layer, kind, row segment -> each (layer, kind) region is [T][heads][d]
        for l in range(NL):
            for k, which in enumerate("qkv"):
                h = int(self.heads[k])
                keys.append(self._keys(l, which, owners))
                e0s.append(pos0 * h * d)
                sizes.append(lens * h * d)
        keys = np.concatenate(keys).view(np.int64)
        e0 = np.concatenate(e0s)
        off = np.zeros(len(e0) + 1, np.int64)
        np.cumsum(np.concatenate(sizes), out=off[1:])
        seg = torch.from_numpy(np.concatenate([keys, e0, off])).cuda()
        wgen.fill_segments(self.buf, seg, len(e0), int(off[-1]), tr.sigma)
        if self.layer_batched:                 # q, k, v as [NL][T][heads][d], per_layer apart
            views, o = [], 0
            for h in self.heads:
                views.append(self.buf.as_strided((NL, T, int(h), d), (per_layer, int(h) * d, d, 1), o))
                o += T * int(h) * d
            return views
        views = []
        o = 0
        for l in range(NL):
            parts = []
            for h in self.heads:
                m = T * int(h) * d
                parts.append(self.buf[o:o + m].view(T, int(h), d))
                o += m
            views.append(parts)
        return views

    def _keys(self, layer, which, owners):
        """Value-stream keys (uint64) of the owners (requests, then groups) for one layer/kind."""
        R = self.tr.num_requests
        idx = np.where(owners >= workloads.GROUP_OWNER, R + (owners - workloads.GROUP_OWNER), owners)
        return self.keys[layer, "qkv".index(which)][idx]

    def step(self, keep_layers: Sequence[int] = (), keep_plan: bool = False) -> Optional[StepRecord]:
        torch, tr = self.torch, self.tr
        n, T, _ = self.sched.schedule()
        if n == 0:
            self.sched.update()
            return None
        plan = self.sched.plan(n, T, self.width)
        step_no = plan.step
        q_lens, seq_lens = plan.q_lens, plan.seq_lens
        vals = self._values(plan.ids, q_lens, seq_lens)
        bt = torch.from_numpy(plan.block_tables).cuda()
        lens = torch.from_numpy(seq_lens).cuda()
        cu = torch.from_numpy(plan.cu_seqlens_q).cuda()
        slots = torch.from_numpy(plan.slot_mapping).cuda()
        # decode rows by the balanced-split decode, prefill rows by the chunk kernel; with
        # both kinds in the step, in one launch over fewer decode slots (never more than
        # self.slots, so the split workspace fits)
        NL = tr.num_layers
        mixed = self.one_launch and bool((q_lens == 1).any()) and bool((q_lens >= 2).any())
        dslots = self.slots
        if mixed:
            cdt = pkv.FP8 if tr.cache_dtype == "fp8" else pkv.BF16
            dslots = pkv.mixed_decode_slots(q_lens, seq_lens, cdt, tr.num_kv_heads, tr.group, tr.head_dim,
                                            tr.block_size, NL if self.layer_batched else 1)
        mp = pkv.build_mixed_step(q_lens, seq_lens, tr.num_kv_heads, tr.group, dslots, self.min_piece,
                                  self.chunk_slots, self.min_piece_tiles)
        chunk_dev = mp.chunks.to_device(tr.head_dim, num_layers=NL if self.layer_batched else 1)
        if len(mp.decode_rows):
            rows = torch.from_numpy(mp.decode_rows).cuda()
            plan_d = torch.from_numpy(mp.split.plan).cuda()
            ws = self.split_ws if mp.split.max_pieces > 1 else None
        msl = int(seq_lens.max())
        out = torch.empty(((NL,) if self.layer_batched else ()) + (T, tr.num_q_heads, tr.head_dim),
                          dtype=torch.bfloat16, device="cuda")
        kept = {}
        swap_in = self.sched.swap_pairs()[1] if self.host_space is not None else np.zeros((0, 2), np.int32)
        if len(swap_in):
            self._swap_workspace(len(swap_in))
        # the layers' launches, checked and marshalled ahead of the timed region: all
        # layers in each launch (the same calls on [NL][...] tensors), or the layers in turn
        launches = []
        for l in ([None] if self.layer_batched else range(NL)):
            q, k, v = vals if l is None else vals[l]
            kc, vc = (self.k_cache, self.v_cache) if l is None else (self.k_cache[l], self.v_cache[l])
            launches.append(pkv.kv_cache_write(k, v, kc, vc, slots, tr.block_size, tr.k_scale, tr.v_scale,
                                               defer=True))
            if mixed:
                launches.append(pkv.paged_attention_mixed(
                    out, q, kc, vc, bt, lens, cu, mp, ((rows, plan_d, ws), chunk_dev), tr.num_kv_heads,
                    tr.block_size, msl, tr.softmax_scale, tr.k_scale, tr.v_scale, defer=True))
            elif len(mp.decode_rows):
                launches.append(pkv.paged_attention_decode_split(
                    out, q, kc, vc, bt, lens, plan_d, mp.split, tr.num_kv_heads, tr.block_size, msl,
                    tr.softmax_scale, tr.k_scale, tr.v_scale, ws, rows=rows, cu_seqlens_q=cu, defer=True))
            if chunk_dev is not None and not mixed:
                work, merges, cws = chunk_dev
                launches.append(pkv.paged_attention_prefill_chunks(
                    out, q, kc, vc, bt, lens, cu, work, merges, mp.chunks.num_partials, cws, tr.num_kv_heads,
                    tr.block_size, msl, tr.softmax_scale, tr.k_scale, tr.v_scale, defer=True))
            if l is not None and l in keep_layers:
                launches.append(lambda l=l: kept.__setitem__(l, out.clone()))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        if len(swap_in) and self.copy_stream is not None:
            torch.cuda.current_stream().wait_stream(self.copy_stream)
        h0 = time.perf_counter()
        ei = None
        if len(swap_in):                       # swapped requests' K/V back before the layers
            pkv.swap_in(self.k_cache, self.v_cache, swap_in, self.host_space, self.swap_ws)
            ei = torch.cuda.Event(enable_timing=True)
            ei.record()
        for launch in launches:
            launch()
        if self.layer_batched:
            for l in keep_layers:
                kept[l] = out[l].clone()
        e1.record()
        host_s = time.perf_counter() - h0
        self.sched.update()
        es0 = es1 = None
        swap_out = self.sched.swap_pairs()[0] if self.host_space is not None else np.zeros((0, 2), np.int32)
        if len(swap_out):                      # victims' K/V to the host before the next step
            self._swap_workspace(len(swap_out))
            es0 = torch.cuda.Event(enable_timing=True)
            es1 = torch.cuda.Event(enable_timing=True)
            es0.record()
            if self.copy_stream is not None:
                torch.cuda.current_stream().wait_stream(self.copy_stream)
            pkv.swap_out(self.k_cache, self.v_cache, swap_out, self.host_space, self.swap_ws,
                         copy_stream=self.copy_stream)
            if self.copy_stream is not None:   # the allocator must not hand it out before the DMA ends
                self.swap_ws.record_stream(self.copy_stream)
            es1.record()
        # a row makes an output token when it decodes or completes its context
        ids = plan.ids
        made = (plan.stages == 1) | (seq_lens == self.tr.prompt[ids] + self.n_out[ids])
        first = ids[made & (self.n_out[ids] == 0)]
        self.n_out[ids[made]] += 1
        ctx = int(seq_lens.sum())
        row_bytes = 2 * tr.num_kv_heads * tr.head_dim
        per_layer = (ctx * row_bytes * self.e_kv                              # K/V read by attention
                     + T * row_bytes * (2 + self.e_kv)                        # write: bf16 in, cache out
                     + T * tr.num_q_heads * tr.head_dim * 2 * 2)              # queries in, outputs out
        return StepRecord(step_no, n, T, ctx, int((plan.stages == 0).sum()), per_layer * tr.num_layers,
                          (e0, e1), kept, plan if keep_plan else None, first.tolist(), host_s, (ei, es0, es1),
                          (len(swap_in), len(swap_out)), self._decode_by_class(plan))

    def _decode_by_class(self, plan):
        if self.classes is None:
            return ()
        cls = self.classes[plan.ids[plan.stages == 1]]
        return tuple(np.bincount(cls, minlength=int(self.classes.max()) + 1).tolist())

    def _swap_workspace(self, n):
        nb = pkv.swap_workspace_bytes(n, self.tr.num_layers, self.pair_bytes // (2 * self.tr.num_layers))
        if self.swap_ws is None or self.swap_ws.numel() < nb:
            self.swap_ws = self.torch.empty(max(nb, 64 << 20), dtype=self.torch.uint8, device="cuda")


def run(tr: workloads.Trace, max_steps: Optional[int] = None, keep=None, progress=None, **replay_args):
    """Replay the trace (or its first max_steps steps). keep: {step: layers} whose outputs
    (and plans) are kept; replay_args go to Replay. Returns (records, summary)."""
    import gc
    import torch
    rp = Replay(tr, **replay_args)
    recs: List[StepRecord] = []
    keep = keep or {}
    # no cyclic garbage collection inside the loop: a full collection over the records
    # kept so far can stall the host for tens of ms while a step's layers are enqueued
    gc_on = gc.isenabled()
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    steps = 0
    try:
        while True:
            c = rp.sched.counters()
            if c["finished"] == tr.num_requests or (max_steps is not None and steps >= max_steps):
                break
            s = c["step"]
            r = rp.step(keep_layers=keep.get(s, ()), keep_plan=s in keep)
            steps += 1
            if r is not None:
                recs.append(r)
            if progress and steps % 1000 == 0:
                progress(steps)
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    wall = time.perf_counter() - t0
    c = rp.sched.counters()
    t_layers = np.array([r.ev[0].elapsed_time(r.ev[1]) * 1e-3 for r in recs])
    t_in = np.array([r.ev[0].elapsed_time(r.swap_ev[0]) * 1e-3 if r.swap_ev and r.swap_ev[0] else 0.0 for r in recs])
    t_out = np.array([r.swap_ev[1].elapsed_time(r.swap_ev[2]) * 1e-3 if r.swap_ev and r.swap_ev[1] else 0.0
                      for r in recs])
    t = t_layers + t_out                   # a step: swap-ins, the layers, then its swap-outs
    qtok = np.array([r.q_tokens for r in recs], np.float64)
    byts = np.array([r.attention_bytes for r in recs], np.float64)
    rows = np.array([r.rows for r in recs], np.float64)
    tps = qtok / t
    # latencies in attention time (the GPU time of the steps' layers; host time excluded):
    # time to first token from the start of the arrival step to the end of the step that
    # made the first output; time between tokens = the time of each decode row's step
    nsteps = int(c["step"])
    t_step = np.zeros(nsteps + 1)
    first_step = np.full(tr.num_requests, -1, np.int64)
    for r, ti in zip(recs, t):
        t_step[r.step] = ti
        first_step[list(r.first_outputs)] = r.step
    t_end = np.cumsum(t_step)
    got = first_step >= 0
    ttft = t_end[first_step[got]] - (t_end[tr.arrival[got]] - t_step[tr.arrival[got]])
    dec = np.array([r.rows - r.prefill_rows for r in recs], np.int64)
    tbt = np.repeat(t, dec)

    def pct(x, qs=(50, 95, 99)):
        return {f"p{q}": round(float(np.percentile(x, q)) * 1e3, 3) for q in qs} if len(x) else {}

    summary = {
        "trace": tr.name, "cache_dtype": tr.cache_dtype, "steps": int(c["step"]), "requests": tr.num_requests,
        "finished": int(c["finished"]), "preemptions": int(c["preempted"]),
        "preemption_rate_per_step": round(c["preempted"] / max(c["step"], 1), 4),
        "cached_prompt_tokens": int(c["cached_tokens"]),
        "avg_running_batch": round(float(rows.mean()), 2), "query_tokens": int(qtok.sum()),
        "context_tokens_per_layer": int(sum(r.context_tokens for r in recs)),
        "attention_s_total": round(float(t.sum()), 4),
        "tokens_per_s_per_step": {"mean": round(float(tps.mean()), 1), "p50": round(float(np.percentile(tps, 50)), 1),
                                  "p99": round(float(np.percentile(tps, 99)), 1)},
        "tokens_per_s_overall": round(float(qtok.sum() / t.sum()), 1),
        "requests_per_s": round(float(c["finished"] / t.sum()), 2),      # per second of attention
        "hbm_GBps_per_step": {"mean": round(float((byts / t).mean() / 1e9), 1),
                              "p50": round(float(np.percentile(byts / t, 50) / 1e9), 1)},
        "hbm_GBps_overall": round(float(byts.sum() / t.sum() / 1e9), 1),
        "step_ms": {**pct(t, (50, 90, 99, 99.9)), "max": round(float(t.max()) * 1e3, 3) if len(t) else 0.0},
        "host_enqueue_ms": pct(np.array([r.host_s for r in recs]), (50, 99)),
        "ttft_ms": pct(ttft), "tbt_ms": pct(tbt),
        "wall_s": round(wall, 2),
    }
    if rp.classes is not None:                 # latencies per priority class
        by = {}
        for c in range(int(rp.classes.max()) + 1):
            sel = rp.classes[got] == c
            tb = np.repeat(t, [r.decode_by_class[c] for r in recs])
            by[str(c)] = {"requests": int((rp.classes == c).sum()), "ttft_ms": pct(ttft[sel]), "tbt_ms": pct(tb)}
        summary["by_priority_class"] = by
    if rp.host_space is not None:
        sc = rp.sched.swap_counters()
        b_in = sum(r.swap_blocks[0] for r in recs) * rp.pair_bytes
        b_out = sum(r.swap_blocks[1] for r in recs) * rp.pair_bytes
        summary["swap"] = {**sc, "swap_in_s": round(float(t_in.sum()), 4), "swap_out_s": round(float(t_out.sum()), 4),
                           "GB_in": round(b_in / 1e9, 3), "GB_out": round(b_out / 1e9, 3),
                           "GBps_in": round(b_in / max(float(t_in.sum()), 1e-12) / 1e9, 1),
                           "GBps_out": round(b_out / max(float(t_out.sum()), 1e-12) / 1e9, 1)}
    return recs, summary
