"""Config 5 trace replay on the GPU: libpkv's scheduler step drives the cache write and
the mixed attention launch of 16 layers; sampled rows (prefill, recompute after a
preemption, decode) are compared with the oracle's attention over the dense K/V of the
request, element by element. The scheduler itself is bit-exact vs its oracle on the CPU
(test_sched_host.py); here the device path is checked end to end."""
import numpy as np
import pytest

import workloads
from oracle import attention as oatt
from oracle import fp8 as ofp8
from workloads import replay

from gpu_setup import TOL, out_f64

pytestmark = pytest.mark.gpu


def _dense(tr, which, layer, req, L):
    x = tr.rows_f32(which, layer, req, 0, L).astype(np.float64)
    if tr.cache_dtype == "fp8":
        scale = tr.k_scale if which == "k" else tr.v_scale
        x = ofp8.decode(ofp8.encode(x.astype(np.float32), scale), scale)
    return x


def _check_step(tr, rec, rng, max_rows=8, tokens_per_row=3, prefer=()):
    plan = rec.plan
    cu = plan.cu_seqlens_q
    rows = list(range(len(plan.ids)))
    first = [r for r in rows if int(plan.ids[r]) in set(prefer)][:max_rows // 2]   # rows that must be checked
    # prefill rows, later chunks of a cut prefill (or rows after a cached prefix) first
    pre = sorted((r for r in rows if plan.stages[r] == 0), key=lambda r: plan.q_lens[r] == plan.seq_lens[r])
    dec = [r for r in rows if plan.stages[r] == 1]
    pick = pre[:max_rows // 2] + list(rng.choice(dec, size=min(len(dec), max_rows - min(len(pre), max_rows // 2)),
                                                 replace=False))
    pick = first + [r for r in pick if r not in first][:max_rows - len(first)]
    checked = 0
    for layer, out in rec.kept.items():
        o = out_f64(out)
        assert np.isfinite(o).all()
        for r in pick:
            req, q, L = int(plan.ids[r]), int(plan.q_lens[r]), int(plan.seq_lens[r])
            K = _dense(tr, "k", layer, req, L)
            V = _dense(tr, "v", layer, req, L)
            toks = sorted(set([0, q - 1] + rng.integers(0, q, size=tokens_per_row).tolist()))
            qs = tr.rows_f32("q", layer, req, L - q, L)[toks].astype(np.float64)
            ref, _ = oatt.attend(qs, K, V, [L - q + t for t in toks], tr.softmax_scale, tr.group)
            got = o[cu[r] + np.array(toks)]
            tol = TOL["fp8" if tr.cache_dtype == "fp8" else "bf16"]
            err = np.abs(got - ref).max()
            assert err <= tol, f"step {rec.step} layer {layer} request {req} (q {q}, L {L}): err {err:.3e}"
            checked += 1
    return checked


@pytest.mark.parametrize("cache_dtype,steps,keep_steps", [
    ("bf16", 160, (0, 1, 112, 115, 145, 159)),
    ("fp8", 120, (0, 112, 115, 119)),
])
def test_config5_replay_sampled_parity(cache_dtype, steps, keep_steps):
    tr = workloads.config5(cache_dtype)
    keep = {s: (0, tr.num_layers - 1) for s in keep_steps}
    recs, summary = replay.run(tr, max_steps=steps, keep=keep)
    assert summary["steps"] == steps
    by_step = {r.step: r for r in recs}
    rng = np.random.default_rng(5)
    checked = 0
    for s in keep_steps:
        checked += _check_step(tr, by_step[s], rng)
    assert checked >= 20
    if steps > 112:
        assert summary["preemptions"] > 0
        # the step after the first preemption re-prefills a request with its outputs
        p = by_step[112].plan
        assert any(st_ == 0 and q > tr.prompt[i] for i, st_, q in zip(p.ids, p.stages, p.q_lens))


def test_prefix_trace_replay_sampled_parity():
    # shared system prompts: prefill rows start after a cached prefix whose K/V another
    # request wrote; the oracle attends over the request's own dense K/V
    from oracle import scheduler as osch
    tr = workloads.config5_prefix("bf16")
    toks = [tr.prompt_tokens(r) for r in range(tr.num_requests)]
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, prompt_tokens=toks)
    hit_steps = []
    for plan, _ in osch.run(ref, 512, 140):
        if ((plan.stages == 0) & (plan.q_lens < plan.seq_lens)).any():
            hit_steps.append(plan.step)
    assert len(hit_steps) >= 3
    keep_steps = hit_steps[:2] + hit_steps[-2:]
    keep = {s: (0, tr.num_layers - 1) for s in keep_steps}
    recs, summary = replay.run(tr, max_steps=140, keep=keep)
    assert summary["cached_prompt_tokens"] > 0
    by_step = {r.step: r for r in recs}
    rng = np.random.default_rng(7)
    checked = 0
    for s in keep_steps:
        checked += _check_step(tr, by_step[s], rng)
    assert checked >= 12


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_chunked_prefill_replay_sampled_parity(cache_dtype):
    # token budget 2048, chunks of 512: long prompts are computed over several steps; a
    # later chunk attends over the K/V its request's earlier chunks wrote in earlier steps
    from oracle import scheduler as osch
    tr = workloads.config5(cache_dtype)
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, max_batched_tokens=2048, chunk_tokens=512)
    chunk_steps = []
    for plan, _ in osch.run(ref, 512, 140):
        later = (plan.stages == 0) & (plan.q_lens < plan.seq_lens)
        if later.any() and (plan.q_lens[later] > 1).any():
            chunk_steps.append(plan.step)
    assert len(chunk_steps) >= 4
    keep_steps = chunk_steps[:2] + chunk_steps[-2:]
    keep = {s: (0, tr.num_layers - 1) for s in keep_steps}
    recs, summary = replay.run(tr, max_steps=140, keep=keep, token_budget=2048, chunk_tokens=512)
    assert summary["steps"] == 140
    by_step = {r.step: r for r in recs}
    for s in keep_steps:                       # the device replay took the oracle's schedule
        assert int(by_step[s].q_tokens) <= 2048 + int((by_step[s].plan.stages == 1).sum())
    rng = np.random.default_rng(11)
    checked = 0
    for s in keep_steps:
        checked += _check_step(tr, by_step[s], rng)
    assert checked >= 12


def test_policy_variants_replay_sampled_parity():
    # LIFO victims among the bulk class, priority admission, a short host space (swap and
    # recompute both happen): rows of re-admitted victims attend to the right K/V
    from oracle import scheduler as osch
    tr = workloads.config5("bf16")
    prio = workloads.priority_classes(tr)
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, swap_blocks=64, victim="lifo", priority=prio)
    plans, back, again = {}, [], []
    for plan, _ in osch.run(ref, 512, 300):
        plans[plan.step] = plan
        if plan.swap_in:
            back.append(plan.step)
        if any(st_ == 0 and q > tr.prompt[i] for i, st_, q in zip(plan.ids, plan.stages, plan.q_lens)):
            again.append(plan.step)
    assert back and again
    keep_steps = sorted(set(back[:2] + again[:2]))
    keep = {s: (0, tr.num_layers - 1) for s in keep_steps}
    recs, summary = replay.run(tr, max_steps=max(keep_steps) + 1, keep=keep, swap_blocks=64, victim="lifo",
                               priority=prio)
    assert summary["preemptions"] > 0 and summary["swap"]["swapped_out"] > 0
    by_step = {r.step: r for r in recs}
    rng = np.random.default_rng(19)
    checked = 0
    for s in keep_steps:
        p = by_step[s].plan
        assert (p.ids == plans[s].ids).all() and (p.seq_lens == plans[s].seq_lens).all()
        swapped_blocks = {int(b) for _, b in plans[s].swap_in}
        prefer = [int(i) for k, (i, st_, q) in enumerate(zip(p.ids, p.stages, p.q_lens))
                  if (st_ == 0 and q > tr.prompt[i]) or swapped_blocks & set(p.block_tables[k].tolist())]
        assert prefer
        checked += _check_step(tr, by_step[s], rng, prefer=prefer)
    assert checked >= 8
