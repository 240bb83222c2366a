"""Config 5 trace replay on the GPU: libpkv's scheduler step drives the cache write and
the mixed attention launches of 16 layers. For the kept steps, every query row (prefill,
recompute after a preemption, later chunks, rows after a cached prefix, swapped-in
requests, decode) of every kept layer is compared with the oracle's attention over the
request's dense K/V, element by element; the oracle's side (its own scheduler plan and
attention) runs in a child program (gpu_setup.oracle_job). The scheduler itself is
bit-exact vs its oracle on the CPU (test_sched_host.py); here the device path is
checked end to end, and each kept step's plan must equal the oracle's."""
import numpy as np
import pytest

import workloads
from workloads import replay

from gpu_setup import TOL, oracle_job, out_f64, report_error

pytestmark = pytest.mark.gpu

ALL_LAYERS = tuple(range(16))


def _check_full(tr, recs, job, what):
    """Every row of every kept (step, layer) of a replay against the oracle job's results."""
    ref = oracle_job(job)
    by_step = {r.step: r for r in recs}
    tol = TOL["fp8" if tr.cache_dtype == "fp8" else "bf16"]
    worst, rows = 0.0, 0
    for s in job["steps"]:
        rec, k = by_step[s], f"s{s}"
        p = rec.plan
        for name, a in (("ids", p.ids), ("stages", p.stages), ("q_lens", p.q_lens), ("seq_lens", p.seq_lens),
                        ("cu", p.cu_seqlens_q)):
            assert np.array_equal(np.asarray(a), ref[f"{k}_{name}"]), f"step {s}: {name} differs from the oracle's plan"
        for layer in job["layers"]:
            got = out_f64(rec.kept[layer])
            want = ref[f"{k}_l{layer}_out"].astype(np.float64)
            err = np.abs(got - want)
            bad = np.argwhere(~(err <= tol))
            if len(bad):
                t = int(bad[0][0])
                r = int(np.searchsorted(p.cu_seqlens_q, t, side="right") - 1)
                raise AssertionError(f"{what} step {s} layer {layer}: {len(bad)} elements beyond {tol}; first at "
                                     f"token {t} (request {int(p.ids[r])}, q {int(p.q_lens[r])}, "
                                     f"L {int(p.seq_lens[r])}), err {err.max():.3e}")
            worst = max(worst, float(err.max()))
        rows += len(p.ids)
    print(f"[parity] {what}: {len(job['steps'])} steps x {len(job['layers'])} layers, {rows} rows, "
          f"max |out err| {worst:.3e} (tol {tol})", flush=True)
    return by_step


@pytest.mark.parametrize("cache_dtype,steps,keep_steps,layer_batched", [
    ("bf16", 160, (1, 3, 112, 115, 159), True),
    ("fp8", 120, (0, 2, 112, 119), True),
    ("bf16", 160, (1, 3, 112, 115, 159), False),      # one launch per kernel and layer
])
def test_config5_replay_full_rows(cache_dtype, steps, keep_steps, layer_batched):
    tr = workloads.config5(cache_dtype)
    job = {"kind": "replay", "trace": "config5", "cache_dtype": cache_dtype, "steps": list(keep_steps),
           "layers": list(ALL_LAYERS)}
    recs, summary = replay.run(tr, max_steps=steps, keep={s: ALL_LAYERS for s in keep_steps},
                               layer_batched=layer_batched)
    assert summary["steps"] == steps
    by_step = _check_full(tr, recs, job, f"config 5 replay ({cache_dtype} cache, "
                                         f"{'layer-batched' if layer_batched else 'per-layer'} launches)")
    if steps > 112:
        assert summary["preemptions"] > 0
        # the step after the first preemption re-prefills a request with its outputs
        p = by_step[112].plan
        assert any(st_ == 0 and q > tr.prompt[i] for i, st_, q in zip(p.ids, p.stages, p.q_lens))


EDGE_LAYERS = (0, 15)


def test_prefix_trace_replay_full_rows():
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
    job = {"kind": "replay", "trace": "config5_prefix", "cache_dtype": "bf16", "steps": keep_steps,
           "layers": list(EDGE_LAYERS)}
    recs, summary = replay.run(tr, max_steps=140, keep={s: EDGE_LAYERS for s in keep_steps})
    assert summary["cached_prompt_tokens"] > 0
    _check_full(tr, recs, job, "prefix-cache replay")


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_chunked_prefill_replay_full_rows(cache_dtype):
    # token budget 2048, chunks of 512: long prompts are computed over several steps; a
    # later chunk attends over the K/V its request's earlier chunks wrote in earlier steps
    from oracle import scheduler as osch
    tr = workloads.config5(cache_dtype)
    sched = {"max_batched_tokens": 2048, "chunk_tokens": 512}
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, **sched)
    chunk_steps = []
    for plan, _ in osch.run(ref, 512, 140):
        later = (plan.stages == 0) & (plan.q_lens < plan.seq_lens)
        if later.any() and (plan.q_lens[later] > 1).any():
            chunk_steps.append(plan.step)
    assert len(chunk_steps) >= 4
    keep_steps = chunk_steps[:2] + chunk_steps[-2:]
    job = {"kind": "replay", "trace": "config5", "cache_dtype": cache_dtype, "sched": sched, "steps": keep_steps,
           "layers": list(EDGE_LAYERS)}
    recs, summary = replay.run(tr, max_steps=140, keep={s: EDGE_LAYERS for s in keep_steps}, token_budget=2048,
                               chunk_tokens=512)
    assert summary["steps"] == 140
    by_step = _check_full(tr, recs, job, f"chunked-prefill replay ({cache_dtype} cache)")
    for s in keep_steps:                       # the device replay took the oracle's schedule
        assert int(by_step[s].q_tokens) <= 2048 + int((by_step[s].plan.stages == 1).sum())


def test_policy_variants_replay_full_rows():
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
    job = {"kind": "replay", "trace": "config5", "cache_dtype": "bf16",
           "sched": {"swap_blocks": 64, "victim": "lifo", "priority": True}, "steps": keep_steps,
           "layers": list(EDGE_LAYERS)}
    recs, summary = replay.run(tr, max_steps=max(keep_steps) + 1, keep={s: EDGE_LAYERS for s in keep_steps},
                               swap_blocks=64, victim="lifo", priority=prio)
    assert summary["preemptions"] > 0 and summary["swap"]["swapped_out"] > 0
    by_step = _check_full(tr, recs, job, "policy-variant replay (LIFO, priorities, swap)")
    for s in keep_steps:                       # the kept steps hold re-admitted victims
        p = by_step[s].plan
        swapped_blocks = {int(b) for _, b in plans[s].swap_in}
        assert any((st_ == 0 and q > tr.prompt[i]) or swapped_blocks & set(p.block_tables[k].tolist())
                   for k, (i, st_, q) in enumerate(zip(p.ids, p.stages, p.q_lens)))
