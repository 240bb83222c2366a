"""Swap copies on the GPU (pkv_swap_out / pkv_swap_in through the C ABI) against the
oracle's block copies (oracle/swap.py), byte for byte: small caches of random bits with
two kernel launches' worth of pairs, host blocks in runs and scattered; the full trace
geometry (16 layers, 4,096 blocks, 1 GiB of K/V swapped each way), every byte; and the
trace replay with preemption by swap, where every row of the kept steps (those with
swapped-in requests) is compared with the oracle's attention over its dense K/V."""
import numpy as np
import pytest
import torch

import paged_kv_cache_42_amd as pkv
import workloads
from oracle import scheduler as osch
from oracle import swap as osw
from workloads import replay

pytestmark = pytest.mark.gpu


def _bytes(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _pinned(nbytes, fill):
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h.fill_(fill)
    return h


@pytest.mark.parametrize("cache_dtype,copy_stream", [("bf16", False), ("fp8", False), ("bf16", True)])
def test_swap_out_and_in_match_the_oracle_bytes(cache_dtype, copy_stream):
    L, nb, bs, hkv, d, H = 3, 600, 16, 2, 64, 512
    rng = np.random.default_rng(17)
    if cache_dtype == "bf16":
        k0 = rng.integers(0, 1 << 16, (L, nb, bs, hkv, d), dtype=np.uint16)
        v0 = rng.integers(0, 1 << 16, k0.shape, dtype=np.uint16)
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        k0 = rng.integers(0, 256, (L, nb, bs, hkv, d), dtype=np.uint8)
        v0 = rng.integers(0, 256, k0.shape, dtype=np.uint8)
        to_dev = lambda a: torch.from_numpy(a).cuda()
    k, v = to_dev(k0), to_dev(v0)
    kb, vb = k0.view(np.uint8).reshape(L, nb, -1), v0.view(np.uint8).reshape(L, nb, -1)
    block_bytes = kb.shape[2]
    # 300 pairs (two launches): a run of consecutive host blocks, a descending run, scattered ones
    dev = rng.choice(nb, 300, replace=False).astype(np.int32)
    rest = np.setdiff1d(np.arange(H), np.r_[100:180, 300:260:-1])
    host = np.r_[np.arange(100, 180), np.arange(300, 260, -1), rng.choice(rest, 180, replace=False)].astype(np.int32)
    out_pairs = np.stack([dev, host], 1)
    hs = _pinned(H * L * 2 * block_bytes, 0xA5)
    ws = torch.empty(pkv.swap_workspace_bytes(300, L, block_bytes), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream() if copy_stream else None
    pkv.swap_out(k, v, out_pairs, hs, ws, copy_stream=cs)
    if cs is not None:                         # the DMA leg runs on cs: the swap-in waits for it
        torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    want = np.full((H, L, 2, block_bytes), 0xA5, np.uint8)
    osw.swap_out(kb, vb, out_pairs.tolist(), want)
    assert (hs.numpy().reshape(want.shape) == want).all()
    assert (_bytes(k).reshape(kb.shape) == kb).all() and (_bytes(v).reshape(vb.shape) == vb).all()

    # back into other device blocks of caches refilled with another pattern
    k.view(torch.uint8).fill_(0x5A)
    v.view(torch.uint8).fill_(0x5A)
    new_dev = rng.choice(nb, 300, replace=False).astype(np.int32)
    in_pairs = np.stack([host, new_dev], 1)
    pkv.swap_in(k, v, in_pairs, hs, ws)
    torch.cuda.synchronize()
    wk = np.full(kb.shape, 0x5A, np.uint8)
    wv = np.full(vb.shape, 0x5A, np.uint8)
    osw.swap_in(want, in_pairs.tolist(), wk, wv)
    assert (_bytes(k).reshape(kb.shape) == wk).all() and (_bytes(v).reshape(vb.shape) == wv).all()


def test_no_pairs_is_a_no_op():
    k = torch.zeros((2, 8, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    hs = _pinned(4 * 2 * 2 * 4096, 7)
    pkv.swap_out(k, v, np.zeros((0, 2), np.int32), hs, None)
    pkv.swap_in(k, v, np.zeros((0, 2), np.int32), hs, None)
    torch.cuda.synchronize()
    assert (hs.numpy() == 7).all() and not k.view(torch.int16).any()


def test_full_trace_geometry_one_gib_each_way():
    # 16 layers x 4,096 blocks of random bits; 2048 pairs x 16 layers x (K, V) x 16 KiB =
    # 1 GiB each way, every byte of the host space and of both planes against the oracle
    tr = workloads.config5("bf16")
    L, nb, bs, hkv, d = tr.num_layers, tr.num_blocks, tr.block_size, tr.num_kv_heads, tr.head_dim
    rng = np.random.default_rng(23)
    k0 = rng.integers(0, 1 << 16, (L, nb, bs, hkv, d), dtype=np.uint16)
    v0 = rng.integers(0, 1 << 16, k0.shape, dtype=np.uint16)
    k = torch.from_numpy(k0.view(np.int16)).cuda().view(torch.bfloat16)
    v = torch.from_numpy(v0.view(np.int16)).cuda().view(torch.bfloat16)
    kb, vb = k0.view(np.uint8).reshape(L, nb, -1), v0.view(np.uint8).reshape(L, nb, -1)
    block_bytes = kb.shape[2]
    n = 2048
    dev = rng.permutation(nb)[:n].astype(np.int32)
    host = rng.permutation(n).astype(np.int32)
    hs = _pinned(n * L * 2 * block_bytes, 0xA5)
    ws = torch.empty(pkv.swap_workspace_bytes(n, L, block_bytes), dtype=torch.uint8, device="cuda")
    print(f"[swap] full geometry: {n} pairs, {n * L * 2 * block_bytes / 2 ** 30:.2f} GiB", flush=True)
    pkv.swap_out(k, v, np.stack([dev, host], 1), hs, ws)
    torch.cuda.synchronize()
    want = np.full((n, L, 2, block_bytes), 0xA5, np.uint8)
    osw.swap_out(kb, vb, np.stack([dev, host], 1).tolist(), want)
    assert np.array_equal(hs.numpy().reshape(want.shape), want), "host space differs from the oracle"
    k.view(torch.uint8).fill_(0)
    v.view(torch.uint8).fill_(0)
    new_dev = rng.permutation(nb)[:n].astype(np.int32)
    pkv.swap_in(k, v, np.stack([host, new_dev], 1), hs, ws)
    torch.cuda.synchronize()
    wk, wv = np.zeros_like(kb), np.zeros_like(vb)
    osw.swap_in(want, np.stack([host, new_dev], 1).tolist(), wk, wv)
    assert np.array_equal(_bytes(k).reshape(kb.shape), wk) and np.array_equal(_bytes(v).reshape(vb.shape), wv)


@pytest.mark.parametrize("overlap,cache_dtype", [(False, "bf16"), (True, "bf16"), (True, "fp8")])
def test_replay_with_swap_full_rows(overlap, cache_dtype):
    # the trace replay with a host space of 4096 blocks: preempted requests are swapped out
    # and come back without a prefill; their decode rows after the swap-in must attend to
    # the K/V they had
    from test_gpu_sched_replay import EDGE_LAYERS, _check_full
    tr = workloads.config5(cache_dtype)
    ref = osch.Scheduler(tr.arrival, tr.prompt, tr.max_tokens, tr.num_blocks, tr.free_order, tr.block_size,
                         tr.max_running, swap_blocks=4096)
    back = {}
    for plan, _ in osch.run(ref, 512, 400):
        if plan.swap_in:
            back[plan.step] = plan
    assert len(back) >= 2
    keep_steps = sorted(back)[:3]
    job = {"kind": "replay", "trace": "config5", "cache_dtype": cache_dtype, "sched": {"swap_blocks": 4096},
           "steps": keep_steps, "layers": list(EDGE_LAYERS)}
    recs, summary = replay.run(tr, max_steps=max(keep_steps) + 1, keep={s: EDGE_LAYERS for s in keep_steps},
                               swap_blocks=4096, swap_overlap=overlap)
    assert summary["swap"]["swapped_out"] > 0 and summary["swap"]["blocks_in"] > 0
    by_step = _check_full(tr, recs, job, f"swap replay ({cache_dtype} cache, overlap {overlap})")
    for s in keep_steps:
        rec = by_step[s]
        assert rec.swap_blocks[0] == len(back[s].swap_in)
        swapped = set(int(b) for _, b in back[s].swap_in)
        assert any(swapped & set(rec.plan.block_tables[k].tolist()) for k in range(len(rec.plan.ids)))
