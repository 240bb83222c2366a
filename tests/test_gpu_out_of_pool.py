"""Block-table entries outside the pool (a corrupt table) on the mixed-step launches.

Such an entry is never dereferenced. The decode paths skip its keys; the prefill paths
(the one-launch varlen kernel and the chunk kernels) read its rows as zero keys and
values. Both are checked against the oracle on the same step: prefill rows with the bad
entries pointed at an all-zero block of the pool, decode rows with the keys of the bad
blocks removed. What a row computes is the page-walk attention of "Project 17:
Production Serving: Continuous Batching and PagedAttention", "Step 6"."""
import zlib

import numpy as np
import pytest
import torch

import workloads
from gpu_setup import (assert_close, build_step, oracle_attention_full, oracle_planes, oracle_scales, out_f64,
                       run_mixed_two_launch, run_varlen)
from oracle import attention as oatt
from oracle import cache as ocache

pytestmark = pytest.mark.gpu

LSE_ATOL = 2.0 ** -8   # weights enter P.V rounded to bf16 (as in the other mixed-step tests)

CASES = [("bf16", 128, 4, 16), ("bf16", 128, 4, 32), ("bf16", 64, 4, 16), ("fp8", 128, 4, 16)]


@pytest.mark.parametrize("cdt,d,G,bs", CASES, ids=[f"{a}-d{b}-g{c}-bs{e}" for a, b, c, e in CASES])
def test_out_of_pool_entries(cdt, d, G, bs):
    seed = zlib.crc32(f"oop{cdt}{d}{G}{bs}".encode()) % 10_000
    # seq 0: a chunk of 200 rows after 400 cached; seq 1, 3: decode rows; seq 2: a full
    # prefill with no bad entry
    L = [600, 40, 300, 257]
    q = [200, 1, 300, 1]
    Hkv = 2
    w = workloads.small_varlen(seed, L, q, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, block_size=bs,
                               dtype="bf16", cache_dtype=cdt, pool_extra=3)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    tabs, bt, cu, slots, kp, vp = oracle_planes(st)
    assert (st.bt == bt).all()
    used = {int(x) for s in range(w.num_seqs) for x in bt[s, : (int(L[s]) + bs - 1) // bs]}
    spare = min(set(range(w.num_blocks)) - used)
    # the spare block holds zeros on both sides (code 0 is +0 in E4M3 too)
    st.k_cache.view(torch.uint8)[spare].zero_()
    st.v_cache.view(torch.uint8)[spare].zero_()
    kp[spare] = 0
    vp[spare] = 0
    bad = {0: (5, w.num_blocks + 3), 3: (2, -1)}          # seq: (table index, bad id)
    bt_bad = bt.copy()
    bt_zero = bt.copy()
    for s, (j, v) in bad.items():
        bt_bad[s, j] = v
        bt_zero[s, j] = spare
    st.bt_d = torch.from_numpy(bt_bad).cuda()

    # expected: prefill rows over the zero block; decode rows without the bad block's keys
    ref, ref_lse = oracle_attention_full(st, kp, vp, bt_zero, cu)
    qf = workloads.storage_to_f64(w.q_all(), w.dtype)
    ks, vs = oracle_scales(w)
    for s in (1, 3):
        n = int(L[s])
        K = ocache.decode_rows(kp, bt_zero[s], n, w.cache_dtype, ks)
        V = ocache.decode_rows(vp, bt_zero[s], n, w.cache_dtype, vs)
        keep = np.ones(n, bool)
        if s in bad:
            j = bad[s][0]
            keep[j * bs: min((j + 1) * bs, n)] = False
        r = int(cu[s + 1]) - 1
        o, l = oatt.attend(qf[r:r + 1], K[keep], V[keep], [int(keep.sum()) - 1], w.softmax_scale, w.group)
        ref[r], ref_lse[r] = o[0], l[0]

    # the check tells the two readings apart: seq 0's rows with the bad block's keys
    # skipped (as decode does) would have log-sum-exps well away from the zero-row ones
    n0, r0, r1 = int(L[0]), int(cu[0]), int(cu[1])
    K = ocache.decode_rows(kp, bt_zero[0], n0, w.cache_dtype, ks)
    V = ocache.decode_rows(vp, bt_zero[0], n0, w.cache_dtype, vs)
    keep = np.ones(n0, bool)
    keep[bad[0][0] * bs: (bad[0][0] + 1) * bs] = False
    pos = n0 - (r1 - r0) + np.arange(r1 - r0)
    _, l_skip = oatt.attend(qf[r0:r1], K[keep], V[keep], np.cumsum(keep)[pos] - 1, w.softmax_scale, w.group)
    assert np.abs(l_skip - ref_lse[r0:r1]).max() > 4 * LSE_ATOL

    dt = "fp8" if cdt == "fp8" else "bf16"
    out, lse = run_varlen(st)
    assert_close(out_f64(out), ref, dt, f"{w.name} one launch")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
    for cs in (None, 5000):                                 # uncut blocks, and single-tile pieces
        o2, l2 = run_mixed_two_launch(st, chunk_slots=cs)
        got = out_f64(o2)
        assert not np.isnan(got).any(), f"{w.name} two launches ({cs}): unwritten rows"
        assert_close(got, ref, dt, f"{w.name} two launches ({cs})")
        np.testing.assert_allclose(l2.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
