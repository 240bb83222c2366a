"""Pins for the oracle's paged attention: closed forms, invariants, brute force and
an independent library routine (torch scaled_dot_product_attention, float64)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, cache
from oracle.allocator import BlockPool, SeqTables
from oracle.metadata import build_block_table
import workloads


def _setup(w: workloads.Workload, fill_rows=None):
    """Allocate tables, write every context token, return planes and metadata."""
    t = SeqTables(BlockPool(w.num_blocks, w.free_order), w.block_size)
    for s, L in enumerate(w.seq_lens):
        t.reserve(s, int(L))
    tabs = [t.tables[s] for s in range(w.num_seqs)]
    W = max(1, w.max_blocks_per_seq())
    all_lens = w.seq_lens
    bt_all, _, slots_all = build_block_table(tabs, all_lens, all_lens, w.block_size, W)
    kp = cache.empty_plane(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype)
    vp = cache.empty_plane(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.cache_dtype)
    ks, vs = zip(*[w.kv(s) for s in range(w.num_seqs)]) if w.num_seqs else ((), ())
    if w.num_seqs:
        cache.write(kp, np.concatenate(ks), w.dtype, w.cache_dtype, slots_all, w.k_scale)
        cache.write(vp, np.concatenate(vs), w.dtype, w.cache_dtype, slots_all, w.v_scale)
    bt, cu, _ = build_block_table(tabs, w.q_lens, w.seq_lens, w.block_size, W)
    q = workloads.storage_to_f64(w.q_all(), w.dtype)
    return tabs, kp, vp, bt, cu, q


def _dense_kv(w, s):
    k, v = w.kv(s)
    return workloads.storage_to_f64(k, w.dtype), workloads.storage_to_f64(v, w.dtype)


def _sdpa(q, K, V, positions, scale, group):
    """torch SDPA in float64 with an explicit mask (keys <= position) and KV heads
    repeated per group; q [n][Hq][d], K/V [L][Hkv][d]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)                         # [Hq][n][d]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(group, 0)
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(group, 0)
    mask = torch.arange(K.shape[0])[None, :] <= torch.as_tensor(positions)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 4, 16))
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    out, lse = attention.attend(q, K, V, [0], 0.25, 2)
    for h in range(4):
        assert (out[0, h] == V[0, h // 2]).all()
        assert lse[0, h] == pytest.approx(0.25 * q[0, h] @ K[0, h // 2], abs=1e-14)


def test_zero_query_and_equal_keys_average_values():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((37, 2, 8))
    V = rng.standard_normal((37, 2, 8))
    out, lse = attention.attend(np.zeros((1, 2, 8)), K, V, [36], 1.0, 1)
    np.testing.assert_allclose(out[0], V.mean(0), rtol=0, atol=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(37), abs=1e-14)
    Keq = np.repeat(K[:1], 37, axis=0)
    out2, _ = attention.attend(rng.standard_normal((1, 2, 8)), Keq, V, [36], 1.0, 1)
    np.testing.assert_allclose(out2[0], V.mean(0), rtol=0, atol=1e-13)


def test_constant_values_and_weights_sum_to_one():
    rng = np.random.default_rng(2)
    L, d = 24, 32
    q = rng.standard_normal((1, 2, d))
    K = rng.standard_normal((L, 1, d))
    V = np.full((L, 1, d), 0.375)
    out, _ = attention.attend(q, K, V, [L - 1], 1 / math.sqrt(d), 2)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-15)
    # one-hot values: the output row is the weight vector itself
    Voh = np.zeros((L, 1, d))
    Voh[np.arange(L), 0, np.arange(L)] = 1.0
    out, _ = attention.attend(q, K, Voh, [L - 1], 1 / math.sqrt(d), 2)
    for h in range(2):
        w = out[0, h, :L]
        assert (w > 0).all() and w.sum() == pytest.approx(1.0, abs=1e-14)
        z = K[:, 0, :] @ q[0, h]
        assert np.argmax(w) == np.argmax(z) and np.argmin(w) == np.argmin(z)


@pytest.mark.parametrize("group", [1, 2, 4])
def test_dense_matches_sdpa_decode_and_causal_chunks(group):
    rng = np.random.default_rng(10 + group)
    Hkv, d, L = 2, 24, 41
    Hq = Hkv * group
    K = rng.standard_normal((L, Hkv, d))
    V = rng.standard_normal((L, Hkv, d))
    for nq in (1, 5, L):
        q = rng.standard_normal((nq, Hq, d))
        pos = L - nq + np.arange(nq)
        ours, lse = attention.attend(q, K, V, pos, 0.3, group)
        ref = _sdpa(q, K, V, pos, 0.3, group)
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)
        # log-sum-exp against torch.logsumexp of the masked scores
        for i in range(nq):
            for h in range(Hq):
                z = torch.from_numpy(0.3 * K[: pos[i] + 1, h // group] @ q[i, h])
                assert lse[i, h] == pytest.approx(torch.logsumexp(z, 0).item(), abs=1e-12)


def test_full_prefill_is_standard_causal():
    rng = np.random.default_rng(3)
    L, H, d = 19, 3, 8
    q = rng.standard_normal((L, H, d))
    K = rng.standard_normal((L, H, d))
    V = rng.standard_normal((L, H, d))
    ours, _ = attention.attend(q, K, V, np.arange(L), 1 / math.sqrt(d), 1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(1, 0, 2) for a in (q, K, V)), is_causal=True)
    np.testing.assert_allclose(ours, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_config1_paged_equals_dense_and_literal_loop():
    w = workloads.config1()
    tabs, kp, vp, bt, cu, q = _setup(w)
    out, lse = attention.paged_attention(q, kp, vp, "f32", bt, w.seq_lens, cu,
                                         w.softmax_scale, w.group)
    for s in range(4):
        K, V = _dense_kv(w, s)
        ref = _sdpa(q[s:s + 1], K, V, [int(w.seq_lens[s]) - 1], w.softmax_scale, w.group)
        np.testing.assert_allclose(out[s:s + 1], ref, rtol=1e-12, atol=1e-13)
        lit = attention.paged_attention_literal(q[s], tabs[s], kp, vp, "f32",
                                                int(w.seq_lens[s]), w.group)
        np.testing.assert_allclose(out[s], lit, rtol=1e-11, atol=1e-12)
    assert w.softmax_scale == 1 / 8


@pytest.mark.parametrize("seed", range(4))
def test_random_small_literal_loop_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([1, 2, 4, 8]))
    lens = rng.integers(1, 40, size=3)
    w = workloads.small_decode(seed, lens, num_q_heads=4, num_kv_heads=2, head_dim=8,
                               block_size=bs, dtype="bf16")
    tabs, kp, vp, bt, cu, q = _setup(w)
    out, _ = attention.paged_attention(q, kp, vp, "bf16", bt, w.seq_lens, cu, w.softmax_scale, 2)
    for s in range(3):
        lit = attention.paged_attention_literal(q[s], tabs[s], kp, vp, "bf16", int(lens[s]), 2)
        np.testing.assert_allclose(out[s], lit, rtol=1e-11, atol=1e-12)


def test_physical_permutation_invariance_is_exact():
    w = workloads.small_decode(7, [33, 1, 16, 17, 64], num_q_heads=6, num_kv_heads=3,
                               head_dim=16, block_size=8)
    tabs, kp, vp, bt, cu, q = _setup(w)
    out, lse = attention.paged_attention(q, kp, vp, "f32", bt, w.seq_lens, cu, 0.2, 2)
    perm = np.random.default_rng(9).permutation(w.num_blocks)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    out2, lse2 = attention.paged_attention(q, kp2, vp2, "f32", bt2, w.seq_lens, cu, 0.2, 2)
    assert (out == out2).all() and (lse == lse2).all()


def test_mha_special_case():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((9, 3, 8))
    V = rng.standard_normal((9, 3, 8))
    q = rng.standard_normal((1, 3, 8))
    out, _ = attention.attend(q, K, V, [8], 0.5, 1)
    for h in range(3):
        o1, _ = attention.attend(q[:, h:h + 1], K[:, h:h + 1], V[:, h:h + 1], [8], 0.5, 1)
        assert (o1[0, 0] == out[0, h]).all()


@pytest.mark.parametrize("P", [1, 3, 16, 40, 41, 1000])
def test_split_merge_equals_unsplit(P):
    rng = np.random.default_rng(P)
    L = 41
    K = rng.standard_normal((L, 2, 16)) * 2
    V = rng.standard_normal((L, 2, 16))
    q = rng.standard_normal((4, 16)) * 2
    ref, lse_ref = attention.attend(q[None], K, V, [L - 1], 0.7, 2)
    out, lse = attention.split_merge(q, K, V, 0.7, 2, P)
    np.testing.assert_allclose(out, ref[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref[0], rtol=0, atol=1e-13)


def test_empty_context_row():
    out, lse = attention.attend(np.ones((1, 2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)),
                                [-1], 1.0, 2)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_fp8_cache_attention_uses_dequantised_values():
    w = workloads.small_decode(11, [20, 5], num_q_heads=4, num_kv_heads=2, head_dim=16,
                               block_size=4, dtype="bf16", cache_dtype="fp8")
    w.k_scale, w.v_scale = 0.5, 0.25
    tabs, kp, vp, bt, cu, q = _setup(w)
    assert kp.dtype == np.uint8
    out, _ = attention.paged_attention(q, kp, vp, "fp8", bt, w.seq_lens, cu, 0.25, 2,
                                       k_scale=0.5, v_scale=0.25)
    from oracle import fp8
    for s in range(2):
        k, v = w.kv(s)
        Kd = fp8.decode(fp8.encode(workloads.bf16_to_f32(k), 0.5), 0.5)
        Vd = fp8.decode(fp8.encode(workloads.bf16_to_f32(v), 0.25), 0.25)
        ref = _sdpa(q[s:s + 1], Kd, Vd, [int(w.seq_lens[s]) - 1], 0.25, 2)
        np.testing.assert_allclose(out[s:s + 1], ref, rtol=1e-12, atol=1e-13)
