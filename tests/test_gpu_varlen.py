"""paged_attention_prefill_varlen (prefill chunks + decode rows in one launch) on the
GPU vs the oracle, element by element, plus invariants."""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_42_amd as pkv
import workloads

from gpu_setup import (assert_close, build_step, oracle_attention_full, oracle_planes, out_f64, run_mixed,
                       run_mixed_two_launch, run_varlen)

pytestmark = pytest.mark.gpu

LSE_ATOL = 2.0 ** -8   # weights enter P.V rounded to bf16 (see the decode tests)


# two-launch variants: (decode split slots, chunk slots, min piece tiles); None = the
# device's resident count; 5000 chunk slots cut every block into single tiles
TWO_LAUNCH = ((None, None, 0), (3, 5000, 0), (None, 7, 2), (None, 0, 0))
# pkv_paged_attention_mixed variants: (decode slots, chunk slots, min piece tiles); None
# decode slots = mixed_decode_slots
ONE_LAUNCH = ((None, None, 0), (1, 5000, 0), (None, 0, 0), (64, 7, 2))


def _check(w, two_launch=TWO_LAUNCH, one_launch=ONE_LAUNCH):
    st = build_step(w)
    tabs, bt, cu, slots, kp, vp = oracle_planes(st)
    assert (st.bt == bt).all() and (st.cu == cu).all() and (st.slots == slots).all()
    ref, ref_lse = oracle_attention_full(st, kp, vp, bt, cu)
    dt = "fp8" if w.cache_dtype == "fp8" else "bf16"
    out, lse = run_varlen(st)
    assert_close(out_f64(out), ref, dt, w.name)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
    # the same step as two launches (split decode rows + prefill-only varlen)
    for n, cs, mpt in two_launch:
        o2, l2 = run_mixed_two_launch(st, num_slots=n, chunk_slots=cs, min_piece_tiles=mpt)
        got = out_f64(o2)
        tag = f"{w.name} two launches ({n} / {cs} / {mpt})"
        assert not np.isnan(got).any(), f"{tag}: unwritten rows"
        assert_close(got, ref, dt, tag)
        np.testing.assert_allclose(l2.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
    # and through the mixed entry point (one launch with 8k KV heads)
    for n, cs, mpt in one_launch:
        o3, l3 = run_mixed(st, num_slots=n, chunk_slots=cs, min_piece_tiles=mpt)
        got = out_f64(o3)
        tag = f"{w.name} mixed entry ({n} / {cs} / {mpt})"
        assert not np.isnan(got).any(), f"{tag}: unwritten rows"
        assert_close(got, ref, dt, tag)
        np.testing.assert_allclose(l3.cpu().numpy(), ref_lse, rtol=0, atol=LSE_ATOL)
    return st, out, lse


def test_config2_mixed_step():
    w = workloads.config2()
    st, out, lse = _check(w)
    # decode rows of the mixed launch agree with the decode kernel (different splits of
    # the same context, so to rounding only)
    last = torch.from_numpy(st.cu[1:].astype(np.int64) - 1).cuda()
    q_last = st.q[last].contiguous()                 # each sequence's last new token
    o_dec = torch.empty_like(q_last)
    pkv.paged_attention_decode(o_dec, q_last, st.k_cache, st.v_cache, st.bt_d, st.lens_d, w.num_kv_heads,
                               w.block_size, int(w.seq_lens.max()), w.softmax_scale)
    torch.cuda.synchronize()
    dec = np.where(w.q_lens == 1)[0]
    rows = torch.from_numpy(st.cu[dec].astype(np.int64)).cuda()
    diff = (out[rows].float() - o_dec[torch.from_numpy(dec).cuda()].float()).abs().max().item()
    assert diff <= 2.0 ** -7, diff


CASES = []
for cdt in ("bf16", "fp8"):
    for d in (64, 128):
        for G in (1, 4, 8):
            for bs in (16, 32):
                CASES.append((cdt, d, G, bs))


@pytest.mark.parametrize("cdt,d,G,bs", CASES, ids=[f"{a}-d{b}-g{c}-bs{e}" for a, b, c, e in CASES])
def test_small_mixed_steps(cdt, d, G, bs):
    seed = zlib.crc32(f"v{cdt}{d}{G}{bs}".encode()) % 10_000
    # decode rows, short and long prefill chunks, a full prefill (no cached prefix),
    # chunks crossing tile and item boundaries, a row with no new tokens
    L = [1, 40, 300, 17, 150, 64, 513, 20, 9]
    q = [1, 1, 300, 17, 33, 2, 200, 0, 7]
    Hkv = 2
    w = workloads.small_varlen(seed, L, q, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, block_size=bs,
                               dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    _check(w)


# one-launch mixed kernel shapes (8 KV heads): bf16 at head_dim 128 with decode rows only,
# chunks only, and both; E4M3 and head_dim 64 with both; contexts crossing tiles, blocks
# and slots
ONE_CASES = [("bf16", 128, G, bs, kind) for G in (1, 4) for bs in (16, 32) for kind in ("both", "decode", "chunks")]
ONE_CASES += [(cdt, d, 4, bs, "both") for cdt, d in (("fp8", 128), ("bf16", 64), ("fp8", 64)) for bs in (16, 32)]
ONE_CASES += [("bf16", 128, 2, 16, "both-kv16"), ("fp8", 64, 2, 16, "both-kv16")]   # two KV-head groups per slot


@pytest.mark.parametrize("cdt,d,G,bs,kind", ONE_CASES, ids=[f"{a}-d{b}-g{c}-bs{e}-{f}" for a, b, c, e, f in ONE_CASES])
def test_one_launch_mixed_steps(cdt, d, G, bs, kind):
    seed = zlib.crc32(f"m{cdt}{d}{G}{bs}{kind}".encode()) % 10_000
    Hkv = 16 if kind.endswith("kv16") else 8
    kind = kind.split("-")[0]
    L = {"both": [1, 40, 300, 17, 150, 64, 513, 2000, 9, 700],
         "decode": [1, 40, 300, 17, 1500, 64, 513],
         "chunks": [300, 17, 150, 64, 513]}[kind]
    q = {"both": [1, 1, 300, 17, 33, 1, 200, 1, 7, 1],
         "decode": [1] * 7,
         "chunks": [300, 17, 33, 2, 200]}[kind]
    w = workloads.small_varlen(seed, L, q, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, block_size=bs,
                               dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    _check(w, two_launch=(), one_launch=ONE_LAUNCH + ((3, 0, 0), (1000, 0, 0)))


def test_physical_permutation_bitwise():
    L, q = [700, 129, 64, 2], [300, 1, 64, 2]
    w = workloads.small_varlen(31, L, q, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16, pool_extra=30)
    st1 = build_step(w)
    st2 = build_step(w, pool_order=np.random.default_rng(5).permutation(w.num_blocks).astype(np.int32))
    assert not (st1.bt == st2.bt).all()
    o1, l1 = run_varlen(st1)
    o2, l2 = run_varlen(st2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_unsupported_and_invalid_are_rejected():
    w = workloads.small_varlen(3, [5], [5], num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16)
    st = build_step(w)
    with pytest.raises(pkv.PkvError):
        pkv.build_varlen_work([6], [5], 2, 2)                       # q_len > seq_len
    with pytest.raises(pkv.PkvError):
        pkv.build_varlen_work([5], [5], 2, 3)                       # group 3 unsupported
    work = torch.from_numpy(pkv.build_varlen_work(w.q_lens, w.seq_lens, 2, 2)).cuda()
    out = torch.empty_like(st.q)
    with pytest.raises(pkv.PkvError):
        pkv.paged_attention_prefill_varlen(out.float(), st.q.float(), st.k_cache, st.v_cache, st.bt_d, st.lens_d,
                                           st.cu_d, work, 2, 16, 5, 0.125)   # fp32 queries unsupported
