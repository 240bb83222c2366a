"""Large score jumps late in the context, on every attention launch path, against the
oracle element by element.

The softmax of "Project 17", "Step 6" holds for any range of scores. The kernels keep a
running maximum per row (the chunk kernel moves its reference only when a score passes
it by more than 8 in log2 units), so a key whose score jumps far above everything before
it, after the first tile or piece, must rescale what was summed so far. The seeded inputs
are bounded (|x| <= 2.95 sigma), so such keys are planted: the K row at a chosen late
position is set to a power-of-two multiple of one query row of its group (exact in bf16;
E4M3 caches get the encoded codes), the same bytes on the device and in the oracle's
planes. With |q|^2 ~ head_dim, factor c lifts that head's score by about
c * sqrt(head_dim) * log2(e) log2 units: c = 1 gives a jump of ~16 (d 128), c = 32 one of
~520; c = -32 plants a key no row can weigh."""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import fp8 as ofp8

from gpu_setup import (assert_close, build_step, oracle_attention_full, oracle_planes, oracle_scales, out_f64,
                       report_error, run_decode, run_decode_split, run_mixed, run_mixed_two_launch, run_varlen)

pytestmark = pytest.mark.gpu

LSE_ATOL = 2.0 ** -8
FACTORS = (32.0, 1.0, -32.0, 4.0)


def lse_rtol(head_dim):
    """Relative part of the log-sum-exp bound: a planted score is a head_dim-term fp32 dot
    product of a few hundred (natural log units); each matrix-core accumulation step may
    round by up to one fp32 unit (2^-23 relative, not necessarily to nearest), so the
    score, and the log-sum-exp it dominates, may move by head_dim * 2^-23 of itself on
    top of the 2^-8 that the bf16 weights allow."""
    return head_dim * 2.0 ** -23


def _plant(st, kp, plants):
    """plants: (sequence, position, query token, query head, factor). The K row of the
    query head's KV head at that position becomes factor x that query row, on the device
    and in the oracle's plane kp."""
    w = st.w
    kscale, _ = oracle_scales(w)
    for s, p, t, h, f in plants:
        assert 0 <= p < w.seq_lens[s] and 0 <= t < w.q_lens[s]
        g = h // w.group
        x = workloads.bf16_to_f32(w.q(s)[t, h]) * np.float32(f)          # exact (power of two)
        if w.cache_dtype == "fp8":
            sc = kscale[g] if np.ndim(kscale) else kscale
            bits = ofp8.encode(x, sc).astype(np.uint8)
            dev = st.k_cache
            src = torch.from_numpy(bits)
        else:
            bits = workloads.bf16_bits(x)
            dev = st.k_cache.view(torch.int16)
            src = torch.from_numpy(bits.view(np.int16))
        blk, off = int(st.bt[s, p // w.block_size]), p % w.block_size
        kp[blk, off, g] = bits
        dev[blk, off, g] = src.cuda()
    torch.cuda.synchronize()


def _decode_plants(w, rng):
    """Late keys for decode rows: in the last tiles and in the middle (later slots or
    partitions than the first), several factors per sequence."""
    plants = []
    for s, L in enumerate(w.seq_lens):
        L = int(L)
        if L < 40:
            continue
        for i, p in enumerate((L - 3, L // 2 + 17, max(17, L // 4 + 5))):
            plants.append((s, p, 0, int(rng.integers(w.num_q_heads)), FACTORS[(s + i) % len(FACTORS)]))
    return plants


@pytest.mark.parametrize("cdt", ["bf16", "fp8"])
def test_decode_paths_with_late_outlier_keys(cdt):
    w = workloads.small_decode(61, [3000, 700, 129, 4097, 40, 1500], num_q_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    tabs, bt, cu, slots, kp, vp = oracle_planes(st)
    _plant(st, kp, _decode_plants(w, np.random.default_rng(61)))
    ref, ref_lse = oracle_attention_full(st, kp, vp, bt, cu)
    assert ref_lse.max() > 100, "the planted keys must dominate some rows"
    runs = [(f"split {n} slots", run_decode_split(st, num_slots=n)[:2]) for n in (None, 7, 40, 300)]
    runs += [(f"partitioned P={P}", run_decode(st, partition_size=P)) for P in (0, 16, 512)]
    for tag, (out, lse) in runs:
        o, l_ = out_f64(out), lse.cpu().numpy().astype(np.float64)
        report_error(f"outlier keys, {cdt} cache, {tag}", o, ref, l_, ref_lse)
        assert_close(o, ref, cdt, tag)
        np.testing.assert_allclose(l_, ref_lse, rtol=lse_rtol(w.head_dim), atol=LSE_ATOL)


MIXED = [("bf16", 128, 4, 2), ("bf16", 64, 8, 2), ("fp8", 128, 4, 2), ("bf16", 128, 1, 2), ("bf16", 128, 4, 8),
         ("fp8", 64, 4, 8)]


@pytest.mark.parametrize("cdt,d,G,Hkv", MIXED, ids=[f"{a}-d{b}-g{c}-kv{e}" for a, b, c, e in MIXED])
def test_mixed_paths_with_late_outlier_keys(cdt, d, G, Hkv):
    seed = zlib.crc32(f"out{cdt}{d}{G}{Hkv}".encode()) % 10_000
    # decode rows, a chunk after a long cached prefix, a full prefill, a short chunk
    L = [600, 1300, 400, 2000, 90]
    q = [1, 300, 400, 1, 37]
    w = workloads.small_varlen(seed, L, q, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, block_size=16,
                               dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    tabs, bt, cu, slots, kp, vp = oracle_planes(st)
    rng = np.random.default_rng(seed)
    plants = []
    for s in range(w.num_seqs):
        Ls, qs = int(L[s]), int(q[s])
        c0 = Ls - qs
        for i, t in enumerate(sorted({qs - 1, qs // 2, min(qs - 1, 70)})):
            pos = c0 + t                                   # the query token's own position
            for p in {pos, max(0, pos - 5), max(65, min(pos, c0 // 2 + 65))}:
                if p <= pos and p >= 65:                   # past the first 64-key tile, visible to the row
                    plants.append((s, p, t, int(rng.integers(w.num_q_heads)), FACTORS[(s + i + p) % len(FACTORS)]))
    _plant(st, kp, plants)
    ref, ref_lse = oracle_attention_full(st, kp, vp, bt, cu)
    assert ref_lse.max() > 100, "the planted keys must dominate some rows"
    runs = [("one launch", run_varlen(st))]
    # split decode + chunk kernel: uncut, cut over resident slots, cut into single tiles
    # (a row whose first pieces are wholly masked), a small cut with a minimum piece
    for n, cs, mpt in ((None, 0, 0), (None, None, 0), (3, 5000, 0), (None, 7, 2)):
        runs.append((f"two launches ({n} / {cs} / {mpt})", run_mixed_two_launch(st, num_slots=n, chunk_slots=cs,
                                                                                min_piece_tiles=mpt)))
    # the mixed entry point (one launch with 8k KV heads)
    for n, cs, mpt in ((None, None, 0), (1, 5000, 0), (3, 0, 0)):
        runs.append((f"mixed entry ({n} / {cs} / {mpt})", run_mixed(st, num_slots=n, chunk_slots=cs,
                                                                   min_piece_tiles=mpt)))
    for tag, (out, lse) in runs:
        o, l_ = out_f64(out), lse.cpu().numpy().astype(np.float64)
        assert not np.isnan(o).any(), f"{tag}: unwritten rows"
        report_error(f"outlier keys, {cdt} d{d} G{G}, {tag}", o, ref, l_, ref_lse)
        assert_close(o, ref, cdt, tag)
        np.testing.assert_allclose(l_, ref_lse, rtol=lse_rtol(d), atol=LSE_ATOL)
