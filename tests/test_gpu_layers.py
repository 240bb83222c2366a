"""Layer-batched launches (the *_layers entry points: one launch per kernel for several
layers that share a step's metadata) against one launch per layer. The kernels are the
same, so every layer's cache bytes, outputs and log-sum-exps must be bit-identical to the
per-layer call on that layer's own tensors. The layers' planes differ (blocks rotated,
signs flipped on odd layers), their queries sit in one buffer with a gap between layers,
and the decode and chunk plans split sequences, so each layer also has partials of its
own in the shared workspace."""
import numpy as np
import pytest
import torch

import paged_kv_cache_42_amd as pkv
import workloads
from gpu_setup import build_step

pytestmark = pytest.mark.gpu

NL = 3


def _flip(x):
    """Sign flip, bit-exact for bf16 and E4M3 codes."""
    if x.dtype == torch.uint8:
        return x ^ 0x80
    return (x.view(torch.int16) ^ -32768).view(x.dtype)


def _finite(x):
    """The plane with its NaN codes (the fill of unused blocks) made finite, so that blocks
    rotated into use read numbers: E4M3 0x7f / 0xff -> 0x7e / 0xfe, bf16 NaN -> 0."""
    if x.dtype == torch.uint8:
        return torch.where((x & 0x7F) == 0x7F, x - 1, x)
    return torch.where(torch.isnan(x), torch.zeros_like(x), x)


def _layer_planes(plane):
    """[NL][...] contiguous: layer l = plane with its blocks rotated by l, signs flipped on
    odd l, NaN codes made finite."""
    return torch.stack([_finite(_flip(torch.roll(plane, l, 0)) if l % 2 else torch.roll(plane, l, 0))
                        for l in range(NL)]).contiguous()


def _all_written(out, what):
    bad = torch.isnan(out.float()).flatten(2).any(dim=2).nonzero().tolist()
    assert not bad, f"{what}: (layer, row) pairs never written or NaN: {bad[:20]}"


def _strided(xs, gap_rows=5):
    """The per-layer tensors xs [T][H][d] as one [NL][T][H][d] view with a NaN gap between layers."""
    T, H, d = xs[0].shape
    per = (T + gap_rows) * H * d
    buf = torch.full((NL * per,), float("nan"), dtype=xs[0].dtype, device="cuda")
    v = buf.as_strided((NL, T, H, d), (per, H * d, d, 1))
    for l, x in enumerate(xs):
        v[l].copy_(x)
    return v


def _queries(q):
    return [_flip(torch.roll(q, l, 0)) if l % 2 else torch.roll(q, l, 0) for l in range(NL)]


def _same(a, b, what):
    ai = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32) if a.dtype == torch.float32 else a
    bi = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32) if b.dtype == torch.float32 else b
    assert torch.equal(ai, bi), f"{what}: layer-batched result differs from the per-layer call"


@pytest.mark.parametrize("cdt", ["bf16", "fp8"])
def test_cache_write_layers(cdt):
    w = workloads.small_varlen(71, [300, 40, 1000], [300, 1, 77], num_q_heads=16, num_kv_heads=4, head_dim=128,
                               block_size=16, dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    slots = torch.from_numpy(st.slots).cuda()
    T = w.total_q
    g = torch.Generator(device="cuda").manual_seed(5)
    ks = [torch.randn((T, w.num_kv_heads, w.head_dim), device="cuda", generator=g).bfloat16() for _ in range(NL)]
    vs = [torch.randn((T, w.num_kv_heads, w.head_dim), device="cuda", generator=g).bfloat16() for _ in range(NL)]
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    kc_ref, vc_ref = kc.clone(), vc.clone()
    for l in range(NL):
        pkv.kv_cache_write(ks[l], vs[l], kc_ref[l], vc_ref[l], slots, w.block_size, w.k_scale, w.v_scale)
    pkv.kv_cache_write(_strided(ks), _strided(vs), kc, vc, slots, w.block_size, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    _same(kc, kc_ref, "K planes")
    _same(vc, vc_ref, "V planes")


@pytest.mark.parametrize("cdt,d", [("bf16", 128), ("fp8", 128), ("bf16", 64)])
def test_decode_split_layers(cdt, d):
    w = workloads.small_decode(72, [3000, 129, 4097, 1, 700, 16, 2500, 2, 33], num_q_heads=32, num_kv_heads=8,
                               head_dim=d, block_size=16, dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    B, Hq = w.num_seqs, w.num_q_heads
    msl = int(w.seq_lens.max())
    split = pkv.build_decode_split(w.seq_lens, 37)
    assert split.max_pieces > 1, "the plan must leave partials"
    plan_d = torch.from_numpy(split.plan).cuda()
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    qs = _queries(st.q)
    args = (st.bt_d, st.lens_d, plan_d, split, w.num_kv_heads, w.block_size, msl, w.softmax_scale, w.k_scale,
            w.v_scale)
    ref = []
    for l in range(NL):
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attention_decode_split(out, qs[l], kc[l], vc[l], *args, pkv.decode_split_workspace(split, Hq, d),
                                         lse)
        ref.append((out, lse))
    out = torch.full((NL, B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((NL, B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = pkv.decode_split_workspace(split, Hq, d, num_layers=NL)
    ws.view(torch.uint8).fill_(0x7F)
    pkv.paged_attention_decode_split(out, _strided(qs), kc, vc, *args, ws, lse)
    torch.cuda.synchronize()
    for l in range(NL):
        _same(out[l], ref[l][0], f"layer {l} output")
        _same(lse[l], ref[l][1], f"layer {l} log-sum-exp")
    assert not torch.equal(ref[0][0].view(torch.int16), ref[1][0].view(torch.int16)), "layers must differ"
    _all_written(out, "split decode")


@pytest.mark.parametrize("cdt,d,G", [("bf16", 128, 4), ("fp8", 128, 4), ("bf16", 64, 8)])
def test_chunks_and_mixed_step_layers(cdt, d, G):
    Hkv = 2
    w = workloads.small_varlen(73, [600, 1300, 400, 2000, 90, 3], [1, 300, 400, 1, 37, 3], num_q_heads=Hkv * G,
                               num_kv_heads=Hkv, head_dim=d, block_size=16, dtype="bf16", cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    T, Hq = w.total_q, w.num_q_heads
    msl = int(w.seq_lens.max())
    mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, Hkv, G, 5, 0, 64)
    assert mp.chunks.num_partials > 0 and mp.split.max_pieces > 1, "both plans must leave partials"
    plan_d = torch.from_numpy(mp.split.plan).cuda()
    rows = torch.from_numpy(mp.decode_rows).cuda()
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    qs = _queries(st.q)

    def step(out, q, k, v, lse, nl):
        pkv.paged_attention_decode_split(out, q, k, v, st.bt_d, st.lens_d, plan_d, mp.split, Hkv, w.block_size, msl,
                                         w.softmax_scale, w.k_scale, w.v_scale,
                                         pkv.decode_split_workspace(mp.split, Hq, d, num_layers=nl), lse, rows=rows,
                                         cu_seqlens_q=st.cu_d)
        work, merges, cws = mp.chunks.to_device(d, num_layers=nl)
        pkv.paged_attention_prefill_chunks(out, q, k, v, st.bt_d, st.lens_d, st.cu_d, work, merges,
                                           mp.chunks.num_partials, cws, Hkv, w.block_size, msl, w.softmax_scale,
                                           w.k_scale, w.v_scale, lse=lse)

    ref = []
    for l in range(NL):
        out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        step(out, qs[l], kc[l], vc[l], lse, 1)
        ref.append((out, lse))
    out = torch.full((NL, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((NL, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    step(out, _strided(qs), kc, vc, lse, NL)
    torch.cuda.synchronize()
    for l in range(NL):
        _same(out[l], ref[l][0], f"layer {l} output")
        _same(lse[l], ref[l][1], f"layer {l} log-sum-exp")
    _all_written(out, "mixed step")


@pytest.mark.parametrize("cdt,d,G", [("bf16", 128, 4), ("fp8", 128, 4), ("bf16", 64, 8), ("fp8", 64, 4)])
def test_mixed_entry_one_launch_and_layers(cdt, d, G):
    """pkv_paged_attention_mixed (one launch: decode slots and chunk items in one grid) and
    its layer-batched form against the split decode + chunk kernel of the same plan, per
    layer: the same device code on the same work, so bit-identical."""
    Hkv = 8
    w = workloads.small_varlen(79, [600, 1300, 400, 2000, 90, 3, 250], [1, 300, 400, 1, 37, 3, 1],
                               num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d, block_size=16, dtype="bf16",
                               cache_dtype=cdt)
    if cdt == "fp8":
        w.k_scale, w.v_scale = 0.5, 0.25
    st = build_step(w)
    T, Hq = w.total_q, w.num_q_heads
    msl = int(w.seq_lens.max())
    mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, Hkv, G, 5, 0, 256)
    assert mp.chunks.num_partials > 0 and mp.split.max_pieces > 1, "both plans must leave partials"
    plan_d = torch.from_numpy(mp.split.plan).cuda()
    rows = torch.from_numpy(mp.decode_rows).cuda()
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    qs = _queries(st.q)
    ref = []
    for l in range(NL):
        out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attention_decode_split(out, qs[l], kc[l], vc[l], st.bt_d, st.lens_d, plan_d, mp.split, Hkv,
                                         w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale,
                                         pkv.decode_split_workspace(mp.split, Hq, d), lse, rows=rows,
                                         cu_seqlens_q=st.cu_d)
        work, merges, cws = mp.chunks.to_device(d)
        pkv.paged_attention_prefill_chunks(out, qs[l], kc[l], vc[l], st.bt_d, st.lens_d, st.cu_d, work, merges,
                                           mp.chunks.num_partials, cws, Hkv, w.block_size, msl, w.softmax_scale,
                                           w.k_scale, w.v_scale, lse=lse)
        ref.append((out, lse))
        one = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        one_lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attention_mixed(one, qs[l], kc[l], vc[l], st.bt_d, st.lens_d, st.cu_d, mp, mp.to_device(d, Hq),
                                  Hkv, w.block_size, msl, w.softmax_scale, w.k_scale, w.v_scale, lse=one_lse)
        torch.cuda.synchronize()
        _same(one, out, f"layer {l} one-launch output")
        _same(one_lse, lse, f"layer {l} one-launch log-sum-exp")
    out = torch.full((NL, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((NL, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attention_mixed(out, _strided(qs), kc, vc, st.bt_d, st.lens_d, st.cu_d, mp,
                              mp.to_device(d, Hq, num_layers=NL), Hkv, w.block_size, msl, w.softmax_scale,
                              w.k_scale, w.v_scale, lse=lse)
    torch.cuda.synchronize()
    for l in range(NL):
        _same(out[l], ref[l][0], f"layer {l} layer-batched one-launch output")
        _same(lse[l], ref[l][1], f"layer {l} layer-batched one-launch log-sum-exp")
    _all_written(out, "layer-batched mixed step")


K_HEAD = np.array([0.25, 3.0, 1.0, 0.7], np.float32)
V_HEAD = np.array([2.0, 0.3, 0.5, 4.0], np.float32)


def test_layers_with_per_head_e4m3_scales():
    """The layer-batched cache write, split decode and chunk kernel with per-KV-head E4M3
    scales (shared by the layers, as the entry points define them): every layer's cache
    codes, outputs and log-sum-exps bit-identical to the per-layer calls with the same
    head scales."""
    Hkv, G, d = 4, 4, 128
    w = workloads.small_varlen(75, [700, 1200, 40, 1500, 300], [1, 260, 3, 1, 300], num_q_heads=Hkv * G,
                               num_kv_heads=Hkv, head_dim=d, block_size=16, dtype="bf16", cache_dtype="fp8")
    w.k_scale, w.v_scale = 0.5, 0.25
    kh = K_HEAD.copy()
    vh = V_HEAD.copy()
    st = build_step(w)
    T, Hq = w.total_q, w.num_q_heads
    slots = torch.from_numpy(st.slots).cuda()
    g = torch.Generator(device="cuda").manual_seed(9)
    ks = [torch.randn((T, Hkv, d), device="cuda", generator=g).bfloat16() for _ in range(NL)]
    vs = [torch.randn((T, Hkv, d), device="cuda", generator=g).bfloat16() for _ in range(NL)]
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    kc_ref, vc_ref = kc.clone(), vc.clone()
    for l in range(NL):
        pkv.kv_cache_write(ks[l], vs[l], kc_ref[l], vc_ref[l], slots, w.block_size, w.k_scale, w.v_scale,
                           k_head_scales=kh, v_head_scales=vh)
    pkv.kv_cache_write(_strided(ks), _strided(vs), kc, vc, slots, w.block_size, w.k_scale, w.v_scale,
                       k_head_scales=kh, v_head_scales=vh)
    torch.cuda.synchronize()
    _same(kc, kc_ref, "K codes")
    _same(vc, vc_ref, "V codes")

    msl = int(w.seq_lens.max())
    mp = pkv.build_mixed_step(w.q_lens, w.seq_lens, Hkv, G, 7, 0, 64)
    assert mp.chunks.num_partials > 0 and mp.split.max_pieces > 1, "both plans must leave partials"
    plan_d = torch.from_numpy(mp.split.plan).cuda()
    rows = torch.from_numpy(mp.decode_rows).cuda()
    qs = _queries(st.q)

    def step(out, q, k, v, lse, nl):
        pkv.paged_attention_decode_split(out, q, k, v, st.bt_d, st.lens_d, plan_d, mp.split, Hkv, w.block_size, msl,
                                         w.softmax_scale, w.k_scale, w.v_scale,
                                         pkv.decode_split_workspace(mp.split, Hq, d, num_layers=nl), lse, rows=rows,
                                         cu_seqlens_q=st.cu_d, k_head_scales=kh, v_head_scales=vh)
        work, merges, cws = mp.chunks.to_device(d, num_layers=nl)
        pkv.paged_attention_prefill_chunks(out, q, k, v, st.bt_d, st.lens_d, st.cu_d, work, merges,
                                           mp.chunks.num_partials, cws, Hkv, w.block_size, msl, w.softmax_scale,
                                           w.k_scale, w.v_scale, lse=lse, k_head_scales=kh, v_head_scales=vh)

    ref = []
    for l in range(NL):
        out = torch.full((T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        step(out, qs[l], kc[l], vc[l], lse, 1)
        ref.append((out, lse))
    out = torch.full((NL, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((NL, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    step(out, _strided(qs), kc, vc, lse, NL)
    torch.cuda.synchronize()
    for l in range(NL):
        _same(out[l], ref[l][0], f"layer {l} output")
        _same(lse[l], ref[l][1], f"layer {l} log-sum-exp")
    _all_written(out, "mixed step with per-head scales")


def test_layer_descriptor_errors():
    w = workloads.small_decode(74, [100, 50], num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                               dtype="bf16")
    st = build_step(w)
    kc, vc = _layer_planes(st.k_cache), _layer_planes(st.v_cache)
    slots = torch.from_numpy(st.slots).cuda()
    k = torch.zeros((NL, 2, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="layer axis"):
        pkv.kv_cache_write(k[:2], k[:2], kc, vc, slots, 16)
    # a layer-batched write over overlapping layers is refused before the call
    ov = k.as_strided((NL, 2, 2, 64), (64, 128, 64, 1))
    with pytest.raises(ValueError, match="overlap"):
        pkv.kv_cache_write(ov, ov, kc, vc, slots, 16)
