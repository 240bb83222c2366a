"""Per-KV-head E4M3 scales on the GPU: every attention launch (decode with and without
context partitions, the balanced-split decode, the varlen kernel, and the mixed step as
split decode + chunk kernel, cut and uncut, and the mixed entry) against the oracle on caches written with a
different scale per KV head. Distinct factors per head make a wrong head index show as a
large error. The cache bytes themselves are checked in test_gpu_cache_write.py."""
import numpy as np
import pytest

import paged_kv_cache_42_amd as pkv
import workloads

from gpu_setup import (assert_close, build_step, oracle_attention_full, oracle_planes, out_f64, run_decode,
                       run_decode_split, run_mixed, run_mixed_two_launch, run_varlen)

pytestmark = pytest.mark.gpu

K_HEAD = np.array([0.25, 3.0, 1.0, 0.7, 5.5, 0.125, 1.3, 2.0], np.float32)
V_HEAD = np.array([2.0, 0.3, 0.5, 4.0, 1.0, 0.9, 8.0, 0.0625], np.float32)


def _scaled(w):
    w.k_scale, w.v_scale = 0.5, 0.25
    w.k_head_scales = K_HEAD[:w.num_kv_heads].copy()
    w.v_head_scales = V_HEAD[:w.num_kv_heads].copy()
    return w


def _oracle(w):
    st = build_step(w)
    tabs, bt, cu, slots, kp, vp = oracle_planes(st)
    ref, _ = oracle_attention_full(st, kp, vp, bt, cu)
    return st, ref


@pytest.mark.parametrize("d,hkv,G", [(64, 2, 4), (128, 8, 2), (64, 8, 1)])
def test_decode_paths_per_head(d, hkv, G):
    w = _scaled(workloads.small_decode(61 + d + hkv, [1, 15, 16, 17, 100, 333, 64], num_q_heads=hkv * G,
                                       num_kv_heads=hkv, head_dim=d, block_size=16, dtype="bf16",
                                       cache_dtype="fp8"))
    st, ref = _oracle(w)
    for P in (0, 32):
        out, _ = run_decode(st, partition_size=P)
        assert_close(out_f64(out), ref, "fp8", f"decode P={P}")
    for slots in (None, 5):
        out, _, _ = run_decode_split(st, num_slots=slots)
        assert_close(out_f64(out), ref, "fp8", f"split slots={slots}")


@pytest.mark.parametrize("d,hkv,G", [(64, 2, 4), (128, 8, 2)])
def test_mixed_step_paths_per_head(d, hkv, G):
    w = _scaled(workloads.small_varlen(71 + d + hkv, [300, 64, 7, 130, 1], [200, 10, 1, 130, 1],
                                       num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=d, block_size=16,
                                       dtype="bf16", cache_dtype="fp8"))
    st, ref = _oracle(w)
    out, _ = run_varlen(st)
    assert_close(out_f64(out), ref, "fp8", "varlen")
    for chunk_slots in (0, None):
        out, _ = run_mixed_two_launch(st, chunk_slots=chunk_slots)
        assert_close(out_f64(out), ref, "fp8", f"two-launch chunk_slots={chunk_slots}")
    # the mixed entry: one launch of decode slots beside chunk items at 8 KV heads
    for num_slots, chunk_slots in ((None, None), (3, 0)):
        out, _ = run_mixed(st, num_slots=num_slots, chunk_slots=chunk_slots)
        assert_close(out_f64(out), ref, "fp8", f"mixed entry slots={num_slots} chunk_slots={chunk_slots}")


def test_per_head_argument_errors():
    import torch
    w = workloads.small_decode(81, [5], num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16",
                               cache_dtype="fp8")
    st = build_step(w)
    for kh in (np.array([1.0, -1.0], np.float32), np.array([1.0, np.inf], np.float32)):
        with pytest.raises(pkv.PkvError):
            run = pkv.paged_attention_decode
            out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
            run(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, 2, 16, 5, w.softmax_scale,
                k_head_scales=kh)
    with pytest.raises(ValueError):
        out = torch.empty((1, 4, 64), dtype=torch.bfloat16, device="cuda")
        pkv.paged_attention_decode(out, st.q, st.k_cache, st.v_cache, st.bt_d, st.lens_d, 2, 16, 5,
                                   w.softmax_scale, k_head_scales=np.ones(3, np.float32))
