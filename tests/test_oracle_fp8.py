"""Pins for the oracle's OCP E4M3 codec."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_values_fixed_by_format():
    d = fp8.decode_code
    assert d(0x38) == 1.0            # exponent 7 = bias
    assert d(0x7E) == 448.0          # largest finite: 1.75 * 2**8
    assert d(0x01) == 2.0 ** -9      # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert d(0x08) == 2.0 ** -6      # smallest normal
    assert d(0x40) == 2.0
    assert d(0xC0) == -2.0
    assert d(0x00) == 0.0 and math.copysign(1, d(0x80)) < 0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    finite = [d(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(finite, finite[1:]))   # strictly increasing


def test_round_trip_of_every_code():
    for c in range(256):
        v = fp8.decode_code(c)
        got = int(fp8.encode(np.float32(v))[()])
        if math.isnan(v):
            assert got & 0x7F == 0x7F
        else:
            assert got == c, (hex(c), v, hex(got))


def test_ties_to_even_and_saturation():
    e = lambda x: int(fp8.encode(np.float32(x))[()])
    assert e(1.0625) == 0x38      # midway 1.0 / 1.125 -> even mantissa
    assert e(1.1875) == 0x3A      # midway 1.125 / 1.25 -> even mantissa
    assert e(2.0 ** -10) == 0x00  # midway 0 / 2**-9 -> 0
    assert e(3 * 2.0 ** -10) == 0x02
    assert e(449.0) == 0x7E and e(1e9) == 0x7E and e(-1e9) == 0xFE
    assert e(np.inf) == 0x7E and e(-np.inf) == 0xFE
    assert e(np.nan) & 0x7F == 0x7F
    assert e(-0.0) == 0x80 and e(-1e-30) == 0x80


def test_scale_divides_before_rounding():
    x = np.linspace(-900, 900, 301).astype(np.float32)
    assert (fp8.encode(x, 2.0) == fp8.encode(x * np.float32(0.5))).all()
    np.testing.assert_array_equal(fp8.decode(fp8.encode(x, 4.0), 4.0) / 4.0,
                                  fp8.decode(fp8.encode(x * np.float32(0.25))))


def _torch_codes(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_exhaustive_bf16_inputs_against_torch_cast():
    # every bf16 bit pattern, widened to float32; torch's cast is an independent
    # round-to-nearest-even E4M3 conversion; it overflows (NaN) from 464 up, where
    # this codec saturates instead, so only |x| < 464 is compared with it.
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32)
    ours = fp8.encode(x)
    ok = np.isfinite(x) & (np.abs(x) < 464.0)
    theirs = _torch_codes(np.where(ok, x, 0).astype(np.float32))
    np.testing.assert_array_equal(ours[ok], theirs[ok])
    big = np.isfinite(x) & (np.abs(x) >= 464.0)
    assert ((ours[big] & 0x7F) == 0x7E).all()


def test_random_float32_inputs_against_torch_cast():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-12, 6, 200_000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    np.testing.assert_array_equal(fp8.encode(x), _torch_codes(x))


def test_per_head_scales_reduce_to_per_tensor_and_follow_the_head_axis():
    # per-head scale = per-tensor scale x head factor (float64 product of float32 values)
    hs = fp8.head_scales(0.5, np.array([1.0, 3.0, 0.25], np.float32))
    assert hs.tolist() == [0.5, 1.5, 0.125]
    rng = np.random.default_rng(5)
    x = rng.normal(0, 2, (7, 3, 16)).astype(np.float32)          # [T][Hkv][d]
    # all factors 1: identical codes to the per-tensor encoder
    ones = fp8.head_scales(0.5, np.ones(3, np.float32))
    assert (fp8.encode(x, ones[:, None]) == fp8.encode(x, 0.5)).all()
    # each head's slice is the per-tensor encoding with that head's scale
    codes = fp8.encode(x, hs[:, None])
    for h in range(3):
        assert (codes[:, h] == fp8.encode(x[:, h], float(hs[h]))).all()
    # decode by hand: code 0x38 is 1.0, so head h decodes it to its scale
    c = np.full((2, 3, 4), 0x38, np.uint8)
    assert (fp8.decode(c, hs[:, None]) == np.broadcast_to(hs[:, None], (2, 3, 4))).all()


def test_paged_attention_with_per_head_scales_equals_hand_dequantised_dense():
    from oracle import attention as oatt
    from oracle import cache as ocache
    rng = np.random.default_rng(9)
    T, Hkv, d, G, bs = 11, 2, 8, 2, 4
    ks = fp8.head_scales(0.5, np.array([0.25, 4.0], np.float32))
    vs = fp8.head_scales(2.0, np.array([1.5, 0.125], np.float32))
    k = rng.normal(0, 1, (T, Hkv, d)).astype(np.float32)
    v = rng.normal(0, 1, (T, Hkv, d)).astype(np.float32)
    kp = ocache.empty_plane(3, bs, Hkv, d, "fp8")
    vp = ocache.empty_plane(3, bs, Hkv, d, "fp8")
    slots = np.array([8, 9, 10, 11, 0, 1, 2, 3, 4, 5, 6])        # blocks 2, 0, 1
    ocache.write(kp, k, "f32", "fp8", slots, ks)
    ocache.write(vp, v, "f32", "fp8", slots, vs)
    q = rng.normal(0, 1, (1, Hkv * G, d))
    out, _ = oatt.paged_attention(q, kp, vp, "fp8", np.array([[2, 0, 1]], np.int32), [T], [0, 1], 0.3, G, ks, vs)
    # by hand: codes of each head times that head's scale, then plain attention
    K = np.stack([fp8.decode(fp8.encode(k[:, h], float(ks[h])), float(ks[h])) for h in range(Hkv)], 1)
    V = np.stack([fp8.decode(fp8.encode(v[:, h], float(vs[h])), float(vs[h])) for h in range(Hkv)], 1)
    ref, _ = oatt.attend(q, K, V, [T - 1], 0.3, G)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
