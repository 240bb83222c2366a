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
