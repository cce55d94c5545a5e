"""Pins for the oracle's E4M3 format code, from the format definition and an
independent library conversion (torch's float8_e4m3fn cast on the CPU)."""

import math

import numpy as np
import pytest
import torch

from oracle.fp8 import e4m3_decode, e4m3_encode, e4m3_quantize, e4m3_dequantize


def test_named_codes():
    # values fixed by the bit layout: sign | exponent (bias 7) | 3-bit mantissa
    assert e4m3_decode(0x00) == 0.0
    assert e4m3_decode(0x38) == 1.0            # e = 7, m = 0
    assert e4m3_decode(0x39) == 1.125
    assert e4m3_decode(0xC0) == -2.0           # sign, e = 8
    assert e4m3_decode(0x7E) == 448.0          # largest finite: 1.75 * 2^8
    assert e4m3_decode(0x01) == 2.0 ** -9      # smallest subnormal
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert e4m3_decode(0x08) == 2.0 ** -6      # smallest normal
    assert math.isnan(e4m3_decode(0x7F)) and math.isnan(e4m3_decode(0xFF))


def test_every_finite_code_round_trips():
    n = 0
    for c in range(256):
        v = e4m3_decode(c)
        if math.isnan(v):
            continue
        n += 1
        assert e4m3_encode(v) == c, hex(c)
    assert n == 254


def test_ties_go_to_even_code_and_saturation():
    assert e4m3_encode(1.0625) == 0x38        # midway 1.0 / 1.125 -> even 0x38
    assert e4m3_encode(1.1875) == 0x3A        # midway 1.125 / 1.25 -> even 0x3A
    assert e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert e4m3_encode(0.5 * 2.0 ** -9) == 0x00
    assert e4m3_encode(1e9) == 0x7E
    assert e4m3_encode(-1e9) == 0xFE
    assert e4m3_encode(-0.0) == 0x80
    assert e4m3_encode(464.0) == 0x7E


def test_monotone_decode():
    vals = [e4m3_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_quantize_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000).astype(np.float32) * 3).astype(np.float16)
    scale = np.float32(np.abs(x.astype(np.float32)).max() / np.float32(448.0))
    codes = e4m3_quantize(x, scale)
    q = np.clip(x.astype(np.float32) / scale, -448, 448).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # dequantised values are code * scale exactly in float64
    back = e4m3_dequantize(codes, scale)
    exp = torch.from_numpy(ref).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(scale)
    assert np.array_equal(back, exp)


def test_quantize_relative_error_bound():
    # round-to-nearest with 3 mantissa bits: relative error <= 2^-4 for normals
    rng = np.random.default_rng(8)
    x = rng.uniform(0.02, 400, 50000).astype(np.float32)
    codes = e4m3_quantize(x, 1.0)
    back = e4m3_dequantize(codes, 1.0)
    rel = np.abs(back - x) / x
    assert rel.max() <= 2.0 ** -4 + 1e-12
