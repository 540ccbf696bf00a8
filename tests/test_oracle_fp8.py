"""Pins for the oracle's OCP E4M3 decode/encode (CPU only)."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8_e4m3 as fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_values.txt")


def _spec_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


@pytest.mark.parametrize("code,value", _spec_rows())
def test_decode_matches_spec_table(code, value):
    got = fp8.DECODE_TABLE[code]
    if math.isnan(value):
        assert math.isnan(got)
    else:
        assert got == value
        assert math.copysign(1.0, got) == math.copysign(1.0, value)


def test_decode_matches_torch_for_all_codes():
    # torch's float8_e4m3fn storage type is an independent implementation
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.DECODE_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_only_two_nan_codes_and_monotone_positive_codes():
    assert sorted(np.flatnonzero(np.isnan(fp8.DECODE_TABLE)).tolist()) == [0x7F, 0xFF]
    pos = fp8.DECODE_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(fp8.DECODE_TABLE[0x80:0xFF], -pos)


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.DECODE_TABLE[codes].astype(np.float32)
    assert np.array_equal(fp8.encode(vals, 1.0), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    pos = fp8.DECODE_TABLE[:0x7F]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = np.float32((lo + hi) / 2)          # 5 significant bits: exact in fp32
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert fp8.encode(mid, 1.0) == even, hex(c)
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1e9))
        assert fp8.encode(below, 1.0) == c
        assert fp8.encode(above, 1.0) == c + 1
        assert fp8.encode(-mid, 1.0) == (even | 0x80)


def test_saturation_nan_and_signed_zero():
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e30, np.inf], dtype=np.float32)
    assert np.all(fp8.encode(big, 1.0) == 0x7E)
    assert np.all(fp8.encode(-big, 1.0) == 0xFE)
    assert fp8.encode(np.float32(np.nan), 1.0) == 0x7F
    assert fp8.encode(np.float32(-0.0), 1.0) == 0x80
    assert fp8.encode(np.float32(0.0), 1.0) == 0x00
    tiny = np.float32(2.0 ** -11)
    assert fp8.encode(tiny, 1.0) == 0x00
    assert fp8.encode(-tiny, 1.0) == 0x80
    assert fp8.encode(np.float32(2.0 ** -10), 1.0) == 0x00     # tie between 0 and 2^-9 -> even
    assert fp8.encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)), 1.0) == 0x01


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    return bits.view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.125, 0.0124163])
def test_encode_matches_torch_on_every_bf16_pattern_in_range(scale):
    x = _all_bf16_as_f32()
    s = np.float32(scale)
    with np.errstate(all="ignore"):
        y = x / s
    codes = fp8.encode(x, s)
    # torch converts without saturating; compare where |y| stays below the
    # 448/480 midpoint (both round to nearest even there) and y is not NaN
    ok = np.isfinite(y) & (np.abs(y) < 464.0)
    ref = torch.from_numpy(y[ok].copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[ok], ref)
    # everything else: NaN -> 0x7F, the rest saturates with its sign
    rest = ~ok
    exp = np.where(np.isnan(y[rest]), 0x7F, np.where(np.signbit(y[rest]), 0xFE, 0x7E))
    assert np.array_equal(codes[rest], exp.astype(np.uint8))


def test_encode_divides_in_binary32():
    # 1/3 is not exact in fp32: dividing in fp64 and rounding once could differ.
    x = np.float32(1.0)
    s = np.float32(3.0)
    y = np.float32(x / s)
    assert fp8.encode(x, s) == fp8.encode(y, 1.0)
