"""Pins of the oracle's number formats against their published definitions.

bf16 and E4M3 are checked against an independent library cast (torch) and
hand-derived format points; E2M1 against hand-derived points (OCP MX v1.0)
and structural properties.  No GPU.
"""
import struct

import numpy as np
import pytest
import torch

from conftest import read_golden


def f32_bits_to_float(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ------------------------------------------------------------------ bf16 --

def torch_bf16(a):
    return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_random_bit_patterns(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    a = f32_bits_to_float(bits)
    a = a[np.isfinite(a)]
    assert np.array_equal(orc.f32_to_bf16(a), torch_bf16(a))


def test_bf16_ties_and_overflow(orc):
    # every exact tie (low half == 0x8000) over all exponents and both signs,
    # plus the patterns just around each tie and the overflow boundary
    hi = np.arange(0, 0x7F80, dtype=np.uint32)
    ties = (hi << 16) | 0x8000
    around = np.concatenate([ties, ties - 1, ties + 1, ties | 0x80000000])
    a = f32_bits_to_float(around)
    a = a[np.isfinite(a)]
    assert np.array_equal(orc.f32_to_bf16(a), torch_bf16(a))
    big = f32_bits_to_float(np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000], np.uint32))
    got = orc.f32_to_bf16(big)
    # 0x7F7F7FFF rounds down to max finite; the rest round to +-inf
    assert list(got) == [0x7F7F, 0x7F80, 0x7F80, 0xFF80]


def test_bf16_subnormals_and_zero(orc):
    bits = np.arange(0, 1 << 23, 997, dtype=np.uint32)  # fp32 subnormals
    a = np.concatenate([f32_bits_to_float(bits), -f32_bits_to_float(bits)])
    assert np.array_equal(orc.f32_to_bf16(a), torch_bf16(a))
    assert orc.f32_to_bf16(np.array([-0.0], np.float32))[0] == 0x8000


# ------------------------------------------------------------------ E4M3 --

def test_e4m3_value_table_structure(orc):
    vals = [orc.e4m3_value(c) for c in range(127)]
    # strictly increasing, 0 first, 448 last (largest finite, code 0x7E)
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert vals[0] == 0.0 and vals[126] == 448.0
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    # uniform spacing 2^-9 through the subnormals into the first binade
    assert np.allclose(np.diff(vals[:16]), 2.0 ** -9)
    # every code equals torch's decode of the same byte
    codes = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn)
    assert vals == codes.to(torch.float64).tolist()


def test_e4m3_golden_points(orc):
    rows = [ln.split() for ln in read_golden("codec_points.txt") if ln.startswith("e4m3")]
    assert len(rows) >= 20
    vals = np.array([float(r[1]) for r in rows], np.float32)
    want = np.array([int(r[2], 16) for r in rows], np.uint8)
    assert np.array_equal(orc.e4m3_encode(vals), want)


def _e4m3_sweep():
    rng = np.random.default_rng(7)
    # random mantissas across every binade the format touches, both signs
    exps = rng.integers(-14, 10, size=400_000)
    mant = rng.random(400_000) + 1.0
    a = (mant * np.exp2(exps)).astype(np.float32)
    a[::2] *= -1
    # exact midpoints between neighbouring codes and their fp32 neighbours
    v = np.array([float(torch.tensor(c, dtype=torch.uint8).view(torch.float8_e4m3fn).float())
                  for c in range(127)])
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    m = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    return np.concatenate([a, m, -m, v.astype(np.float32)])


def test_e4m3_matches_torch_cast_after_clamp(orc):
    a = _e4m3_sweep()
    clamped = np.clip(a, -448.0, 448.0)
    want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(a), want)


def test_e4m3_saturates_and_keeps_sign(orc):
    a = np.array([449, 463.9, 464, 480, 1e30, -1e30, -0.0], np.float32)
    assert list(orc.e4m3_encode(a)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80]


# ------------------------------------------------------------------ E2M1 --

def test_e2m1_golden_points(orc):
    rows = [ln.split() for ln in read_golden("codec_points.txt") if ln.startswith("e2m1")]
    assert len(rows) >= 15
    vals = np.array([float(r[1]) for r in rows], np.float32)
    want = np.array([int(r[2], 16) for r in rows], np.uint8)
    assert np.array_equal(orc.e2m1_encode(vals), want)


def test_e2m1_monotone_and_nearest(orc):
    a = np.linspace(0, 8, 200_001, dtype=np.float32)
    c = orc.e2m1_encode(a).astype(int)
    assert np.all(np.diff(c) >= 0)                     # monotone in |v|
    vals = np.array([orc.e2m1_value(i) for i in range(8)])
    err = np.abs(vals[c] - a.astype(np.float64))
    # never farther than half the local gap, except past the saturation point
    gaps = np.array([0.5, 0.5, 0.5, 0.5, 1, 1, 2, 2])
    inside = a <= 6
    assert np.all(err[inside] <= gaps[c[inside]] / 2 + 1e-12)
    # the negative side mirrors the positive side with the sign bit set
    assert np.array_equal(orc.e2m1_encode(-a[1:]), c[1:] | 8)
