"""Pins of the oracle's NVFP4 encoder (E2M1 codes, E4M3 scale per 16
values, fp32 global encode scale).

Pins: hand-worked blocks (tests/golden/block_examples.txt, nvfp4_*) with
rounding ties, signed zero, scale rounding and code saturation; exact
power-of-two invariance (scaling gs by 2^m scales every stored scale by 2^m
and leaves every code unchanged, binary scaling being exact); the decoded
row lies within one scale unit of x; the block maximum takes code 6 whenever
the scale is a normal E4M3 value; scales are E4M3 of fl32(amax/6 * gs) as
torch's float8_e4m3fn cast rounds it; gather-form dispatch rows are the
encoded source rows and unused rows are zero.  No GPU.
"""
import numpy as np
import pytest
import torch

from conftest import read_golden
from combine_topk_ids_amd.workloads import random_bf16, random_routing

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def golden():
    ex, cur = {}, None
    for ln in read_golden("block_examples.txt"):
        f = ln.split()
        if f[0] == "begin":
            cur = ex.setdefault(f[1], {})
        elif f[0] == "end":
            cur = None
        elif cur is not None:
            cur[f[0]] = f[1:]
    return ex


def e4m3_values(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def decode(pay, sc, gs):
    lo, hi = pay & 0xF, pay >> 4
    codes = np.empty((pay.shape[0], pay.shape[1] * 2), np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    mag = E2M1[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return mag * np.repeat(e4m3_values(sc), 16, axis=1) / gs, codes


@pytest.mark.parametrize("name", ["nvfp4_1", "nvfp4_2", "nvfp4_3"])
def test_nvfp4_golden(orc, name):
    g = golden()[name]
    x = np.array([int(v, 16) for v in g["x"]], np.uint16).reshape(1, -1)
    pay, sc = orc.encode_rows_nvfp4(x, float(g["gs"][0]))
    assert pay[0].tolist() == [int(v, 16) for v in g["payload"]]
    assert sc[0].tolist() == [int(v, 16) for v in g["scales"]]


def test_power_of_two_global_scale(orc):
    rng = np.random.default_rng(1)
    x = random_bf16(rng, (64, 256))
    base_p, base_s = orc.encode_rows_nvfp4(x, 1.0)
    for m in (-3, -1, 2, 5):
        p, s = orc.encode_rows_nvfp4(x, 2.0 ** m)
        # normal E4M3 scales stay normal and unsaturated at these m
        ok = (e4m3_values(base_s) >= 2.0 ** -6 * 2 ** max(0, -m)) & \
             (e4m3_values(base_s) * 2.0 ** m <= 448)
        assert np.array_equal(e4m3_values(s)[ok], e4m3_values(base_s)[ok] * 2.0 ** m)
        rows_ok = np.repeat(ok, 8, axis=1)
        assert np.array_equal(p[rows_ok], base_p[rows_ok])


@pytest.mark.parametrize("gs", [1.0, 0.37, 250.0, 3.0e-4])
def test_decoded_within_one_scale_unit(orc, gs):
    rng = np.random.default_rng(2)
    x = random_bf16(rng, (80, 512), scale=float(rng.choice([0.01, 1.0, 30.0])))
    pay, sc = orc.encode_rows_nvfp4(x, gs)
    deq, codes = decode(pay, sc, gs)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    unit = np.repeat(e4m3_values(sc), 16, axis=1) / gs
    # For a normal, unsaturated scale: E2M1 gaps are at most 2 units (4 -> 6)
    # and saturation past 6 costs below 6 * 2^-4 units, because a normal
    # E4M3 scale is within 2^-4 of amax/6 * gs.  Subnormal scales (gs too
    # small for the block) and scales saturated at 448 (gs too large) have no
    # such bound, as in any saturating format.
    sv = e4m3_values(sc)
    nz = np.repeat((sv >= 2.0 ** -6) & (sv < 448), 16, axis=1)
    assert np.all(np.abs(deq - xf)[nz] <= unit[nz] * (1 + 2.0 ** -20))
    # the scale is E4M3 of fl32(amax / 6 * gs), as torch rounds it
    amax = np.abs(xf.reshape(80, 32, 16)).max(axis=2).astype(np.float32)
    want = (amax / np.float32(6.0)).astype(np.float32) * np.float32(gs)
    want = torch.from_numpy(np.minimum(want, 448).astype(np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(sc, want)
    # the block maximum takes code 6 (magnitude code 7) when its scale is a
    # normal E4M3 value below saturation
    normal = (e4m3_values(sc) >= 2.0 ** -6) & (e4m3_values(sc) < 448)
    blockmax = np.abs(codes & 7).reshape(80, 32, 16).max(axis=2)
    assert np.all(blockmax[normal] == 7)


def test_zero_and_tiny_blocks(orc):
    x = np.zeros((2, 32), np.uint16)
    x[1, :16] = 0x0001          # smallest bf16 subnormal: the scale underflows to 0
    x[1, 16] = 0x8000           # -0 in an otherwise zero block
    pay, sc = orc.encode_rows_nvfp4(x, 1.0)
    assert np.all(pay == 0) and np.all(sc == 0)


def test_nvfp4_dispatch_gather(orc):
    rng = np.random.default_rng(3)
    n, e, k, h = 100, 8, 2, 64
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (n, h))
    pl = orc.plan(ids, e, 2, 4, n * k, h)
    pay, sc = orc.dispatch_nvfp4(x, pl, 0.5)
    enc_p, enc_s = orc.encode_rows_nvfp4(x, 0.5)
    src = pl["packed_src"]
    live = src >= 0
    assert np.array_equal(pay[live], enc_p[src[live]]) and np.array_equal(sc[live], enc_s[src[live]])
    assert np.all(pay[~live] == 0) and np.all(sc[~live] == 0)
