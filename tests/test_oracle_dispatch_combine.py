"""Pins of the oracle's dispatch (encode + pack) and combine.

Dispatch: the oracle packs in gather form (row r takes packed_src[r]); the
tests check the scatter form P[slot[t,j]] == encode(X[t]) (an inverted map
turns the scatter into one gather, so both must agree), hand-worked FP8 and
MX blocks, the closed-form block invariants (the block maximum always lands
on the largest code), error bounds of each format, and a library (torch)
cast of whole FP8 rows.  Combine: the identity round trip (dispatch, identity
experts, weights summing to 1, combine) returns x bit-exactly; one-hot and
k = 1 weights give a pure gather; results stay within one bf16 ulp of the
exact sum.  No GPU.
"""
import struct

import numpy as np
import pytest
import torch

from conftest import read_golden
from combine_topk_ids_amd.workloads import (WORKLOADS, make_inputs, random_bf16,
                                            random_routing, to_bf16_bits)


def bf16_to_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def hex_to_f32(hx):
    return struct.unpack("<f", struct.pack("<I", int(hx, 16)))[0]


# ----------------------------------------------------------- worked blocks --

def test_fp8_blocks_golden(orc):
    for ln in read_golden("block_examples.txt"):
        f = ln.split()
        if f[0] != "fp8":
            continue
        scale = hex_to_f32(f[2])
        vi, ci = f.index("values"), f.index("codes")
        vals = [float(v) for v in f[vi + 1:ci]]
        codes = [int(c, 16) for c in f[ci + 1:]]
        x = np.zeros((1, 128), np.float32)
        x[0, :len(vals)] = vals
        pay, sc = orc.encode_rows("fp8", to_bf16_bits(x))
        assert sc[0, 0] == np.float32(scale)
        assert pay[0, :len(codes)].tolist() == codes
        assert np.all(pay[0, len(codes):] == 0)


def test_mx_block_golden(orc):
    for ln in read_golden("block_examples.txt"):
        f = ln.split()
        if f[0] != "mx":
            continue
        vi, bi = f.index("values"), f.index("bytes")
        vals = [float(v) for v in f[vi + 1:bi]]
        want = [int(b, 16) for b in f[bi + 1:]]
        x = np.zeros((1, 32), np.float32)
        x[0, :len(vals)] = vals
        pay, sc = orc.encode_rows("mxfp4", to_bf16_bits(x))
        assert sc[0, 0] == int(f[2])
        assert pay[0, :len(want)].tolist() == want
        assert np.all(pay[0, len(want):] == 0)


# --------------------------------------------------- format invariants ----

def e4m3_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_fp8_rows_against_torch_cast_and_bounds(orc):
    rng = np.random.default_rng(3)
    # mixed magnitudes: blocks at very different scales, plus zero blocks
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, size=(64, 8))).repeat(128, axis=1).astype(np.float32)
    x[5, 128:256] = 0.0
    x[6, 0:128] = -0.0
    xb = to_bf16_bits(x)
    pay, sc = orc.encode_rows("fp8", xb)
    xf = bf16_to_f64(xb).reshape(64, 8, 128)
    amax = np.abs(xf).max(axis=2)
    s = (amax.astype(np.float32) / np.float32(448.0))
    assert np.array_equal(sc, s)
    # library cast of fl32(x / s) (numpy's IEEE float32 division; torch's cast)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xf.astype(np.float32) / s[:, :, None]).astype(np.float32)
    zero = s == 0
    q[np.broadcast_to(zero[:, :, None], q.shape)] = 0.0
    want = torch.from_numpy(np.clip(q, -448, 448).reshape(64, 1024)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(pay, want)
    # I9: the block maximum lands on +-448 (0x7E / 0xFE)
    codes = pay.reshape(64, 8, 128)
    arg = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((top[~zero] & 0x7F) == 0x7E)
    # zero blocks: zero codes and a zero scale
    assert np.all(codes[zero] == 0) and np.all(sc[zero] == 0)
    # error bound: |q*s - x| <= 2^-4 |x| + 2^-10 s  (plus fp32 rounding slack)
    deq = e4m3_decode(pay).reshape(64, 8, 128) * s[:, :, None].astype(np.float64)
    bound = (2.0 ** -4) * np.abs(xf) + (2.0 ** -10) * s[:, :, None] * (1 + 2 ** -20)
    assert np.all(np.abs(deq - xf) <= bound * (1 + 2 ** -20))


def test_mx_rows_invariants_and_bounds(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 1024)).astype(np.float32)
    x *= np.exp2(rng.integers(-100, 100, size=(32, 32))).repeat(32, axis=1).astype(np.float32)
    x[3, 64:96] = 0.0
    xb = to_bf16_bits(x)
    pay, sc = orc.encode_rows("mxfp4", xb)
    xf = bf16_to_f64(xb).reshape(32, 32, 32)
    lo, hi = pay & 0xF, pay >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(32, 32, 32)
    amax = np.abs(xf).max(axis=2)
    zero = amax == 0
    assert np.all(sc[zero] == 0) and np.all(codes[zero] == 0)
    X = sc.astype(np.int64) - 127
    # the scale is 2^(floor(log2 amax) - 2), so amax * 2^-X lies in [4, 8)
    r = amax[~zero] * np.exp2(-X[~zero].astype(np.float64))
    assert np.all((r >= 4) & (r < 8))
    arg = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.isin(top[~zero] & 7, [6, 7]))
    # error bound: within half a quantum inside +-6, at most 2 quanta-units
    # (saturation of (6, 8)) otherwise, all times 2^X
    val = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    deq = np.where(codes & 8, -1.0, 1.0) * val[codes & 7] * np.exp2(X)[:, :, None]
    v = np.abs(xf) * np.exp2(-X.astype(np.float64))[:, :, None]
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    lim = np.where(v <= 6, half, v - 6) * np.exp2(X)[:, :, None]
    assert np.all(np.abs(deq - xf)[~zero] <= lim[~zero] + 1e-300)


def test_mx_subnormal_and_huge_blocks(orc):
    # bf16 subnormal block: floor(log2 amax) < -125 clamps X to -127
    tiny = np.zeros((1, 32), np.uint16)
    tiny[0, :4] = [0x0001, 0x8002, 0x0040, 0x0000]
    pay, sc = orc.encode_rows("mxfp4", tiny)
    assert sc[0, 0] == 0
    # largest bf16 values: floor(log2 amax) = 127, X = 125
    big = np.zeros((1, 32), np.uint16)
    big[0, 0] = 0x7F7F
    pay, sc = orc.encode_rows("mxfp4", big)
    assert sc[0, 0] == 125 + 127 and (pay[0, 0] & 0xF) == 7


# ------------------------------------------------------ dispatch packing --

@pytest.mark.parametrize("fmt,h", [("bf16", 256), ("fp8", 384), ("mxfp4", 96)])
def test_dispatch_scatter_equals_gather(orc, fmt, h):
    rng = np.random.default_rng(11)
    n, e, k, ep, a = 300, 16, 4, 4, 8
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (n, h))
    pl = orc.plan(ids, e, ep, a, n * 4, h)
    sentinel = 0xAB
    pdt, pshape, sdt, sshape = orc.payload_shape(fmt, pl["r_max"], h)
    pay0 = np.full(pshape, sentinel, pdt)
    sc0 = np.full(sshape, sentinel, sdt or np.uint8)
    pay, sc = orc.dispatch(fmt, x, pl, zero_tail=False, payload=pay0.copy(), scales=sc0.copy())
    enc, enc_sc = orc.encode_rows(fmt, x)
    # scatter form: row slot[t, j] holds encode(x[t])
    for t in range(n):
        for j in range(k):
            s = pl["slot"][t, j]
            if s >= 0:
                assert np.array_equal(pay[s], enc[t])
                if sc is not None:
                    assert np.array_equal(sc[s], enc_sc[t])
    # pad rows are zero bytes; tail rows untouched without the flag
    ru = pl["r_used"]
    pad = np.nonzero(pl["packed_src"][:ru] < 0)[0]
    assert pad.size > 0 and np.all(pay[pad] == 0)
    if sc is not None:
        assert np.all(sc[pad] == 0)
    assert np.all(pay[ru:] == pay0[ru:])
    pay2, _ = orc.dispatch(fmt, x, pl, zero_tail=True, payload=pay0.copy(), scales=sc0.copy())
    assert np.all(pay2[ru:] == 0) and np.array_equal(pay2[:ru], pay[:ru])


# ---------------------------------------------------------------- combine --

@pytest.mark.parametrize("name", ["tiny_bf16_n128", "uniform_bf16_n4096"])
def test_identity_round_trip_is_exact(orc, name):
    w = WORKLOADS[name]
    inp = make_inputs(w, 0)
    pl = orc.plan(inp["ids"], w.e, w.ep, w.a, w.capacity, w.h)
    pay, _ = orc.dispatch("bf16", inp["hidden"], pl)
    out = orc.combine(pl["slot"], inp["weights"], pay)
    x = inp["hidden"]
    # bit-exact, except that a -0 input comes back as +0 (the sum starts at +0)
    negz = x == 0x8000
    assert np.array_equal(out[~negz], x[~negz]) and np.all(out[negz] == 0)


def test_combine_within_one_ulp_of_exact_sum(orc):
    rng = np.random.default_rng(5)
    n, k, h, rows = 200, 6, 128, 1500
    slot = rng.integers(-1, rows, size=(n, k)).astype(np.int32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    y = random_bf16(rng, (rows, h))
    out = orc.combine(slot, w, y)
    yf = bf16_to_f64(y)
    exact = np.zeros((n, h))
    for j in range(k):
        m = slot[:, j] >= 0
        exact[m] += w[m, j, None].astype(np.float64) * yf[slot[m, j]]
    got = bf16_to_f64(out)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    # k fp32 roundings (relative 2^-24 each, on partial sums no larger than
    # sum |w y|) plus one bf16 rounding
    mag = np.zeros((n, h))
    for j in range(k):
        m = slot[:, j] >= 0
        mag[m] += np.abs(w[m, j, None].astype(np.float64) * yf[slot[m, j]])
    assert np.all(np.abs(got - exact) <= ulp + k * 2.0 ** -23 * mag)


def test_combine_gather_cases(orc):
    rng = np.random.default_rng(6)
    rows, h = 50, 64
    y = random_bf16(rng, (rows, h))
    # k = 1, w = 1: a pure gather
    slot = rng.integers(0, rows, size=(20, 1)).astype(np.int32)
    out = orc.combine(slot, np.ones((20, 1), np.float32), y)
    assert np.array_equal(out, y[slot[:, 0]])
    # one-hot weights over k = 4 return the chosen row exactly
    slot = rng.integers(0, rows, size=(20, 4)).astype(np.int32)
    pick = rng.integers(0, 4, size=20)
    w = np.zeros((20, 4), np.float32)
    w[np.arange(20), pick] = 1.0
    out = orc.combine(slot, w, y)
    assert np.array_equal(out, y[slot[np.arange(20), pick]])
    # every slot masked: +0; negative-zero products also sum to +0
    out = orc.combine(np.full((3, 2), -1, np.int32), np.ones((3, 2), np.float32), y)
    assert np.all(out == 0)
    yneg = np.full((1, h), 0x8000, np.uint16)  # -0.0
    out = orc.combine(np.zeros((2, 1), np.int32), np.ones((2, 1), np.float32), yneg)
    assert np.all(out == 0)


def test_combine_rejects_rows_it_does_not_have(orc):
    """The oracle's combine indexes y by slot; a slot past y's rows, or
    weights of another shape, is refused before the C loop runs."""
    rng = np.random.default_rng(8)
    y = random_bf16(rng, (10, 16))
    with pytest.raises(ValueError):
        orc.combine(np.array([[3, 10]], np.int32), np.ones((1, 2), np.float32), y)
    with pytest.raises(ValueError):
        orc.combine(np.array([[3, 4]], np.int32), np.ones((1, 3), np.float32), y)
    orc.combine(np.array([[3, 9]], np.int32), np.ones((1, 2), np.float32), y)  # in range


def test_dispatch_rejects_inputs_it_would_read_past(orc):
    """packed_src naming a token x does not have, a short packed_src, gates of
    another shape, or a caller payload of the wrong shape is refused before
    the C loop runs."""
    rng = np.random.default_rng(9)
    x = random_bf16(rng, (4, 16))
    pl = dict(packed_src=np.array([0, 3, -1, 4], np.int32), r_max=4, r_used=4,
              slot=np.array([[0], [1], [3], [-1]], np.int32))
    with pytest.raises(ValueError):
        orc.dispatch("bf16", x, pl)
    with pytest.raises(ValueError):
        orc.dispatch("bf16", x, dict(pl, packed_src=np.array([0, 1], np.int32)))
    with pytest.raises(ValueError):
        orc.dispatch_nvfp4(random_bf16(rng, (4, 32)), pl, 1.0)
    with pytest.raises(ValueError):
        orc.dispatch_gated("bf16", x, pl, np.ones((4, 2), np.float32))
    with pytest.raises(ValueError):
        orc.dispatch_gated("bf16", x, dict(pl, slot=np.array([[0], [1], [4], [-1]], np.int32)),
                           np.ones((4, 1), np.float32))
    ok = dict(pl, packed_src=np.array([0, 3, -1, 2], np.int32))
    with pytest.raises(ValueError):
        orc.dispatch("bf16", x, ok, payload=np.zeros((3, 16), np.uint16))
    pay, _ = orc.dispatch("bf16", x, ok)
    assert np.array_equal(pay[1], x[3]) and np.all(pay[2] == 0)
    with pytest.raises(ValueError):
        orc.routing_map_to_topk(np.ones((2, 4), np.uint8), np.ones((2, 3), np.float32), 2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_threads_do_not_change_results(orc, fmt):
    """The oracle's row loops on one thread and on several give the same bytes
    (plan, every packed and scale row, encoded rows, combine), so the timed
    all-cores baseline computes what the single-thread oracle computes."""
    rng = np.random.default_rng(900)
    n, h, e, k, ep, a = 700, 256, 32, 4, 8, 4
    ids, w = random_routing(rng, n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (n, h))
    res = []
    prev = orc.threads()
    for threads in (1, 5):
        orc.set_threads(threads)
        assert orc.threads() == threads
        pl = orc.plan(ids, e, ep, a, n * min(k, e // ep), h)
        pay, sc = orc.dispatch(fmt, x, pl)
        enc, enc_sc = orc.encode_rows(fmt, x)
        y = random_bf16(np.random.default_rng(901), (pl["r_max"], h))
        out = orc.combine(pl["slot"], w, y)
        res.append([pl["slot"], pl["packed_src"], pl["expert_offsets"], pay, enc, out]
                   + ([sc, enc_sc] if sc is not None else []))
    orc.set_threads(prev)
    for a_, b_ in zip(*res):
        assert np.array_equal(a_, b_)
