"""Pins of the oracle's gated dispatch, unweighted combine and routing-map
conversion.

Pins: hand-worked examples (tests/golden/gated_examples.txt); a gate of 1
reduces to the ungated dispatch, and a gate 2^j leaves FP8 and MX codes
unchanged while scaling the scale exactly (both follow from exact power-of-two
scaling in binary floating point); bf16 gated rows equal torch's cast of the
fp32 product; dequantised gated rows stay within each format's error bound of
w * x; the unweighted combine equals a float32 running sum in j order cast by
torch; the gated identity round trip stays within its derived bound; the
routing map conversion equals numpy's nonzero per row, inverts the multihot
built from top-k IDs, and flags exactly the rows with more than k experts.
No GPU.
"""
import numpy as np
import pytest
import torch

from conftest import read_golden
from combine_topk_ids_amd.workloads import random_bf16, random_routing

MAP_OVERFLOW = 8


def golden():
    ex, cur = {}, None
    for ln in read_golden("gated_examples.txt"):
        f = ln.split()
        if f[0] == "begin":
            cur = ex.setdefault(f[1], {})
        elif f[0] == "end":
            cur = None
        else:
            cur[f[0]] = f[1:]
    return ex


def bf16_to_f32(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def one_row_plan(n, k):
    """Every pair (t, j) to its own row t*k + j (no pad, no tail)."""
    slot = np.arange(n * k, dtype=np.int32).reshape(n, k)
    return dict(slot=slot, r_max=n * k, r_used=n * k)


def test_gated_bf16_golden(orc):
    g = golden()["gated_bf16"]
    x = np.array([int(v, 16) for v in g["x"]], np.uint16).reshape(1, -1)
    w = np.array([[float(g["w"][0])]], np.float32)
    pay, _ = orc.dispatch_gated("bf16", x, one_row_plan(1, 1), w)
    assert pay[0].tolist() == [int(v, 16) for v in g["out"]]


def test_routing_map_golden(orc):
    g = golden()["map"]
    n, e, k = (int(g[c][0]) for c in ("N", "E", "k"))
    m = np.array([int(v) for v in g["map"]], np.uint8).reshape(n, e)
    probs = ((10 * np.arange(n)[:, None] + np.arange(e)[None, :] + 1) / 64).astype(np.float32)
    ids, w, st = orc.routing_map_to_topk(m, probs, k)
    assert ids.reshape(-1).tolist() == [int(v) for v in g["ids"]]
    assert (w.reshape(-1) * 64).tolist() == [float(v) for v in g["w64"]]
    assert st == int(g["status"][0])


@pytest.mark.parametrize("fmt,h", [("bf16", 264), ("fp8", 384), ("mxfp4", 160)])
def test_gate_of_one_is_the_plain_dispatch(orc, fmt, h):
    rng = np.random.default_rng(1)
    n, e, k = 50, 8, 3
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (n, h), scale=3.0)
    pl = orc.plan(ids, e, 2, 4, n * k, h)
    ones = np.ones((n, k), np.float32)
    a_pay, a_sc = orc.dispatch_gated(fmt, x, pl, ones)
    b_pay, b_sc = orc.dispatch(fmt, x, pl)
    assert np.array_equal(a_pay, b_pay)
    if a_sc is not None:
        assert np.array_equal(a_sc, b_sc)


@pytest.mark.parametrize("fmt,h", [("bf16", 128), ("fp8", 256), ("mxfp4", 128)])
def test_power_of_two_gates_scale_exactly(orc, fmt, h):
    """w = 2^j: fl32(w*x) = 2^j x exactly, so FP8 and MX codes equal those of
    x, the FP8 scale is 2^j s and the E8M0 byte moves by j (no under- or
    overflow at these sizes)."""
    rng = np.random.default_rng(2)
    n, k = 40, 2
    x = random_bf16(rng, (n, h))
    j = rng.integers(-6, 7, size=(n, k))
    w = np.ldexp(np.ones((n, k), np.float32), j).astype(np.float32)
    pl = one_row_plan(n, k)
    g_pay, g_sc = orc.dispatch_gated(fmt, x, pl, w)
    p_pay, p_sc = orc.encode_rows(fmt, x)
    jj = j.reshape(-1)
    for r in range(n * k):
        t = r // k
        if fmt == "bf16":
            assert np.array_equal(bf16_to_f32(g_pay[r]), np.ldexp(bf16_to_f32(x[t]), jj[r]))
        elif fmt == "fp8":
            assert np.array_equal(g_pay[r], p_pay[t])
            assert np.array_equal(g_sc[r], np.ldexp(p_sc[t], jj[r]).astype(np.float32))
        else:
            assert np.array_equal(g_pay[r], p_pay[t])
            assert np.array_equal(g_sc[r].astype(int), p_sc[t].astype(int) + jj[r])


def test_gated_bf16_is_the_cast_of_the_fp32_product(orc):
    rng = np.random.default_rng(3)
    n, k, h = 64, 4, 136
    x = random_bf16(rng, (n, h), scale=10.0)
    w = rng.random((n, k)).astype(np.float32)
    pay, _ = orc.dispatch_gated("bf16", x, one_row_plan(n, k), w)
    v = w.reshape(n, k, 1) * bf16_to_f32(x).reshape(n, 1, h)  # float32 products
    assert np.array_equal(pay, torch_bf16(v.reshape(n * k, h)))


@pytest.mark.parametrize("fmt,h", [("fp8", 512), ("mxfp4", 256)])
def test_gated_rows_within_format_bounds(orc, fmt, h):
    rng = np.random.default_rng(4)
    n, k = 60, 3
    x = random_bf16(rng, (n, h), scale=2.0)
    w = (rng.random((n, k)) + 0.01).astype(np.float32)
    pay, sc = orc.dispatch_gated(fmt, x, one_row_plan(n, k), w)
    v = (w.reshape(n, k, 1) * bf16_to_f32(x).reshape(n, 1, h)).reshape(n * k, h).astype(np.float64)
    if fmt == "fp8":
        table = np.array([(-1.0 if c & 0x80 else 1.0) * orc.e4m3_value(c & 0x7F)
                          for c in range(256)])
        deq = table[pay] * np.repeat(sc.astype(np.float64), 128, axis=1)
        s = np.repeat(sc.astype(np.float64), 128, axis=1)
        # E4M3: half an ulp is 2^-4 relative (normals), 2^-10 absolute in units
        # of s (subnormals), plus the fp32 rounding of v / s
        bound = 2.0 ** -4 * np.abs(v) + 2.0 ** -10 * s + 2.0 ** -20 * np.abs(v)
    else:
        table = np.array([(-1.0 if c & 8 else 1.0) * orc.e2m1_value(c & 7) for c in range(16)])
        lo, hi = pay & 0xF, pay >> 4
        codes = np.empty((n * k, h), np.int64)
        codes[:, 0::2], codes[:, 1::2] = lo, hi
        scale = np.ldexp(1.0, sc.astype(np.int64) - 127)
        deq = table[codes] * np.repeat(scale, 32, axis=1)
        # E2M1 in units of 2^X: steps of 1/2 below 2, 1 in [2, 4), 2 in
        # [4, 6]; the block maximum is below 8 (X = floor(log2 amax) - 2), so
        # rounding or saturating at 6 moves a value by at most 2 * 2^X / 2
        # in range and by less than 2 * 2^X past 6
        bound = 2.0 * np.repeat(scale, 32, axis=1)
    assert np.all(np.abs(deq - v) <= bound)


def test_unweighted_combine_is_a_float32_running_sum(orc):
    rng = np.random.default_rng(5)
    n, k, h, rows = 80, 5, 72, 300
    y = random_bf16(rng, (rows, h), scale=4.0)
    slot = rng.integers(-1, rows, size=(n, k)).astype(np.int32)
    out = orc.combine(slot, None, y)
    assert np.array_equal(out, orc.combine(slot, np.ones((n, k), np.float32), y))
    yf = bf16_to_f32(y)
    acc = np.zeros((n, h), np.float32)
    for j in range(k):
        s = slot[:, j]
        acc = np.where((s >= 0)[:, None], acc + yf[np.maximum(s, 0)], acc).astype(np.float32)
    ref = torch_bf16(acc)
    # torch keeps -0 where the running sum is -0 only if every term was -0;
    # the oracle starts from +0, so compare on everything but exact zeros
    nz = acc != 0
    assert np.array_equal(out[nz], ref[nz]) and np.all(out[~nz] == 0)


def test_gated_identity_round_trip_bound(orc):
    """Identity experts: the unweighted combine of gated bf16 rows returns x
    up to the rounding of each copy (bf16 unit roundoff 2^-8, so at most
    2^-8 w_j |x| each, 2^-8 |x| in all since sum w_j = 1) and the final
    rounding (2^-8 of the result), plus fp32 terms."""
    rng = np.random.default_rng(6)
    n, e, k, h = 300, 16, 4, 64
    ids, w = random_routing(rng, n, e, k)
    x = random_bf16(rng, (n, h))
    pl = orc.plan(ids, e, 4, 1, n * k, h)
    pay, _ = orc.dispatch_gated("bf16", x, pl, w)
    out = orc.combine(pl["slot"], None, pay)
    xf = bf16_to_f32(x).astype(np.float64)
    of = bf16_to_f32(out).astype(np.float64)
    assert np.all(np.abs(of - xf) <= (2.0 ** -8 + 2.0 ** -8 * (1 + 2.0 ** -7) + 2.0 ** -20) * np.abs(xf))


def np_map_to_topk(m, probs, k):
    n, e = m.shape
    ids = np.full((n, k), -1, np.int32)
    w = np.zeros((n, k), np.float32)
    over = False
    for t in range(n):
        nz = np.nonzero(m[t])[0]
        over |= nz.size > k
        nz = nz[:k]
        ids[t, :nz.size] = nz
        w[t, :nz.size] = probs[t, nz] if probs is not None else 1.0
    return ids, w, over


@pytest.mark.parametrize("seed", range(5))
def test_routing_map_matches_numpy(orc, seed):
    rng = np.random.default_rng(50 + seed)
    n, e = int(rng.integers(1, 400)), int(rng.choice([2, 7, 16, 64, 256]))
    k = int(rng.integers(1, min(e, 9) + 1))
    m = (rng.random((n, e)) < rng.uniform(0.0, 0.3)).astype(np.uint8) * rng.integers(1, 256, (n, e)).astype(np.uint8)
    probs = rng.random((n, e)).astype(np.float32)
    ids, w, st = orc.routing_map_to_topk(m, probs, k)
    rids, rw, over = np_map_to_topk(m, probs, k)
    assert np.array_equal(ids, rids) and np.array_equal(w, rw)
    assert st == (MAP_OVERFLOW if over else 0)
    ids2, w2, _ = orc.routing_map_to_topk(m, None, k)
    assert np.array_equal(ids2, rids) and np.all(w2[ids2 >= 0] == 1) and np.all(w2[ids2 < 0] == 0)


def test_routing_map_inverts_the_multihot(orc):
    """Top-k IDs (unique, some masked) -> multihot map and probabilities (as
    _indices_to_multihot builds them) -> back: the same IDs in ascending
    order with their weights."""
    rng = np.random.default_rng(9)
    n, e, k = 500, 32, 6
    ids, w = random_routing(rng, n, e, k, masked_frac=0.2)
    m = np.zeros((n, e), np.uint8)
    pr = np.zeros((n, e), np.float32)
    t = np.broadcast_to(np.arange(n)[:, None], (n, k))
    ok = ids >= 0
    m[t[ok], ids[ok]] = 1
    pr[t[ok], ids[ok]] = w[ok]
    got_ids, got_w, st = orc.routing_map_to_topk(m, pr, k)
    assert st == 0
    order = np.argsort(np.where(ok, ids, e), axis=1, kind="stable")
    want_ids = np.take_along_axis(np.where(ok, ids, -1), order, axis=1)
    want_w = np.take_along_axis(np.where(ok, w, 0), order, axis=1)
    assert np.array_equal(got_ids, want_ids) and np.array_equal(got_w, want_w)
