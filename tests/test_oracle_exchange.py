"""Pins of the oracle's exchange across EP simulated ranks.

Pins: hand-worked examples (tests/golden/exchange_examples.txt); the
all-to-all-v definition restated on top of the single-rank plan (each rank's
send segments, cut out by rows 0-1 of its own table and packed source by
source into C-row receive buffers); the receive order restated as a numpy
lexsort; invariants (the counts all-to-all is a transpose of the count
matrix, receive counts sum the send counts, CAPACITY exactly when a buffer is
offered more than C rows); one rank reduces to the single-buffer plan; the
identity round trip; brute force over every routing of tiny problems.  No GPU.
"""
import itertools

import numpy as np
import pytest

from conftest import read_golden
from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs, random_bf16, random_routing

BAD, DUP, CAP = 1, 2, 4
BIG = 1 << 40  # a send-side capacity no rank reaches


def parse_examples():
    ex, cur = {}, None
    for ln in read_golden("exchange_examples.txt"):
        f = ln.split()
        if f[0] == "begin":
            cur = ex.setdefault(f[1], {})
        elif f[0] == "end":
            cur = None
        else:
            cur[f[0]] = [int(v) for v in f[1:]]
    return ex


@pytest.mark.parametrize("name", ["example1", "example2"])
def test_exchange_golden(orc, name):
    g = parse_examples()[name]
    ep, e, n, k, h, c = (g[x][0] for x in ("EP", "E", "N", "k", "H", "C"))
    ids = np.array(g["ids"], np.int32).reshape(ep, n, k)
    xp = orc.exchange_plan(ids, e, c, h)
    for key in ("expert_counts", "send_counts", "recv_expert_counts", "recv_rows",
                "rank_table", "recv_slot", "recv_src", "status"):
        assert xp[key].reshape(-1).tolist() == g[key], key


def a2av_restatement(orc, ids3, e, cap, h):
    """Receive side built from the all-to-all-v definition on top of the
    single-rank plan: rank d's buffer is, source by source, the segment
    [row1[d], row1[d] + row0[d]) / H of each source's own packed buffer,
    kept up to C rows, then -1 rows.  Returns (recv_slot, recv_src,
    table rows 2-3 of every rank)."""
    ep, n, k = ids3.shape
    plans = [orc.plan(ids3[s], e, ep, 1, BIG, h) for s in range(ep)]
    recv_slot = np.full((ep, n, k), -1, np.int64)
    recv_src = np.full((ep, cap), -1, np.int64)
    rows23 = np.zeros((ep, 2, ep), np.int64)
    for d in range(ep):
        pos = 0
        for s in range(ep):
            t = plans[s]["rank_table"].astype(np.int64)
            lo, cnt = t[1, d] // h, t[0, d] // h
            rows23[d, 0, s] = t[0, d]
            rows23[d, 1, s] = pos * h
            seg_src = plans[s]["packed_src"][lo:lo + cnt]
            slot = plans[s]["slot"]
            for i in range(cnt):
                if pos + i < cap:
                    recv_src[d, pos + i] = s * n + seg_src[i]
            in_seg = (slot >= lo) & (slot < lo + cnt)
            rel = slot - lo + pos
            keep = in_seg & (rel < cap)
            recv_slot[s][keep] = d * cap + rel[keep]
            pos += cnt
    return recv_slot, recv_src, rows23


def lexsort_restatement(ids3, e, cap):
    """Receive rows as a library sort: valid pairs ordered by (destination
    rank, source rank, expert, source-local flat index)."""
    ep, n, k = ids3.shape
    l = e // ep
    s_idx, flat = np.meshgrid(np.arange(ep), np.arange(n * k), indexing="ij")
    ids = ids3.reshape(ep, n * k)
    valid = (ids >= 0) & (ids < e)
    s_v, f_v, e_v = s_idx[valid], flat[valid], ids[valid]
    d_v = e_v // l
    order = np.lexsort((f_v, e_v, s_v, d_v))
    recv_slot = np.full((ep, n * k), -1, np.int64)
    recv_src = np.full((ep, cap), -1, np.int64)
    for d in range(ep):
        sel = order[d_v[order] == d][:cap]
        recv_slot[s_v[sel], f_v[sel]] = d * cap + np.arange(sel.size)
        recv_src[d, :sel.size] = s_v[sel] * n + f_v[sel] // k
    return recv_slot.reshape(ep, n, k), recv_src


def check_exchange(orc, ids3, e, cap, h):
    ep, n, k = ids3.shape
    l = e // ep
    xp = orc.exchange_plan(ids3, e, cap, h)
    # the definition, restated twice
    rs, rsrc, rows23 = a2av_restatement(orc, ids3, e, cap, h)
    assert np.array_equal(xp["recv_slot"], rs)
    assert np.array_equal(xp["recv_src"], rsrc)
    ls, lsrc = lexsort_restatement(ids3, e, cap)
    assert np.array_equal(xp["recv_slot"], ls) and np.array_equal(xp["recv_src"], lsrc)
    t = xp["rank_table"].astype(np.int64)
    assert np.array_equal(t[:, 2:4, :], rows23)
    # the counts all-to-all is a transpose of the count matrix
    cm = xp["expert_counts"].reshape(ep, ep, l)  # [s][d][l]
    assert np.array_equal(xp["recv_expert_counts"], cm.transpose(1, 0, 2))
    assert np.array_equal(xp["send_counts"], cm.sum(2))
    assert np.array_equal(xp["recv_rows"], xp["send_counts"].sum(0))
    # each rank's send half is its own single-rank table (rows 0-1)
    for s in range(ep):
        p = orc.plan(ids3[s], e, ep, 1, BIG, h)
        assert np.array_equal(t[s, :2], p["rank_table"][:2].astype(np.int64))
        assert np.array_equal(xp["expert_counts"][s], p["expert_counts"])
        # fault bits: the sender's BAD/DUP, the receiver's CAPACITY
        assert (int(xp["status"][s]) & (BAD | DUP)) == p["status"]
    over = xp["recv_rows"] > cap
    assert np.array_equal((xp["status"] & CAP) != 0, over)
    # kept rows per buffer and the zero tail
    kept = np.minimum(xp["recv_rows"], cap)
    assert np.array_equal((xp["recv_src"] >= 0).sum(1), kept)
    for d in range(ep):
        assert np.all(xp["recv_src"][d, kept[d]:] == -1)
    # receive rows invert recv_src
    live = xp["recv_slot"] >= 0
    tok = np.broadcast_to(np.arange(ep * n).reshape(ep, n, 1), (ep, n, k))
    assert np.array_equal(xp["recv_src"].reshape(-1)[xp["recv_slot"][live]], tok[live])
    return xp


@pytest.mark.parametrize("seed", range(6))
def test_exchange_random(orc, seed):
    rng = np.random.default_rng(100 + seed)
    ep = int(rng.choice([1, 2, 3, 4, 8]))
    e = ep * int(rng.choice([1, 2, 3, 8]))
    k = int(rng.integers(1, min(e, 6) + 1))
    n = int(rng.integers(1, 300))
    ids, _ = random_routing(rng, ep * n, e, k, masked_frac=0.15)
    mean = n * k  # rows a buffer receives on average
    cap = int(rng.choice([mean // 2 + 1, mean, 2 * mean, ep * n * min(k, e // ep)]))
    check_exchange(orc, ids.reshape(ep, n, k), e, cap, 64)


def test_exchange_faults(orc):
    rng = np.random.default_rng(7)
    ep, n, k, e = 4, 50, 3, 8
    ids, _ = random_routing(rng, ep * n, e, k)
    ids[5, 1] = ids[5, 0]      # rank 0: repeated ID
    ids[n + 3, 2] = 11         # rank 1: out of range
    ids[2 * n + 4, 0] = -7     # rank 2: out of range
    xp = check_exchange(orc, ids.reshape(ep, n, k), e, 10, 32)
    assert xp["status"][0] & DUP and xp["status"][1] & BAD and xp["status"][2] & BAD
    assert np.all(xp["status"] & CAP)  # every buffer is offered far more than 10 rows


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.exchange])
def test_exchange_workloads(orc, name):
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=0, expert_rows=1) if w.experts == "random" else make_inputs(w, 0)
    ids3 = inp["ids"].reshape(w.ranks, w.n, w.k)
    xp = orc.exchange_plan(ids3, w.e, w.capacity, w.h)
    ls, lsrc = lexsort_restatement(ids3, w.e, w.capacity)
    assert np.array_equal(xp["recv_slot"], ls) and np.array_equal(xp["recv_src"], lsrc)
    # the workloads' capacities hold every row: nothing is dropped
    assert np.all(xp["status"] == 0)
    assert np.all(xp["recv_rows"] <= w.capacity)


def test_one_rank_is_the_single_buffer_plan(orc):
    rng = np.random.default_rng(3)
    n, k, e = 333, 4, 16
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.1)
    cap = n * k + 5
    xp = orc.exchange_plan(ids.reshape(1, n, k), e, cap, 128)
    p = orc.plan(ids, e, 1, 1, cap, 128)
    assert np.array_equal(xp["recv_slot"][0], p["slot"])
    ru = p["r_used"]
    assert np.array_equal(xp["recv_src"][0, :ru], p["packed_src"][:ru])
    assert np.all(xp["recv_src"][0, ru:] == -1)
    assert np.array_equal(xp["rank_table"][0, :2], p["rank_table"][:2])
    assert np.array_equal(xp["rank_table"][0, 2:], p["rank_table"][:2])


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_exchange_dispatch_is_the_a2av_of_send_buffers(orc, fmt):
    """Receive buffers equal the all-to-all-v of the ranks' own packed send
    buffers (single-rank oracle dispatch), padded with zero rows to C."""
    rng = np.random.default_rng(11)
    ep, n, k, e, h = 3, 40, 2, 6, 256
    ids, _ = random_routing(rng, ep * n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (ep * n, h))
    cap = 30
    ids3 = ids.reshape(ep, n, k)
    xp = orc.exchange_plan(ids3, e, cap, h)
    pay, sc = orc.exchange_dispatch(fmt, x, xp)
    pay = pay.reshape(ep, cap, -1)
    sc = None if sc is None else sc.reshape(ep, cap, -1)
    for d in range(ep):
        pos = 0
        for s in range(ep):
            p = orc.plan(ids3[s], e, ep, 1, BIG, h)
            spay, ssc = orc.dispatch(fmt, x[s * n:(s + 1) * n], p)
            t = p["rank_table"].astype(np.int64)
            lo, cnt = t[1, d] // h, t[0, d] // h
            take = max(0, min(cnt, cap - pos))
            assert np.array_equal(pay[d, pos:pos + take], spay[lo:lo + take])
            if sc is not None:
                assert np.array_equal(sc[d, pos:pos + take], ssc[lo:lo + take])
            pos += cnt
        tail = min(pos, cap)
        assert np.all(pay[d, tail:] == 0)
        if sc is not None:
            assert np.all(sc[d, tail:].view(np.uint8) == 0)


def test_exchange_identity_round_trip(orc):
    """Identity experts: combine(exchange dispatch(x)) returns x bit-exactly
    (a -0 comes back as +0) when no row is dropped; with drops, a token's
    output is the weighted sum of its kept rows only."""
    rng = np.random.default_rng(5)
    ep, n, k, e, h = 4, 200, 3, 8, 64
    ids, wts = random_routing(rng, ep * n, e, k)
    x = random_bf16(rng, (ep * n, h))
    for cap in (n * k * 2, n * k * 3 // 4):
        xp = orc.exchange_plan(ids.reshape(ep, n, k), e, cap, h)
        pay, _ = orc.exchange_dispatch("bf16", x, xp)
        slot = xp["recv_slot"].reshape(ep * n, k)
        out = orc.combine(slot, wts, pay)
        if np.all(xp["status"] == 0):
            negz = x == 0x8000
            assert np.array_equal(out[~negz], x[~negz]) and np.all(out[negz] == 0)
        else:
            assert np.any(slot == -1)
            wk = np.where(slot >= 0, wts, 0).astype(np.float64)
            xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            ref = wk.sum(1, keepdims=True) * xf
            got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("ep,n,e,k,cap", [(2, 1, 2, 1, 1), (2, 1, 4, 2, 2), (2, 2, 2, 1, 1),
                                          (3, 1, 3, 2, 2), (2, 2, 4, 1, 3)])
def test_exchange_brute_force_tiny(orc, ep, n, e, k, cap):
    """Every routing with unique IDs (any masking) of a tiny problem."""
    rows = [c for c in itertools.product(range(-1, e), repeat=k)
            if len([v for v in c if v >= 0]) == len({v for v in c if v >= 0})]
    for combo in itertools.product(rows, repeat=ep * n):
        ids3 = np.array(combo, np.int32).reshape(ep, n, k)
        xp = orc.exchange_plan(ids3, e, cap, 8)
        rs, rsrc, _ = a2av_restatement(orc, ids3, e, cap, 8)
        assert np.array_equal(xp["recv_slot"], rs), combo
        assert np.array_equal(xp["recv_src"], rsrc), combo
