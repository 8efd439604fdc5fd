"""Pins of the oracle's fixed-capacity layout (capacity factor, dropping).

Pins: a hand-worked example (tests/golden/capacity_examples.txt); the
capacity formula on exact and rounded cases; the slot rule restated on top of
the (separately pinned) single-buffer plan -- a pair's rank inside its expert
is its slot minus the expert's offset there, and it is kept exactly when that
rank is below cap; invariants (kept = min(count, cap) per expert, DROPPED
exactly when some expert is over capacity, packed_src inverts the slots and
marks unused rows); gather-form dispatch and combine drop exactly the pairs
the plan drops.  No GPU.
"""
import numpy as np
import pytest

from conftest import read_golden
from combine_topk_ids_amd.workloads import random_bf16, random_routing

DROPPED, CAP = 16, 4
BIG = 1 << 40


def golden():
    ex, cur = {}, None
    for ln in read_golden("capacity_examples.txt"):
        f = ln.split()
        if f[0] == "begin":
            cur = ex.setdefault(f[1], {})
        elif f[0] == "end":
            cur = None
        else:
            cur[f[0]] = [int(v) for v in f[1:]]
    return ex


def test_capacity_golden(orc):
    g = golden()["example1"]
    n, k, e, ep, cap, h, c = (g[x][0] for x in ("N", "k", "E", "EP", "cap", "H", "C"))
    ids = np.array(g["ids"], np.int32).reshape(n, k)
    p = orc.capacity_plan(ids, e, ep, cap, c, h)
    for key in ("expert_counts", "expert_offsets", "dest_counts", "rank_table", "slot",
                "packed_src"):
        assert p[key].reshape(-1).tolist() == g[key], key
    assert p["status"] == g["status"][0]


@pytest.mark.parametrize("n,k,e,cf,cap", [(4096, 6, 64, 1.0, 384), (4096, 6, 64, 1.25, 480),
                                          (10, 3, 4, 1.0, 8), (10, 3, 4, 0.5, 4),
                                          (7, 2, 5, 2.0, 6), (100, 1, 1, 0.0, 0),
                                          (1, 1, 3, 1.0, 1)])
def test_capacity_formula(orc, n, k, e, cf, cap):
    """ceil(cf N k / E): 4096*6/64 = 384 exactly, x1.25 = 480; 30/4 = 7.5 -> 8;
    3.75 -> 4; 2*14/5 = 5.6 -> 6; 0 -> 0; 1/3 -> 1."""
    assert orc.expert_capacity(n, k, e, cf) == cap


def check_capacity(orc, ids, e, ep, cap, rcap, h):
    n, k = ids.shape
    l = e // ep
    p = orc.capacity_plan(ids, e, ep, cap, rcap, h)
    base = orc.plan(ids, e, ep, 1, BIG, h)           # the pinned single-buffer plan
    valid = base["slot"] >= 0
    eid = np.where(valid, ids, 0)
    rank = np.where(valid, base["slot"] - base["expert_offsets"][eid], -1)
    want = np.where(valid & (rank < cap), eid * cap + rank, -1)
    assert np.array_equal(p["slot"], want)
    cnt = p["expert_counts"]
    assert np.array_equal(cnt, base["expert_counts"])
    kept = np.minimum(cnt, cap)
    assert np.array_equal(p["expert_offsets"], np.arange(e + 1) * cap)
    assert np.array_equal(p["dest_counts"], kept.reshape(ep, l).sum(1))
    t = p["rank_table"].astype(np.int64)
    assert np.array_equal(t[0], kept.reshape(ep, l).sum(1) * h)
    assert np.array_equal(t[1], np.concatenate([[0], np.cumsum(t[0])[:-1]]))
    assert np.all(t[2] == l * cap * h)
    assert np.array_equal(t[3], np.arange(ep) * l * cap * h)
    assert bool(p["status"] & DROPPED) == bool(np.any(cnt > cap))
    assert bool(p["status"] & CAP) == bool(np.any(kept.reshape(ep, l).sum(1) > rcap))
    assert (p["status"] & 3) == base["status"] & 3
    src = p["packed_src"].reshape(e, cap) if cap else np.zeros((e, 0), np.int32)
    for x in range(e):
        assert np.all(src[x, :kept[x]] >= 0) and np.all(src[x, kept[x]:] == -1)
    live = p["slot"] >= 0
    tok = np.broadcast_to(np.arange(n)[:, None], (n, k))
    assert np.array_equal(p["packed_src"][p["slot"][live]], tok[live])
    return p


@pytest.mark.parametrize("seed", range(8))
def test_capacity_random(orc, seed):
    rng = np.random.default_rng(200 + seed)
    e = int(rng.choice([1, 4, 8, 16, 64]))
    ep = int(rng.choice([d for d in (1, 2, 4, 8) if e % d == 0]))
    k = int(rng.integers(1, min(e, 8) + 1))
    n = int(rng.integers(1, 600))
    ids, _ = random_routing(rng, n, e, k, masked_frac=float(rng.choice([0.0, 0.2])))
    cf = float(rng.choice([0.0, 0.3, 0.8, 1.0, 1.5, 4.0]))
    cap = orc.expert_capacity(n, k, e, cf)
    check_capacity(orc, ids, e, ep, cap, int(rng.integers(0, n * k + 1)), 64)


def test_capacity_with_faults(orc):
    rng = np.random.default_rng(9)
    n, e, k = 200, 8, 3
    ids, _ = random_routing(rng, n, e, k)
    ids[3, 1] = ids[3, 0]
    ids[7, 2] = 99
    p = check_capacity(orc, ids, e, 2, 40, 1 << 20, 16)
    assert p["status"] & 3 == 3


def test_capacity_dispatch_and_combine_drop_exactly(orc):
    """Identity experts: tokens with no dropped pair come back bit-exactly;
    the others come back as (sum of their kept gates) * x."""
    rng = np.random.default_rng(10)
    n, e, k, h = 400, 8, 2, 64
    ids, w = random_routing(rng, n, e, k)
    x = random_bf16(rng, (n, h))
    cap = orc.expert_capacity(n, k, e, 0.8)
    p = orc.capacity_plan(ids, e, 2, cap, 1 << 20, h)
    assert p["status"] & DROPPED
    pay, _ = orc.dispatch("bf16", x, p)
    out = orc.combine(p["slot"], w, pay)
    full = np.all(p["slot"] >= 0, axis=1)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    of = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    negz = x == 0x8000
    assert np.array_equal(out[full & ~negz.any(1)], x[full & ~negz.any(1)])
    kw = np.where(p["slot"] >= 0, w, 0).astype(np.float64).sum(1, keepdims=True)
    assert np.all(np.abs(of - kw * xf) <= 2.0 ** -7 * np.abs(kw * xf) + 1e-30)
    # unused rows of every expert are zero bytes
    assert np.all(pay[p["packed_src"] < 0] == 0)
