"""Pins of the oracle's routing plan (counts, offsets, (4, EP) table, slots).

Pins: hand-worked examples (tests/golden/plan_examples.txt); a stable sort
from numpy standing in for the slot rule; invariants the pages fix (counts
sum to N*k, packed sources lie in [0, N), rank rows stay under the dropless
bound N*min(k, L), the table's displacements are the cumsum of its counts);
and brute force over every routing of tiny problems.  No GPU.
"""
import itertools

import numpy as np
import pytest

from conftest import read_golden
from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs, random_routing

BAD, DUP, CAP = 1, 2, 4


def parse_examples():
    ex, cur = {}, None
    for ln in read_golden("plan_examples.txt"):
        f = ln.split()
        if f[0] == "begin":
            cur = ex.setdefault(f[1], {})
        elif f[0] == "end":
            cur = None
        else:
            cur[f[0]] = [int(v) for v in f[1:]]
    return ex


@pytest.mark.parametrize("name", ["example1", "example2"])
def test_plan_golden(orc, name):
    g = parse_examples()[name]
    n, k, e, ep, a, h, c = (g[x][0] for x in ("N", "k", "E", "EP", "A", "H", "C"))
    ids = np.array(g["ids"], np.int32).reshape(n, k)
    p = orc.plan(ids, e, ep, a, c, h)
    assert p["expert_counts"].tolist() == g["expert_counts"]
    assert p["expert_offsets"].tolist() == g["expert_offsets"]
    assert p["dest_counts"].tolist() == g["dest_counts"]
    assert p["rank_table"].reshape(-1).tolist() == g["rank_table"]
    assert p["slot"].reshape(-1).tolist() == g["slot"]
    assert p["packed_src"].tolist() == g["packed_src"]
    assert p["status"] == g["status"][0]


def check_invariants(orc, ids, e, ep, a, cap, h, p, unique=True):
    n, k = ids.shape
    l = e // ep
    valid = (ids >= 0) & (ids < e)
    cnt, off, slot, src = p["expert_counts"], p["expert_offsets"], p["slot"], p["packed_src"]
    # I1: counts add up to the number of valid pairs (N*k when none is masked)
    assert cnt.sum() == valid.sum()
    assert np.array_equal(cnt, np.bincount(ids[valid], minlength=e))
    # I2: offsets are a cumsum of per-expert sizes that are multiples of A
    sizes = np.diff(off)
    assert off[0] == 0 and p["r_used"] == off[-1]
    assert np.all(sizes % a == 0) and np.all(sizes >= cnt) and np.all(sizes - cnt < a)
    assert p["r_used"] <= p["r_max"] == n * k + e * (a - 1)
    # I3/I4: table rows 1 and 3 are exclusive cumsums of rows 0 and 2 (elements)
    t = p["rank_table"].astype(np.int64)
    s_r = cnt.reshape(ep, l).sum(1)
    p_r = sizes.reshape(ep, l).sum(1)
    assert np.array_equal(p["dest_counts"], s_r)
    assert np.array_equal(t[0], s_r * h) and np.array_equal(t[2], p_r * h)
    assert np.array_equal(t[1], np.concatenate([[0], np.cumsum(t[0])[:-1]]))
    assert np.array_equal(t[3], np.concatenate([[0], np.cumsum(t[2])[:-1]]))
    if a == 1:
        assert np.array_equal(t[2], t[0]) and np.array_equal(t[3], t[1])
    # I5: with unique IDs no rank exceeds the dropless bound N*min(k, L)
    if unique:
        assert np.all(s_r <= n * min(k, l))
    assert ((p["status"] & CAP) != 0) == bool(np.any(s_r > cap))
    # I6: slots are injective onto live rows and invert packed_src
    live = slot[valid]
    assert np.all(slot[~valid] == -1)
    assert len(np.unique(live)) == live.size
    tok = np.broadcast_to(np.arange(n)[:, None], (n, k))
    assert np.array_equal(src[slot[valid]], tok[valid])
    # I7: every packed source lies in [0, N); all other rows are -1; each
    # token appears as often as it has valid pairs
    used = src >= 0
    assert np.all(src[used] < n) and used.sum() == valid.sum()
    assert np.array_equal(np.bincount(src[used], minlength=n), valid.sum(1))
    # each live row sits inside its expert's segment, before the pad rows
    e_of = ids[valid]
    assert np.all(live >= off[e_of]) and np.all(live < off[e_of] + cnt[e_of])


def argsort_slots(ids, e, a):
    """Slot rule restated as a library stable sort (numpy), independent of
    the oracle's per-expert walk: order valid pairs by expert with numpy's
    stable argsort; the i-th pair of expert x goes to offsets[x] + i."""
    n, k = ids.shape
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < e))[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    cnt = np.bincount(flat[valid], minlength=e)
    pad = -(-cnt // a) * a
    off = np.concatenate([[0], np.cumsum(pad)])
    first = np.concatenate([[0], np.cumsum(cnt)])
    slots = np.full(n * k, -1, np.int64)
    ex = flat[order]
    slots[order] = off[ex] + (np.arange(order.size) - first[ex])
    return slots.reshape(n, k)


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if not w.exchange])
def test_plan_workloads(orc, name):
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=0, expert_rows=1) if w.experts == "random" else make_inputs(w, 0)
    ids = inp["ids"]
    p = orc.plan(ids, w.e, w.ep, w.a, w.capacity, w.h)
    check_invariants(orc, ids, w.e, w.ep, w.a, w.capacity, w.h, p)
    assert p["status"] == 0
    assert np.array_equal(p["slot"], argsort_slots(ids, w.e, w.a))


@pytest.mark.parametrize("seed", range(6))
def test_plan_random_masked(orc, seed):
    rng = np.random.default_rng(seed)
    e = int(rng.choice([4, 8, 16, 64]))
    ep = int(rng.choice([d for d in (1, 2, 4, 8) if e % d == 0]))
    k = int(rng.integers(1, min(e, 8) + 1))
    n = int(rng.integers(1, 700))
    a = int(rng.choice([1, 2, 3, 128]))
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.2)
    h = 64
    cap = n * min(k, e // ep)
    p = orc.plan(ids, e, ep, a, cap, h)
    check_invariants(orc, ids, e, ep, a, cap, h, p)
    assert np.array_equal(p["slot"], argsort_slots(ids, e, a))


@pytest.mark.parametrize("n,e,k,ep,a", [(1, 3, 1, 1, 1), (2, 3, 2, 1, 2), (3, 3, 1, 3, 1),
                                        (2, 4, 2, 2, 3), (3, 4, 2, 2, 1), (3, 2, 2, 2, 2)])
def test_plan_brute_force_tiny(orc, n, e, k, ep, a):
    """Every routing with unique IDs (and every masking) of a tiny problem."""
    choices = [c for c in itertools.product(range(-1, e), repeat=k)
               if sum(x >= 0 for x in c) == len(set(x for x in c if x >= 0))]
    count = 0
    for combo in itertools.product(choices, repeat=n):
        ids = np.array(combo, np.int32).reshape(n, k)
        p = orc.plan(ids, e, ep, a, n * min(k, e // ep), 5)
        check_invariants(orc, ids, e, ep, a, n * min(k, e // ep), 5, p)
        assert np.array_equal(p["slot"], argsort_slots(ids, e, a))
        # inside each expert segment packed sources are non-decreasing
        off = p["expert_offsets"]
        for x in range(e):
            seg = p["packed_src"][off[x]:off[x] + p["expert_counts"][x]]
            assert np.all(np.diff(seg) >= 0)
        count += 1
    assert count == len(choices) ** n


def test_plan_empty_and_degenerate(orc):
    # N = 0: nothing routed, no rows used, pad-only buffer of E*(A-1) rows
    p = orc.plan(np.zeros((0, 2), np.int32), 4, 2, 3, 0, 8)
    assert p["r_used"] == 0 and p["r_max"] == 8 and np.all(p["packed_src"] == -1)
    assert p["rank_table"].sum() == 0 and p["status"] == 0
    # every slot masked
    p = orc.plan(np.full((5, 3), -1, np.int32), 4, 4, 1, 5, 8)
    assert p["r_used"] == 0 and np.all(p["slot"] == -1) and p["status"] == 0
    # all tokens to one expert; L = 1 so the dropless bound is N itself
    ids = np.zeros((9, 1), np.int32)
    p = orc.plan(ids, 4, 4, 1, 9, 8)
    assert p["dest_counts"].tolist() == [9, 0, 0, 0] and p["status"] == 0
    assert p["slot"].reshape(-1).tolist() == list(range(9))
    # k = E: every token goes to every expert
    ids = np.tile(np.arange(4, dtype=np.int32)[::-1], (3, 1))
    p = orc.plan(ids, 4, 2, 1, 6, 8)
    assert p["expert_counts"].tolist() == [3, 3, 3, 3]
    assert p["slot"][:, ::-1].tolist() == [[0, 3, 6, 9], [1, 4, 7, 10], [2, 5, 8, 11]]


def test_plan_fault_flags(orc):
    ids = np.array([[0, 0], [7, 1], [-3, 2]], np.int32)
    p = orc.plan(ids, 4, 2, 1, 100, 8)
    assert p["status"] == BAD | DUP
    assert p["slot"].tolist() == [[0, 1], [-1, 2], [-1, 3]]
    # capacity: 3 tokens all on rank 0 while capacity is 2
    p = orc.plan(np.array([[0], [1], [0]], np.int32), 4, 2, 1, 2, 8)
    assert p["status"] == CAP and p["dest_counts"].tolist() == [3, 0]
