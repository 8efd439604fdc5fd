"""CPU model of how the tiled plan-and-dispatch launch places a pair.

In tiled mode the counting launch leaves one histogram per count tile of
whole tokens in the workspace; the launch that finishes the plan takes, for
a pair (t, j) of expert e in tile c: the padded exclusive cumsum of the
experts' totals (summed over all tile histograms), plus e's counts in the
tiles before c, plus e's pairs of tile c ahead of (t, j).  This model
restates that arithmetic with numpy.

- With the histograms of the IDs themselves it gives the oracle's slots
  (so the arithmetic is the plan), for several shapes and pad multiples.
- With histograms that do not count these IDs -- zeros, another routing's,
  negative or huge values, as a workspace changed between the two launches
  would hold -- some pairs get a rank at or past their expert's count, and
  some rows fall outside [0, R_max).  Those are the stores the kernel now
  refuses (slot -1, MOE_STATUS_BAD_PLAN); before that check they were made.
"""
import numpy as np
import pytest

from combine_topk_ids_amd.workloads import random_routing

TILE_PAIRS = 2048  # pairs per count tile, whole tokens


def tile_histograms(ids, e):
    n, k = ids.shape
    tt = max(1, TILE_PAIRS // k)
    nt = max(1, -(-n // tt))
    hist = np.zeros((nt, e), np.int64)
    for c in range(nt):
        v = ids[c * tt:(c + 1) * tt].ravel()
        v = v[(v >= 0) & (v < e)]
        hist[c] = np.bincount(v, minlength=e)
    return hist, tt


def model_slots(ids, e, a, hist, tt):
    """(row of every pair or -1, rank of every pair in its expert, totals,
    padded offsets), as the tiled launch computes them from `hist`."""
    n, k = ids.shape
    tot = hist.sum(axis=0)
    pad = np.where(a == 1, tot, -(-tot // a) * a)
    off = np.concatenate([[0], np.cumsum(pad)])
    row = np.full((n, k), -1, np.int64)
    rank = np.full((n, k), -1, np.int64)
    for c in range(hist.shape[0]):
        seen = hist[:c].sum(axis=0)
        for t in range(c * tt, min(n, (c + 1) * tt)):
            for j in range(k):
                x = ids[t, j]
                if x < 0 or x >= e:
                    continue
                rank[t, j] = seen[x]
                row[t, j] = off[x] + seen[x]
                seen[x] += 1
    return row, rank, tot, off


def oracle_like_slots(ids, e, a):
    """Stable counting sort: the plan's slot definition written directly."""
    n, k = ids.shape
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < e)
    cnt = np.bincount(flat[valid], minlength=e)
    off = np.concatenate([[0], np.cumsum(-(-cnt // a) * a)])
    order = np.argsort(np.where(valid, flat, e), kind="stable")
    slot = np.full(n * k, -1, np.int64)
    pos = off[:e].copy()
    for p in order:
        if not valid[p]:
            continue
        slot[p] = pos[flat[p]]
        pos[flat[p]] += 1
    return slot.reshape(n, k)


@pytest.mark.parametrize("n,e,k,a,masked", [(3000, 16, 4, 8, 0.05), (4096, 64, 6, 128, 0.0),
                                            (1025, 100, 3, 1, 0.2), (700, 8, 8, 3, 0.0)])
def test_true_histograms_give_the_plan(n, e, k, a, masked):
    ids, _ = random_routing(np.random.default_rng(n + e), n, e, k, masked_frac=masked)
    hist, tt = tile_histograms(ids, e)
    row, rank, tot, _ = model_slots(ids, e, a, hist, tt)
    assert np.array_equal(row, oracle_like_slots(ids, e, a))
    live = row >= 0
    assert np.all(rank[live] < tot[ids[live]])   # the check never fires
    r_max = n * k + e * (a - 1)
    assert row.max() < r_max


def test_mismatched_histograms_leave_the_expert_and_the_buffer():
    n, e, k, a = 3000, 16, 4, 8
    rng = np.random.default_rng(31)
    ids, _ = random_routing(rng, n, e, k, masked_frac=0.05)
    hist, tt = tile_histograms(ids, e)
    r_max = n * k + e * (a - 1)
    other, _ = random_routing(np.random.default_rng(32), n, e, k)
    stale, _ = tile_histograms(other, e)
    cases = {
        "zeros": np.zeros_like(hist),
        "stale": stale,
        "negative": np.full_like(hist, -5),
        "huge": np.full_like(hist, 1 << 29),
    }
    for name, h in cases.items():
        row, rank, tot, off = model_slots(ids, e, a, h, tt)
        live = ids >= 0
        past_expert = live & (rank >= tot[np.where(live, ids, 0)])
        outside = live & ((row < 0) | (row >= r_max))
        assert (past_expert | outside).any(), name  # BAD_PLAN is raised
        if name in ("zeros", "stale", "negative"):
            assert past_expert.any(), name
        if name in ("negative", "huge"):
            assert outside.any(), name        # unbounded stores would leave the buffer
        # every pair the kernel keeps (rank below its expert's count, row
        # inside the buffer) stays inside [0, R_max)
        kept = live & ~past_expert & ~outside
        assert np.all((row[kept] >= 0) & (row[kept] < r_max)), name
