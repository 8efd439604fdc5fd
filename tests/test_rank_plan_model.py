"""CPU model of the one-launch kernel that counts keys (no padding, A = 1).

Without padding a valid pair's packed row is the number of valid pairs ahead
of it in (expert, flat pair index) order.  The kernel packs each pair into a
21-bit key (expert << 11 | pair index; masked or invalid pairs get
0xFFFFFFFF), splits the keys over the four waves of a workgroup (ID u * 256 +
tid in register u of thread tid, so wave w holds IDs with (i mod 256) // 64
== w), counts in each quarter the keys below each own pair's key, and sums
the four counts.  This module restates that arithmetic with numpy and checks
it against the oracle's plan (the stable counting sort written out), for
random routings with masked, invalid and repeated IDs, and at the key
bounds: 2048 pairs (pair index 2047) and 1024 experts (expert 1023).
"""
import numpy as np
import pytest

import oracle
from combine_topk_ids_amd.workloads import random_routing

NO_KEY = 0xFFFFFFFF
THREADS = 256
WAVE = 64


def keys_of(ids, e):
    flat = ids.ravel().astype(np.int64)
    idx = np.arange(flat.size, dtype=np.int64)
    ok = (flat >= 0) & (flat < e)
    assert flat.size <= 2048 and e <= 1024  # 11 index bits, 10 expert bits
    return np.where(ok, (flat << 11) | idx, NO_KEY).astype(np.uint64), ok


def model_rows(ids, e):
    """Row of every pair (-1 when masked or invalid) as the kernel counts it:
    per wave quarter, the keys below the pair's key; then the sum."""
    keys, ok = keys_of(ids, e)
    n = keys.size
    i = np.arange(n)
    quarter = (i % THREADS) // WAVE
    rows = np.full(n, -1, np.int64)
    for p in np.nonzero(ok)[0]:
        counts = [int(np.sum(keys[quarter == w] < keys[p])) for w in range(THREADS // WAVE)]
        rows[p] = sum(counts)
    return rows.reshape(ids.shape)


@pytest.mark.parametrize("n,e,k,masked,seed", [(128, 256, 8, 0.0, 1), (128, 256, 8, 0.1, 2),
                                               (300, 16, 4, 0.3, 3), (256, 1024, 8, 0.05, 4),
                                               (1, 8, 8, 0.0, 5), (2048, 64, 1, 0.2, 6),
                                               (41, 7, 5, 0.0, 7)])
def test_counted_rows_are_the_plan(n, e, k, masked, seed):
    rng = np.random.default_rng(seed)
    ids, _ = random_routing(rng, n, e, k, masked_frac=masked)
    ids = ids.copy()
    if n > 2:  # an invalid ID, a below -1 ID and a repeated ID in one token
        ids[0, 0] = e
        ids[1, -1] = -3
        if k > 1:
            ids[n - 1, 1] = ids[n - 1, 0]
    pl = oracle.plan(ids, e, 1, 1, n * k, 8)
    assert np.array_equal(model_rows(ids, e), pl["slot"])


def test_keys_reach_the_bounds():
    """Pair index 2047 and expert 1023 are the largest a key holds; the
    order of keys is the order (expert, pair index)."""
    ids = np.full((256, 8), 1023, np.int32)
    ids[255, 7] = 0
    keys, ok = keys_of(ids, 1024)
    assert ok.all() and keys.max() == (1023 << 11) | 2046 and keys[-1] == 2047
    rows = model_rows(ids, 1024)
    assert rows[255, 7] == 0 and rows[0, 0] == 1 and rows[255, 6] == 2047
