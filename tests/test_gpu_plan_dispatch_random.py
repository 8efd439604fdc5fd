"""Seeded random problems through moe_plan_and_dispatch, across its three
modes (one launch, tiled, separate), every format, gates, padding, masking
and zero tails: every plan array, the status word and every packed row
against the CPU oracle, and byte for byte against the two-call path and the
two halves (check_pd).  Shapes are drawn so that each mode gets cases."""
import numpy as np
import pytest
import torch

from combine_topk_ids_amd.workloads import random_bf16, random_routing
from gpu_helpers import say
from test_gpu_plan_dispatch import check_pd

pytestmark = pytest.mark.gpu

N_CASES = 72


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def draw(idx):
    """(n, h, e, k, ep, a, fmt, masked, gated, gs, zero_tail) for case idx."""
    rng = np.random.default_rng(9000 + idx)
    fmt = ["bf16", "fp8", "mxfp4", "nvfp4"][idx % 4]
    e = int(rng.choice([1, 3, 8, 12, 16, 64, 100, 128, 256, 1024]))
    k = int(rng.integers(1, min(e, 16) + 1))
    ep = int(rng.choice([d for d in (1, 2, 3, 4, 5, 8, 16, 32, 64) if e % d == 0]))
    a = int(rng.choice([1, 1, 2, 3, 16, 128]))
    # pairs from one to about 40,000: one launch, tiled and separate
    pairs = int(rng.choice([rng.integers(1, 2049), rng.integers(2049, 20000),
                            rng.integers(20000, 40000)]))
    if idx % 6 == 5:  # many experts and pairs: past the tiled histogram limit
        e = int(rng.choice([256, 1024]))
        k = int(rng.integers(1, 17))
        ep = int(rng.choice([1, 4, 32]))
        pairs = int(rng.integers(20000, 40000))
    if idx >= 36 and idx % 3 == 1:  # expert counts that are not powers of two, past 256
        e = [257, 260, 300, 384, 500, 640, 768, 1000][idx % 8]
        k = min(k, e)
        ep = [d for d in (1, 2, 4, 5, 10, 20) if e % d == 0][-1]
    n = max(1, pairs // k)
    unit = {"bf16": 8, "fp8": 128, "mxfp4": 32, "nvfp4": 32}[fmt]
    h = unit * int(rng.integers(1, max(2, 1536 // unit) + 1))
    h = min(h, max(unit, (1 << 21) // n // unit * unit))  # keeps N*H <= 2M values
    masked = float(rng.choice([0.0, 0.05, 0.3]))
    gated = fmt != "nvfp4" and bool(rng.integers(0, 2))
    gs = float(rng.choice([0.5, 3.0, 336.0])) if fmt == "nvfp4" else None
    zero_tail = bool(rng.integers(0, 2))
    return n, h, e, k, ep, a, fmt, masked, gated, gs, zero_tail


def test_random_cases_cover_every_mode(moe):
    modes = set()
    counted = set()  # one launch without padding: rows by counting keys, by key registers
    for idx in range(N_CASES):
        n, h, e, k, ep, a, fmt, *_ = draw(idx)
        mode = moe.moe_plan_and_dispatch_mode(moe.problem(n, h, k, e, ep, pad_multiple=a, fmt=fmt))
        modes.add(mode)
        if mode == moe.PD_ONE_LAUNCH and a == 1:
            counted.add(1 if n * k <= 256 else 4 if n * k <= 1024 else 8)
    assert modes == {moe.PD_ONE_LAUNCH, moe.PD_TILED, moe.PD_SEPARATE}
    assert counted == {1, 4, 8}


@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_plan_and_dispatch(moe, idx):
    n, h, e, k, ep, a, fmt, masked, gated, gs, zero_tail = draw(idx)
    p = moe.problem(n, h, k, e, ep, pad_multiple=a, fmt=fmt)
    say(f"[random plan+dispatch {idx}] N={n} H={h} E={e} k={k} EP={ep} A={a} {fmt} "
        f"masked={masked} gated={gated} gs={gs} zero_tail={zero_tail} "
        f"mode={moe.moe_plan_and_dispatch_mode(p)}")
    rng = np.random.default_rng(19000 + idx)
    ids, wts = random_routing(rng, n, e, k, masked_frac=masked)
    x = random_bf16(rng, (n, h), scale=float(rng.choice([1e-2, 1.0, 30.0])))
    check_pd(moe, ids=ids, hidden=x, e=e, ep=ep, a=a, fmt=fmt,
             gates=wts if gated else None, gs=gs, zero_tail=zero_tail)
