"""GPU parity of the fixed per-expert capacity layout (through the C ABI)
against the CPU oracle.

Bar: every plan array bit-exact (dropped pairs, DROPPED and CAPACITY bits
included); every packed row (kept rows and the zero rows of underfull
experts) bit-exact; combine within one bf16 ulp.  Inputs come from the
seeded generators only; expected values only from ``oracle``.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import (WORKLOADS, make_inputs, random_bf16,
                                            random_routing)
from gpu_helpers import (SENTINEL, assert_combine_close, assert_rows_are_tokens, say,
                         to_dev_bf16, u16)

pytestmark = pytest.mark.gpu

PLAN_KEYS = ("expert_counts", "expert_offsets", "dest_counts", "rank_table", "slot",
             "packed_src")


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def run_capacity(moe, *, ids, weights, hidden, e, ep, fmt, cap, rcap, expert_out=None,
                 halves=False):
    """halves: the plan and dispatch as moe_plan_and_dispatch_begin + _end
    (the calls bench.py times) instead of moe_dispatch_plan + moe_dispatch."""
    n, k = ids.shape
    h = hidden.shape[1]
    p = moe.problem(n, h, k, e, ep, recv_capacity=rcap, fmt=fmt, expert_capacity=cap)
    plan = moe.alloc_plan(p)
    for f in PLAN_KEYS + ("status",):
        getattr(plan, f).fill_(-7)
    payload, scales = moe.alloc_payload(p)
    payload.view(torch.uint8).fill_(SENTINEL)
    if scales is not None:
        scales.view(torch.uint8).fill_(SENTINEL)
    out = torch.full((n, h), 7.0, dtype=torch.bfloat16, device="cuda")
    ids_d, x_d = torch.from_numpy(ids).cuda(), to_dev_bf16(hidden)
    if halves:
        moe.moe_plan_and_dispatch_begin(p, ids_d, plan)
        moe.moe_plan_and_dispatch_end(p, ids_d, plan, x_d, payload, scales)
    else:
        moe.moe_dispatch_plan(p, ids_d, plan)
        moe.moe_dispatch(p, plan, x_d, payload, scales)
    y = payload if expert_out is None else to_dev_bf16(expert_out)
    moe.moe_combine(p, plan, y, torch.from_numpy(weights).cuda(), out)
    torch.cuda.synchronize()
    got = {f: getattr(plan, f).cpu().numpy() for f in PLAN_KEYS}
    got["rank_table"] = got["rank_table"].view(np.uint32)
    got["packed_src"] = got["packed_src"][:e * cap]
    got["status"] = int(plan.status.cpu().numpy().view(np.uint32)[0])
    got["payload"] = payload.view(torch.uint8).cpu().numpy()
    got["scales"] = None if scales is None else scales.view(torch.uint8).cpu().numpy()
    got["out"] = u16(out)
    return got


def check_capacity(moe, *, ids, weights, hidden, e, ep, fmt, cf, rcap=None, expert_out=None,
                   per_token=False, halves=False):
    """per_token: the oracle encodes each token once and every packed row is
    compared with the encoding of its source token (gather form), instead
    of the oracle's whole dispatch encoding every row."""
    n, k = ids.shape
    h = hidden.shape[1]
    cap = oracle.expert_capacity(n, k, e, cf)
    assert moe.moe_expert_capacity(n, k, e, cf) == cap
    rcap = n * k if rcap is None else rcap
    got = run_capacity(moe, ids=ids, weights=weights, hidden=hidden, e=e, ep=ep, fmt=fmt,
                       cap=cap, rcap=rcap, expert_out=expert_out, halves=halves)
    pl = oracle.capacity_plan(ids, e, ep, cap, rcap, h)
    for f in PLAN_KEYS:
        assert np.array_equal(got[f], pl[f]), f
    assert got["status"] == pl["status"]
    if not per_token:
        pay, sc = oracle.dispatch(fmt, hidden, pl)
        assert np.array_equal(got["payload"], pay.view(np.uint8).reshape(pay.shape[0], -1))
        if sc is not None:
            assert np.array_equal(got["scales"], sc.view(np.uint8).reshape(sc.shape[0], -1))
        y = pay.view(np.uint16) if expert_out is None else expert_out
    else:
        enc, enc_sc = oracle.encode_rows(fmt, hidden)
        assert_rows_are_tokens(got["payload"], got["scales"], enc, enc_sc, pl["packed_src"])
        y = expert_out
    ref = oracle.combine(pl["slot"], weights, y)
    return got, pl, assert_combine_close(got["out"], ref)


@pytest.mark.parametrize("halves", [False, True], ids=["three_calls", "bench_calls"])
def test_capacity_bf16_workload(moe, halves):
    w = WORKLOADS["capacity_bf16_n4096"]
    say(f"[capacity parity] {w.name}: {w.describe()}; halves={halves}")
    inp = make_inputs(w, seed=0)
    got, pl, nonexact = check_capacity(moe, ids=inp["ids"], weights=inp["weights"],
                                       hidden=inp["hidden"], e=w.e, ep=w.ep, fmt="bf16",
                                       cf=w.capacity_factor, rcap=w.capacity, halves=halves)
    assert got["status"] & 16  # factor 1.0: the busiest experts drop pairs
    assert nonexact == 0


@pytest.mark.parametrize("halves", [False, True], ids=["three_calls", "bench_calls"])
def test_capacity_fp8_workload_full(moe, halves):
    """Every plan array, every packed and scale row (kept rows against the
    oracle's encoding of their token, unused rows zero) and every combine
    output of the FP8 fixed-capacity workload at full size."""
    w = WORKLOADS["capacity_fp8_n8192"]
    say(f"[capacity parity] {w.name}: {w.describe()}; halves={halves}")
    cap = oracle.expert_capacity(w.n, w.k, w.e, w.capacity_factor)
    inp = make_inputs(w, seed=0, expert_rows=w.e * cap)
    _, _, nonexact = check_capacity(moe, ids=inp["ids"], weights=inp["weights"],
                                    hidden=inp["hidden"], e=w.e, ep=w.ep, fmt="fp8",
                                    cf=w.capacity_factor, rcap=w.capacity,
                                    expert_out=inp["expert_out"], per_token=True, halves=halves)
    assert nonexact == 0


# n, h, e, k, ep, fmt, capacity factor, masked fraction
FUZZ = [
    (1, 8, 1, 1, 1, "bf16", 1.0, 0.0),
    (777, 520, 16, 5, 4, "bf16", 0.5, 0.1),
    (2049, 384, 64, 7, 8, "fp8", 1.1, 0.05),
    (1000, 96, 1024, 16, 64, "mxfp4", 2.0, 0.2),
    (4097, 160, 12, 12, 3, "mxfp4", 0.9, 0.0),
    (600, 2112, 128, 9, 16, "bf16", 8.0, 0.3),
    (5000, 256, 256, 8, 32, "bf16", 0.01, 0.0),
    (300, 1152, 32, 2, 2, "fp8", 3.0, 0.0),
]


@pytest.mark.parametrize("halves", [False, True], ids=["three_calls", "bench_calls"])
@pytest.mark.parametrize("idx", range(len(FUZZ)),
                         ids=[f"n{c[0]}_h{c[1]}_e{c[2]}_k{c[3]}_{c[5]}_cf{c[6]}" for c in FUZZ])
def test_capacity_fuzz_shapes(moe, idx, halves):
    """Every shape through the plan and dispatch calls, and through
    moe_plan_and_dispatch's halves, which drop the pairs past the capacity in
    the launch that places them (one launch, tiled or separate by size)."""
    n, h, e, k, ep, fmt, cf, masked = FUZZ[idx]
    say(f"[capacity fuzz] N={n} H={h} E={e} k={k} EP={ep} {fmt} cf={cf} masked={masked} halves={halves}")
    rng = np.random.default_rng(700 + idx)
    ids, wts = random_routing(rng, n, e, k, masked_frac=masked)
    x = random_bf16(rng, (n, h))
    cap = oracle.expert_capacity(n, k, e, cf)
    y = None if fmt == "bf16" else random_bf16(rng, (max(e * cap, 1), h))
    check_capacity(moe, ids=ids, weights=wts, hidden=x, e=e, ep=ep, fmt=fmt, cf=cf,
                   rcap=int(rng.integers(1, n * k + 1)), expert_out=y, halves=halves)


def test_capacity_faults_and_skew(moe):
    """Repeated and out-of-range IDs, and every token on one expert."""
    rng = np.random.default_rng(8)
    n, e, k, h = 1500, 16, 4, 64
    ids, wts = random_routing(rng, n, e, k)
    ids[:, 0] = 3               # expert 3 gets every token: most are dropped
    ids[10, 1] = 3              # repeated ID
    ids[20, 2] = 40             # out of range
    x = random_bf16(rng, (n, h))
    for halves in (False, True):
        say(f"[capacity faults] skew to one expert, DUP and BAD; halves={halves}")
        got, _, _ = check_capacity(moe, ids=ids, weights=wts, hidden=x, e=e, ep=4, fmt="bf16",
                                   cf=1.0, rcap=n, halves=halves)
        assert got["status"] & (1 | 2 | 16) == (1 | 2 | 16)
    small = ids[:300]  # 1200 pairs: one launch
    for halves in (False, True):
        say(f"[capacity faults] one-launch size; halves={halves}")
        got, _, _ = check_capacity(moe, ids=small, weights=wts[:300], hidden=x[:300], e=e, ep=4,
                                   fmt="bf16", cf=1.0, rcap=300, halves=halves)
        assert got["status"] & (1 | 2 | 16) == (1 | 2 | 16)
