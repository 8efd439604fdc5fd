"""GPU: the tiled plan-and-dispatch at two slabs per gated bf16 token, and the
bounds every kernel keeps when its plan inputs do not describe the IDs.

The second half forces the conditions from the host: between
moe_plan_and_dispatch_begin and _end the workspace (the counting kernel's
tile histograms) is overwritten with zeros, with seeded garbage and with the
histograms of another routing; slot arrays holding rows past the buffer are
handed to the dispatch and the combine.  Every kernel bounds each store by
the buffer's rows and skips what lies outside, so all of them exit normally;
the tests check that nothing is written outside [0, R_max) (guard rows
after the buffer keep their sentinel) and that MOE_STATUS_BAD_PLAN reports
the mismatch.  A proper _begin + _end afterwards is bit-exact again.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs, random_bf16, random_routing
from gpu_helpers import SENTINEL, assert_combine_close, say, to_dev_bf16, u16

pytestmark = pytest.mark.gpu

GUARD_ROWS = 64


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def test_gated_bf16_two_slabs_tiled_halves(moe):
    """Gated bf16 dispatch at the uniform shape (N = H = 4096, E = 64, k = 6,
    A = 128: two 2048-column slabs per token, 13 count tiles) through
    moe_plan_and_dispatch_begin + _end, then the unweighted combine: every
    plan array, packed row and output against the oracle."""
    w = WORKLOADS["uniform_bf16_n4096"]
    p = moe.problem(w.n, w.h, w.k, w.e, w.ep, recv_capacity=w.capacity, pad_multiple=w.a,
                    fmt="bf16", zero_tail=True)
    assert moe.moe_plan_and_dispatch_mode(p) == moe.PD_TILED
    say(f"[guards] gated bf16 tiled halves: {w.describe()}")
    inp = make_inputs(w, seed=0)
    plan = moe.alloc_plan(p)
    payload, _ = moe.alloc_payload(p)
    payload.view(torch.uint8).fill_(SENTINEL)
    ids = torch.from_numpy(inp["ids"]).cuda()
    gates = torch.from_numpy(inp["weights"]).cuda()
    x = to_dev_bf16(inp["hidden"])
    out = torch.full((w.n, w.h), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_plan_and_dispatch_begin(p, ids, plan)
    moe.moe_plan_and_dispatch_end(p, ids, plan, x, payload, None, topk_weights=gates)
    moe.moe_combine(p, plan, payload, None, out)
    torch.cuda.synchronize()
    pl = oracle.plan(inp["ids"], w.e, w.ep, w.a, w.capacity, w.h)
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])
    assert np.array_equal(plan.packed_src.cpu().numpy(), pl["packed_src"])
    assert np.array_equal(plan.expert_offsets.cpu().numpy(), pl["expert_offsets"])
    assert np.array_equal(plan.rank_table.cpu().numpy().view(np.uint32), pl["rank_table"])
    assert plan.read_status() == pl["status"] == 0
    ref_pay, _ = oracle.dispatch_gated("bf16", inp["hidden"], pl, inp["weights"], zero_tail=True)
    assert np.array_equal(u16(payload), ref_pay)
    ref_out = oracle.combine(pl["slot"], None, ref_pay)
    assert assert_combine_close(u16(out), ref_out) == 0


def _guarded(moe, p):
    """Plan buffers and a payload with GUARD_ROWS sentinel rows after R_max
    (and after packed_src): views of the first R_max rows, and the guards."""
    r_max = moe.moe_max_rows(p)
    plan = moe.alloc_plan(p)
    big_src = torch.full((r_max + GUARD_ROWS,), -77, dtype=torch.int32, device="cuda")
    plan = moe.PlanBuffers(**{**{f: getattr(plan, f) for f in
                                 ("expert_counts", "expert_offsets", "dest_counts", "rank_table",
                                  "slot", "status", "workspace")},
                              "packed_src": big_src[:r_max]})
    big_pay = torch.full((r_max + GUARD_ROWS, p.hidden), 0, dtype=torch.bfloat16, device="cuda")
    big_pay.view(torch.uint8).fill_(SENTINEL)
    return plan, big_src, big_pay, r_max


def _assert_guards(big_src, big_pay, r_max):
    assert torch.all(big_src[r_max:] == -77), "packed_src written past R_max"
    tail = big_pay[r_max:].contiguous().view(torch.uint8)
    assert torch.all(tail == SENTINEL), "payload written past R_max"


def test_tiled_end_with_a_workspace_that_does_not_match(moe):
    """_end after the workspace was overwritten: nothing lands outside the
    buffers, BAD_PLAN is set, and the pairs the histograms do not account
    for get slot -1; a proper _begin + _end restores the exact plan."""
    n, h, e, k, ep, a = 3000, 256, 16, 4, 4, 8
    rng = np.random.default_rng(31)
    ids_np, _ = random_routing(rng, n, e, k, masked_frac=0.05)
    x_np = random_bf16(rng, (n, h))
    p = moe.problem(n, h, k, e, ep, pad_multiple=a, zero_tail=True)
    assert moe.moe_plan_and_dispatch_mode(p) == moe.PD_TILED
    plan, big_src, big_pay, r_max = _guarded(moe, p)
    payload = big_pay[:r_max]
    ids = torch.from_numpy(ids_np).cuda()
    x = to_dev_bf16(x_np)
    ws = plan.workspace.view(torch.int32)
    other_ids, _ = random_routing(np.random.default_rng(32), n, e, k)
    # histograms of another routing, as a workspace reused too early would hold
    moe.moe_plan_and_dispatch_begin(p, torch.from_numpy(other_ids).cuda(), plan)
    torch.cuda.synchronize()
    stale = ws.clone()
    cases = {
        "zeros": torch.zeros_like(ws),
        "garbage": torch.from_numpy(
            np.random.default_rng(33).integers(-2**31, 2**31, ws.numel(), dtype=np.int64)
            .astype(np.int32)).cuda(),
        "large": torch.full_like(ws, 1 << 29),
        "negative": torch.full_like(ws, -5),
        "stale": stale,
    }
    for name, content in cases.items():
        say(f"[guards] tiled _end after a {name} workspace")
        moe.moe_plan_and_dispatch_begin(p, ids, plan)
        ws.copy_(content)
        moe.moe_plan_and_dispatch_end(p, ids, plan, x, payload, None)
        torch.cuda.synchronize()
        st = plan.read_status()
        assert st & moe.STATUS_BAD_PLAN, (name, st)
        slot = plan.slot.cpu().numpy()
        assert slot.min() >= -1 and slot.max() < r_max, name
        src = plan.packed_src.cpu().numpy()
        assert src.min() >= -1 and src.max() < n, name
        _assert_guards(big_src, big_pay, r_max)
    say("[guards] proper _begin + _end afterwards")
    moe.moe_plan_and_dispatch_begin(p, ids, plan)
    moe.moe_plan_and_dispatch_end(p, ids, plan, x, payload, None)
    torch.cuda.synchronize()
    pl = oracle.plan(ids_np, e, ep, a, n * min(k, e // ep), h)
    assert plan.read_status() == pl["status"] == 0
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])
    assert np.array_equal(plan.packed_src.cpu().numpy(), pl["packed_src"])
    ref_pay, _ = oracle.dispatch("bf16", x_np, pl)
    assert np.array_equal(u16(payload), ref_pay)
    _assert_guards(big_src, big_pay, r_max)


def test_dispatch_and_combine_skip_rows_outside_the_buffer(moe):
    """Slots past R_max (or below -1) in the plan arrays: the dispatch writes
    nothing through them and the combine reads nothing through them (it
    sums the pairs whose rows exist); offsets past R_max bound nothing."""
    n, h, e, k, ep, a = 700, 512, 8, 3, 2, 4
    rng = np.random.default_rng(41)
    ids_np, w_np = random_routing(rng, n, e, k)
    x_np = random_bf16(rng, (n, h))
    p = moe.problem(n, h, k, e, ep, pad_multiple=a, zero_tail=True)
    plan, big_src, big_pay, r_max = _guarded(moe, p)
    payload = big_pay[:r_max]
    ids = torch.from_numpy(ids_np).cuda()
    moe.moe_dispatch_plan(p, ids, plan)
    torch.cuda.synchronize()
    pl = oracle.plan(ids_np, e, ep, a, n * min(k, e // ep), h)
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])
    bad = pl["slot"].copy()
    bad[::7, 0] = r_max           # one past the last row
    bad[3::11, 1] = r_max + 40    # inside the guard rows
    bad[5::13, 2] = -9            # below -1
    bad[1, :] = 1 << 30
    plan.slot.copy_(torch.from_numpy(bad))
    # an end offset past the buffer: the last expert's pad rows and the zero
    # tail stay inside it
    offs = plan.expert_offsets.clone()
    plan.expert_offsets[e] = r_max + GUARD_ROWS
    say("[guards] dispatch with out-of-range slots and offsets")
    moe.moe_dispatch(p, plan, to_dev_bf16(x_np), payload, None)
    torch.cuda.synchronize()
    _assert_guards(big_src, big_pay, r_max)
    plan.expert_offsets.copy_(offs)
    # rows a valid slot names hold its token
    got = u16(payload)
    ok = (bad >= 0) & (bad < r_max)
    tt, jj = np.nonzero(ok)
    assert np.array_equal(got[bad[tt, jj]], x_np[tt])
    say("[guards] combine with out-of-range slots")
    y_np = random_bf16(rng, (r_max, h))
    out = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(p, plan, to_dev_bf16(y_np), torch.from_numpy(w_np).cuda(), out)
    torch.cuda.synchronize()
    masked = np.where(ok, bad, -1).astype(np.int32)
    ref = oracle.combine(masked, w_np, y_np)
    assert assert_combine_close(u16(out), ref) == 0
