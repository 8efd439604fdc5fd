"""HIP-graph capture of the exchange, fixed-capacity, NVFP4, one-launch and tiled
plan-and-dispatch paths: every replay, with eager work and synchronisation
between replays, reproduces the eager outputs, and the eager outputs equal
the oracle's.  (No call clears
memory with memset nodes; the exchange's multi-block plan keeps its scratch
in the caller's workspace.)"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs, random_bf16, random_routing
from gpu_helpers import assert_combine_close, say, to_dev_bf16, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def capture_and_replay(step, outputs, scribble, replays=4):
    """Run step eagerly, capture it, then replay with the outputs scribbled
    over before each replay; every replay must give the eager bytes."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(replays):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outputs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), it
    return ref


def test_graph_exchange(moe):
    rng = np.random.default_rng(41)
    ep, n, e, k, cap, h = 4, 3000, 32, 4, 3200, 256   # multi-tile plans per rank, drops
    ids, wts = random_routing(rng, ep * n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (ep * n, h))
    say(f"[graph exchange] EP={ep} N={n} E={e} k={k} C={cap} H={h} mxfp4")
    p = moe.problem(n, h, k, e, ep, recv_capacity=cap, fmt="mxfp4")
    xb = moe.alloc_exchange(p)
    payload, scales = moe.alloc_recv_payload(p)
    y = to_dev_bf16(random_bf16(rng, (ep * cap, h)))
    ids_d, x_d, w_d = torch.from_numpy(ids.reshape(ep, n, k)).cuda(), to_dev_bf16(x), \
        torch.from_numpy(wts).cuda()
    out = torch.empty((ep * n, h), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_exchange_plan(p, ids_d, xb)
        moe.moe_exchange_dispatch(p, xb, x_d, payload, scales)
        moe.moe_exchange_combine(p, xb, y, w_d, out)

    outs = [xb.recv_slot, xb.recv_src, xb.rank_table, xb.recv_rows, xb.status, payload, scales, out]

    def scribble():
        for t in (xb.recv_slot, xb.recv_src, xb.rank_table, xb.recv_rows, xb.status):
            t.fill_(-3)
        payload.fill_(0xEE)
        scales.fill_(0xEE)
        out.fill_(7.0)

    capture_and_replay(step, outs, scribble)
    xp = oracle.exchange_plan(ids.reshape(ep, n, k), e, cap, h)
    assert np.array_equal(xb.recv_slot.cpu().numpy(), xp["recv_slot"])
    assert np.array_equal(xb.recv_src.cpu().numpy(), xp["recv_src"])


def test_graph_capacity_and_nvfp4(moe):
    rng = np.random.default_rng(42)
    n, e, k, h = 5000, 64, 6, 512
    ids, wts = random_routing(rng, n, e, k)
    x = random_bf16(rng, (n, h))
    cap = moe.moe_expert_capacity(n, k, e, 0.9)
    say(f"[graph capacity + nvfp4] N={n} E={e} k={k} cap={cap} H={h}")
    p = moe.problem(n, h, k, e, 8, fmt="nvfp4", expert_capacity=cap)
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    y = to_dev_bf16(random_bf16(rng, (e * cap, h)))
    gs = torch.tensor([30.0], dtype=torch.float32, device="cuda")
    ids_d, x_d, w_d = torch.from_numpy(ids).cuda(), to_dev_bf16(x), torch.from_numpy(wts).cuda()
    out = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_dispatch_plan(p, ids_d, plan)
        moe.moe_dispatch_scaled(p, plan, x_d, gs, payload, scales)
        moe.moe_combine(p, plan, y, w_d, out)

    outs = [plan.slot, plan.packed_src, plan.expert_counts, plan.status, payload, scales, out]

    def scribble():
        for t in (plan.slot, plan.packed_src, plan.expert_counts, plan.status):
            t.fill_(-3)
        payload.fill_(0xEE)
        scales.fill_(0xEE)
        out.fill_(7.0)

    capture_and_replay(step, outs, scribble)
    pl = oracle.capacity_plan(ids, e, 8, cap, n * k, h)
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])
    pay, sc = oracle.dispatch_nvfp4(x, pl, 30.0)
    assert np.array_equal(payload.cpu().numpy(), pay) and np.array_equal(scales.cpu().numpy(), sc)
    ref = oracle.combine(pl["slot"], wts, (y.view(torch.int16).cpu().numpy().view(np.uint16)))
    assert_combine_close(u16(out), ref)


def test_graph_plan_and_dispatch(moe):
    """The one-launch plan and dispatch of a decode shape with a combine."""
    w = WORKLOADS["decode_mxfp4_n128"]
    say(f"[graph plan+dispatch] {w.describe()}")
    inp = make_inputs(w, seed=1, expert_rows=oracle.max_rows(w.n, w.k, w.e, w.a))
    p = moe.problem(w.n, w.h, w.k, w.e, w.ep, recv_capacity=w.capacity, pad_multiple=w.a,
                    fmt=w.fmt)
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    x_d, y_d = to_dev_bf16(inp["hidden"]), to_dev_bf16(inp["expert_out"])
    ids_d, w_d = torch.from_numpy(inp["ids"]).cuda(), torch.from_numpy(inp["weights"]).cuda()
    out = torch.empty((w.n, w.h), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_plan_and_dispatch(p, ids_d, plan, x_d, payload, scales)
        moe.moe_combine(p, plan, y_d, w_d, out)

    outs = [plan.slot, plan.packed_src, plan.expert_offsets, plan.rank_table, plan.status,
            payload, scales, out]

    def scribble():
        for t in (plan.slot, plan.packed_src, plan.expert_offsets, plan.rank_table, plan.status):
            t.fill_(-3)
        payload.fill_(0xEE)
        scales.fill_(0xEE)
        out.fill_(7.0)

    ref = capture_and_replay(step, outs, scribble)
    pl = oracle.plan(inp["ids"], w.e, w.ep, w.a, w.capacity, w.h)
    pay, sc = oracle.dispatch(w.fmt, inp["hidden"], pl)
    assert np.array_equal(ref[0].cpu().numpy(), pl["slot"])
    assert np.array_equal(ref[5].cpu().numpy().view(np.uint8).reshape(pay.shape[0], -1),
                          pay.view(np.uint8).reshape(pay.shape[0], -1))
    assert np.array_equal(ref[6].cpu().numpy().view(np.uint8).reshape(sc.shape[0], -1),
                          sc.view(np.uint8).reshape(sc.shape[0], -1))
    assert assert_combine_close(u16(ref[7]), oracle.combine(pl["slot"], inp["weights"],
                                                             inp["expert_out"])) == 0


def test_graph_plan_and_dispatch_tiled(moe):
    """The two halves of a tiled plan and dispatch (the counting kernel, then
    one launch that finishes the plan and dispatches) with a combine."""
    n, h, e, k, ep, a = 1500, 512, 64, 6, 8, 128
    say(f"[graph plan+dispatch tiled] N={n} H={h} E={e} k={k} A={a} bf16")
    rng = np.random.default_rng(12)
    ids, wts = random_routing(rng, n, e, k, masked_frac=0.05)
    x = random_bf16(rng, (n, h))
    cap = n * min(k, e // ep)
    r_max = oracle.max_rows(n, k, e, a)
    y = random_bf16(rng, (r_max, h))
    # every packed row is written (the tail too), so no scribbled byte survives
    p = moe.problem(n, h, k, e, ep, recv_capacity=cap, pad_multiple=a, zero_tail=True)
    assert moe.moe_plan_and_dispatch_mode(p) == moe.PD_TILED
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    x_d, y_d = to_dev_bf16(x), to_dev_bf16(y)
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    out = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_plan_and_dispatch_begin(p, ids_d, plan)
        moe.moe_plan_and_dispatch_end(p, ids_d, plan, x_d, payload, scales)
        moe.moe_combine(p, plan, y_d, w_d, out)

    outs = [plan.slot, plan.packed_src, plan.expert_offsets, plan.rank_table, plan.status,
            payload, out]

    def scribble():
        for t in (plan.slot, plan.packed_src, plan.expert_offsets, plan.rank_table, plan.status):
            t.fill_(-3)
        payload.view(torch.uint8).fill_(0xEE)
        out.fill_(7.0)

    ref = capture_and_replay(step, outs, scribble)
    pl = oracle.plan(ids, e, ep, a, cap, h)
    pay, _ = oracle.dispatch("bf16", x, pl, zero_tail=True)
    assert np.array_equal(ref[0].cpu().numpy(), pl["slot"])
    assert np.array_equal(ref[1].cpu().numpy(), pl["packed_src"])
    assert np.array_equal(ref[2].cpu().numpy(), pl["expert_offsets"])
    assert np.array_equal(u16(ref[5]).reshape(r_max, -1), pay.view(np.uint16).reshape(r_max, -1))
    assert assert_combine_close(u16(ref[6]), oracle.combine(pl["slot"], wts, y)) == 0
