"""GPU parity of gates applied at dispatch, the unweighted combine and the
dense routing-map input (through the C ABI) against the CPU oracle.

Bar: plan arrays, gated payload and scale bytes, converted IDs, weights and
status bit-exact; combine within one bf16 ulp.  Inputs come from the seeded
generators only; expected values only from ``oracle``.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import (WORKLOADS, make_inputs, random_bf16,
                                            random_routing)
from gpu_helpers import SENTINEL, assert_combine_close, say, to_dev_bf16, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def run_gated(moe, *, ids, weights, hidden, e, ep, a, fmt, expert_out=None, zero_tail=True):
    """plan + gated dispatch + unweighted combine on the GPU."""
    n, k = ids.shape
    h = hidden.shape[1]
    p = moe.problem(n, h, k, e, ep, pad_multiple=a, fmt=fmt, zero_tail=zero_tail)
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    payload.view(torch.uint8).fill_(SENTINEL)
    if scales is not None:
        scales.view(torch.uint8).fill_(SENTINEL)
    x_d = to_dev_bf16(hidden)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(weights).cuda()
    out = torch.full((n, h), 7.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_plan(p, ids_d, plan)
    moe.moe_dispatch_gated(p, plan, x_d, w_d, payload, scales)
    y_d = payload if expert_out is None else to_dev_bf16(expert_out)
    moe.moe_combine(p, plan, y_d, None, out)
    torch.cuda.synchronize()
    return dict(slot=plan.slot.cpu().numpy(), payload=payload.view(torch.uint8).cpu().numpy(),
                scales=None if scales is None else scales.view(torch.uint8).cpu().numpy(),
                out=u16(out), status=int(plan.status.cpu().numpy().view(np.uint32)[0]))


def check_gated(moe, *, ids, weights, hidden, e, ep, a, fmt, expert_out=None):
    h = hidden.shape[1]
    got = run_gated(moe, ids=ids, weights=weights, hidden=hidden, e=e, ep=ep, a=a, fmt=fmt,
                    expert_out=expert_out)
    n, k = ids.shape
    pl = oracle.plan(ids, e, ep, a, n * min(k, e // ep), h)
    assert np.array_equal(got["slot"], pl["slot"])
    pay, sc = oracle.dispatch_gated(fmt, hidden, pl, weights, zero_tail=True)
    assert np.array_equal(got["payload"], pay.view(np.uint8))
    if sc is not None:
        assert np.array_equal(got["scales"], sc.view(np.uint8))
    y = pay.view(np.uint16) if expert_out is None else expert_out
    ref = oracle.combine(pl["slot"], None, y)
    return got, assert_combine_close(got["out"], ref)


@pytest.mark.parametrize("name", ["uniform_bf16_n4096", "decode_mxfp4_n128", "tiny_bf16_n128"])
def test_gated_workload_parity(moe, name):
    """Every output of the workload with gates applied at dispatch."""
    w = WORKLOADS[name]
    say(f"[gated parity] {name}: {w.describe()}")
    r_max = oracle.max_rows(w.n, w.k, w.e, w.a)
    inp = make_inputs(w, seed=0, expert_rows=r_max)
    _, nonexact = check_gated(moe, ids=inp["ids"], weights=inp["weights"], hidden=inp["hidden"],
                              e=w.e, ep=w.ep, a=w.a, fmt=w.fmt, expert_out=inp.get("expert_out"))
    assert nonexact == 0


# n, h, e, k, ep, a, fmt, masked fraction
FUZZ = [
    (300, 7168, 256, 8, 32, 1, "fp8", 0.0),
    (257, 1152, 32, 3, 4, 2, "fp8", 0.2),
    (777, 520, 16, 5, 4, 3, "bf16", 0.1),
    (1000, 96, 1024, 16, 64, 4, "mxfp4", 0.2),
    (4097, 160, 12, 12, 3, 1, "mxfp4", 0.0),
    (600, 2112, 128, 9, 16, 8, "bf16", 0.3),
]


@pytest.mark.parametrize("idx", range(len(FUZZ)),
                         ids=[f"n{c[0]}_h{c[1]}_e{c[2]}_k{c[3]}_{c[6]}" for c in FUZZ])
def test_gated_fuzz_shapes(moe, idx):
    n, h, e, k, ep, a, fmt, masked = FUZZ[idx]
    say(f"[gated fuzz] N={n} H={h} E={e} k={k} EP={ep} A={a} {fmt} masked={masked}")
    rng = np.random.default_rng(500 + idx)
    ids, wts = random_routing(rng, n, e, k, masked_frac=masked)
    x = random_bf16(rng, (n, h), scale=float(rng.choice([1e-3, 1.0, 50.0])))
    y = None if fmt == "bf16" else random_bf16(rng, (oracle.max_rows(n, k, e, a), h))
    check_gated(moe, ids=ids, weights=wts, hidden=x, e=e, ep=ep, a=a, fmt=fmt, expert_out=y)


@pytest.mark.parametrize("fmt,h", [("bf16", 264), ("fp8", 384), ("mxfp4", 160)])
def test_gated_extreme_gates(moe, fmt, h):
    """Zero, negative, subnormal-producing and large gates, and blocks whose
    products underflow."""
    rng = np.random.default_rng(77)
    n, e, k = 96, 8, 4
    ids, _ = random_routing(rng, n, e, k)
    choices = np.array([0.0, -0.0, -0.5, 1.0, 2.0 ** -120, 1e-30, 3.0e4, 0.3, -7.25, 2.0 ** -149],
                       np.float32)
    wts = rng.choice(choices, size=(n, k)).astype(np.float32)
    x = random_bf16(rng, (n, h))
    x[:8] = random_bf16(rng, (8, h), scale=1e-30)
    say(f"[gated extremes] {fmt} H={h}")
    check_gated(moe, ids=ids, weights=wts, hidden=x, e=e, ep=2, a=2, fmt=fmt,
                expert_out=None if fmt == "bf16" else random_bf16(rng, (n * k + e, h)))


def test_gated_exchange_parity(moe):
    """Gates at dispatch on the exchange across 4 simulated ranks (FP8), with
    drops, against the oracle's exchange plan and gated rows."""
    rng = np.random.default_rng(31)
    ep, n, e, k, cap, h = 4, 300, 32, 4, 280, 256
    ids, wts = random_routing(rng, ep * n, e, k, masked_frac=0.1)
    x = random_bf16(rng, (ep * n, h))
    y = random_bf16(rng, (ep * cap, h))
    say(f"[gated exchange] EP={ep} N={n} E={e} k={k} C={cap} H={h} fp8")
    p = moe.problem(n, h, k, e, ep, recv_capacity=cap, fmt="fp8")
    xb = moe.alloc_exchange(p)
    payload, scales = moe.alloc_recv_payload(p)
    payload.fill_(SENTINEL)
    scales.view(torch.uint8).fill_(SENTINEL)
    out = torch.empty((ep * n, h), dtype=torch.bfloat16, device="cuda")
    moe.moe_exchange_plan(p, torch.from_numpy(ids.reshape(ep, n, k)).cuda(), xb)
    moe.moe_exchange_dispatch_gated(p, xb, to_dev_bf16(x), torch.from_numpy(wts).cuda(),
                                    payload, scales)
    moe.moe_exchange_combine(p, xb, to_dev_bf16(y), None, out)
    torch.cuda.synchronize()
    xp = oracle.exchange_plan(ids.reshape(ep, n, k), e, cap, h)
    assert np.array_equal(xb.recv_slot.cpu().numpy(), xp["recv_slot"])
    slot = xp["recv_slot"].reshape(ep * n, k)
    pay, sc = oracle.dispatch_gated("fp8", x, dict(slot=slot, r_max=ep * cap, r_used=ep * cap), wts)
    assert np.array_equal(payload.cpu().numpy(), pay)
    assert np.array_equal(scales.view(torch.uint8).cpu().numpy(), sc.view(np.uint8))
    assert assert_combine_close(u16(out), oracle.combine(slot, None, y)) == 0


def run_map(moe, m, probs, k, with_w=True):
    n, e = m.shape
    p = moe.problem(n, 64, k, e, 1)
    ids = torch.full((max(n, 1), k), -9, dtype=torch.int32, device="cuda")
    w = torch.full((max(n, 1), k), 9.0, dtype=torch.float32, device="cuda") if with_w else None
    st = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.moe_map_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda")
    m_d = torch.from_numpy(np.ascontiguousarray(m)).cuda()
    p_d = None if probs is None else torch.from_numpy(probs).cuda()
    moe.moe_routing_map_to_topk(p, m_d, p_d, ids, w, st, ws)
    torch.cuda.synchronize()
    return (ids.cpu().numpy()[:n], None if w is None else w.cpu().numpy()[:n],
            int(st.cpu().numpy()[0]))


@pytest.mark.parametrize("n,e,k,density", [(1, 8, 2, 0.5), (1000, 64, 6, 0.08), (333, 7, 3, 0.6),
                                           (4096, 256, 8, 0.03), (257, 1024, 16, 0.02),
                                           (513, 100, 4, 0.05)])
def test_routing_map_parity(moe, n, e, k, density):
    say(f"[routing map] N={n} E={e} k={k} density={density}")
    rng = np.random.default_rng(n + e)
    m = ((rng.random((n, e)) < density) * rng.integers(1, 256, (n, e))).astype(np.uint8)
    probs = rng.random((n, e)).astype(np.float32)
    ids, w, st = run_map(moe, m, probs, k)
    rids, rw, rst = oracle.routing_map_to_topk(m, probs, k)
    assert np.array_equal(ids, rids) and np.array_equal(w, rw) and st == rst
    ids2, _, st2 = run_map(moe, m, None, k, with_w=False)
    assert np.array_equal(ids2, rids) and st2 == rst


def test_routing_map_overflow_and_empty(moe):
    rng = np.random.default_rng(4)
    m = (rng.random((300, 32)) < 0.2).astype(np.uint8)
    m[17, :] = 1  # one token routes to every expert
    ids, w, st = run_map(moe, m, None, 4)
    rids, rw, rst = oracle.routing_map_to_topk(m, None, 4)
    assert rst == 8 and st == 8 and np.array_equal(ids, rids) and np.array_equal(w, rw)
    ids, w, st = run_map(moe, np.zeros((0, 16), np.uint8), None, 2)
    assert st == 0 and ids.shape == (0, 2)


def test_routing_map_end_to_end(moe):
    """Dense map and probabilities -> compact top-k on the GPU -> plan,
    dispatch, weighted combine; the oracle runs the same steps."""
    rng = np.random.default_rng(12)
    n, e, k, h = 2000, 64, 6, 512
    ids0, w0 = random_routing(rng, n, e, k, masked_frac=0.1)
    m = np.zeros((n, e), np.uint8)
    probs = np.zeros((n, e), np.float32)
    t = np.broadcast_to(np.arange(n)[:, None], (n, k))
    ok = ids0 >= 0
    m[t[ok], ids0[ok]] = 1
    probs[t[ok], ids0[ok]] = w0[ok]
    x = random_bf16(rng, (n, h))
    say(f"[routing map e2e] N={n} E={e} k={k} H={h}")
    p = moe.problem(n, h, k, e, 8, pad_multiple=4)
    ids = torch.empty((n, k), dtype=torch.int32, device="cuda")
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_map_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    moe.moe_routing_map_to_topk(p, torch.from_numpy(m).cuda(), torch.from_numpy(probs).cuda(),
                                ids, w, st, ws)
    plan = moe.alloc_plan(p)
    payload, _ = moe.alloc_payload(p)
    out = torch.empty((n, h), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_plan(p, ids, plan)
    moe.moe_dispatch(p, plan, to_dev_bf16(x), payload, None)
    moe.moe_combine(p, plan, payload, w, out)
    torch.cuda.synchronize()
    rids, rw, rst = oracle.routing_map_to_topk(m, probs, k)
    assert int(st.item()) == rst == 0
    pl = oracle.plan(rids, e, 8, 4, n * min(k, e // 8), h)
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])
    pay, _ = oracle.dispatch("bf16", x, pl)
    ref = oracle.combine(pl["slot"], rw, pay)
    assert assert_combine_close(u16(out), ref) == 0


@pytest.mark.parametrize("three_calls", [False, True], ids=["bench_step", "three_calls"])
def test_gated_map_workload_bench_step(moe, three_calls):
    """The benchmark's own step for gated_map_bf16_n4096 (N = H = 4096, E = 64,
    k = 6, A = 128; tiled plan-and-dispatch): the dense map and probabilities
    converted on the device, then moe_plan_and_dispatch_begin / _end with the
    gates (or, as three calls, the plan and the gated dispatch), then the
    unweighted combine, on both buffer sets it rotates over; every IDs,
    gates, plan array, packed row and output against the oracle's same
    steps."""
    import bench
    w = WORKLOADS["gated_map_bf16_n4096"]
    say(f"[gated map workload] {w.describe()}; three_calls={three_calls}")
    inp = make_inputs(w, seed=0)
    path = bench.Path(moe, torch, w, inp, copies=2)
    assert path.mode() == "tiled"
    for s in path.sets:
        s["payload"].view(torch.uint8).fill_(SENTINEL)
        s["ids"].fill_(-9)
        s["w"].fill_(9.0)
        s["map_status"].fill_(77)
    for i in range(2):
        (path.step_three_calls if three_calls else path.step)(i)
    torch.cuda.synchronize()
    rids, rw, rst = oracle.routing_map_to_topk(inp["map"], inp["probs"], w.k)
    assert rst == 0
    pl = oracle.plan(rids, w.e, w.ep, w.a, w.capacity, w.h)
    ru = pl["r_used"]
    ref_pay, _ = oracle.dispatch_gated("bf16", inp["hidden"], pl, rw, zero_tail=False)
    ref_out = oracle.combine(pl["slot"], None, ref_pay)
    for s in path.sets:
        assert np.array_equal(s["ids"].cpu().numpy(), rids)
        assert np.array_equal(s["w"].cpu().numpy(), rw)
        assert int(s["map_status"].item()) == 0
        plan = s["plan"]
        assert plan.read_status() == pl["status"] == 0
        for key in ("expert_counts", "expert_offsets", "dest_counts", "slot", "packed_src"):
            assert np.array_equal(getattr(plan, key).cpu().numpy(), pl[key]), key
        assert np.array_equal(plan.rank_table.cpu().numpy().view(np.uint32), pl["rank_table"])
        got = u16(s["payload"])
        assert np.array_equal(got[:ru], ref_pay[:ru])
        assert np.all(got[ru:].view(np.uint8) == SENTINEL)
        assert assert_combine_close(u16(s["out"]), ref_out) == 0
