"""GPU parity of moe_plan_and_dispatch (the plan and the dispatch in one
call: one launch for problems of at most 2048 pairs; the counting kernel and
one launch for problems of at most 2048 histogram entries (count tiles x
experts); the plan's kernels and the dispatch otherwise) against the CPU
oracle, and against the two-call path byte for byte.

Bar: every plan array, the status word, every packed row (payload and
scales, live, pad and tail rows) bit-exact.  Inputs come from the seeded
generators only; expected values only from ``oracle``.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import WORKLOADS, make_inputs, random_bf16, random_routing
from gpu_helpers import SENTINEL, say, to_dev_bf16

pytestmark = pytest.mark.gpu

PLAN_KEYS = ("expert_counts", "expert_offsets", "dest_counts", "rank_table", "slot", "packed_src")


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def run_pd(moe, *, ids, hidden, e, ep, a, fmt, cap, gates=None, gs=None, zero_tail=True,
           two_calls=False, halves=False):
    n, k = ids.shape
    h = hidden.shape[1]
    p = moe.problem(n, h, k, e, ep, recv_capacity=cap, pad_multiple=a, fmt=fmt,
                    zero_tail=zero_tail)
    plan = moe.alloc_plan(p)
    for t in (plan.expert_counts, plan.expert_offsets, plan.dest_counts, plan.rank_table,
              plan.slot, plan.packed_src, plan.status):
        t.fill_(-7)
    payload, scales = moe.alloc_payload(p)
    payload.view(torch.uint8).fill_(SENTINEL)
    if scales is not None:
        scales.view(torch.uint8).fill_(SENTINEL)
    x_d = to_dev_bf16(hidden)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
    w_d = None if gates is None else torch.from_numpy(np.ascontiguousarray(gates)).cuda()
    gs_d = None if gs is None else torch.tensor([gs], dtype=torch.float32, device="cuda")
    if two_calls:
        moe.moe_dispatch_plan(p, ids_d, plan)
        if gs_d is not None:
            moe.moe_dispatch_scaled(p, plan, x_d, gs_d, payload, scales)
        elif w_d is not None:
            moe.moe_dispatch_gated(p, plan, x_d, w_d, payload, scales)
        else:
            moe.moe_dispatch(p, plan, x_d, payload, scales)
    elif halves:
        moe.moe_plan_and_dispatch_begin(p, ids_d, plan)
        moe.moe_plan_and_dispatch_end(p, ids_d, plan, x_d, payload, scales, topk_weights=w_d,
                                      input_scale=gs_d)
    else:
        moe.moe_plan_and_dispatch(p, ids_d, plan, x_d, payload, scales, topk_weights=w_d,
                                  input_scale=gs_d)
    torch.cuda.synchronize()
    r_max = moe.moe_max_rows(p)
    got = {name: getattr(plan, name).cpu().numpy() for name in PLAN_KEYS}
    got["rank_table"] = got["rank_table"].view(np.uint32)
    got["packed_src"] = got["packed_src"][:r_max]
    got["status"] = int(plan.status.cpu().numpy().view(np.uint32)[0])
    got["payload"] = payload.view(torch.uint8).cpu().numpy().reshape(r_max, -1) if r_max else None
    got["scales"] = (None if scales is None or not r_max
                     else scales.view(torch.uint8).cpu().numpy().reshape(r_max, -1))
    return got


def expected(*, ids, hidden, e, ep, a, fmt, cap, gates, gs):
    h = hidden.shape[1]
    pl = oracle.plan(ids, e, ep, a, cap, h)
    if fmt == "nvfp4":
        pay, sc = oracle.dispatch_nvfp4(hidden, pl, gs, zero_tail=True)
    elif gates is not None:
        pay, sc = oracle.dispatch_gated(fmt, hidden, pl, gates, zero_tail=True)
    else:
        pay, sc = oracle.dispatch(fmt, hidden, pl, zero_tail=True)
    r = pl["r_max"]
    pay = pay.view(np.uint8).reshape(r, -1) if r else None
    sc = None if sc is None or not r else sc.view(np.uint8).reshape(r, -1)
    return pl, pay, sc


def check_pd(moe, *, ids, hidden, e, ep, a, fmt, cap=None, gates=None, gs=None, zero_tail=True):
    n, k = ids.shape
    if cap is None:
        cap = n * min(k, e // ep)
    kw = dict(ids=ids, hidden=hidden, e=e, ep=ep, a=a, fmt=fmt, cap=cap, gates=gates, gs=gs)
    got = run_pd(moe, zero_tail=zero_tail, **kw)
    pl, pay, sc = expected(**kw)
    for key in PLAN_KEYS:
        assert np.array_equal(got[key], pl[key]), key
    assert got["status"] == pl["status"]
    ru = pl["r_used"]
    for g, x in ((got["payload"], pay), (got["scales"], sc)):
        if x is None:
            continue
        assert np.array_equal(g[:ru], x[:ru])
        if zero_tail:
            assert np.array_equal(g[ru:], x[ru:])
        else:
            assert np.all(g[ru:] == SENTINEL)
    # the plan and dispatch calls, and the two halves, give the same bytes
    for other in (dict(two_calls=True), dict(halves=True)):
        two = run_pd(moe, zero_tail=zero_tail, **other, **kw)
        for key in PLAN_KEYS + ("status", "payload", "scales"):
            if got[key] is None:
                assert two[key] is None
            else:
                assert np.array_equal(np.asarray(got[key]), np.asarray(two[key])), (key, other)
    return got, pl


@pytest.mark.parametrize("name", ["decode_mxfp4_n128", "tiny_bf16_n128", "decode_nvfp4_n128"])
def test_plan_and_dispatch_workloads(moe, name):
    w = WORKLOADS[name]
    say(f"[plan+dispatch] {name}: {w.describe()}")
    inp = make_inputs(w, seed=0, expert_rows=oracle.max_rows(w.n, w.k, w.e, w.a))
    gs = w.input_scale if w.fmt == "nvfp4" else None
    check_pd(moe, ids=inp["ids"], hidden=inp["hidden"], e=w.e, ep=w.ep, a=w.a, fmt=w.fmt,
             cap=w.capacity, gs=gs)
    if w.fmt != "nvfp4":
        say(f"[plan+dispatch] {name} gated")
        check_pd(moe, ids=inp["ids"], hidden=inp["hidden"], e=w.e, ep=w.ep, a=w.a, fmt=w.fmt,
                 cap=w.capacity, gates=inp["weights"])


# n, h, e, k, ep, a, fmt, masked fraction, gated, zero tail
SHAPES = [
    (1, 8, 1, 1, 1, 1, "bf16", 0.0, False, True),        # smallest
    (3, 136, 5, 3, 5, 2, "bf16", 0.0, True, False),
    (200, 512, 64, 6, 8, 128, "bf16", 0.1, False, True),  # 128-row pads
    (256, 7168, 256, 8, 8, 1, "fp8", 0.0, True, False),   # 2048 pairs, the most in one launch
    (100, 160, 1024, 16, 64, 4, "mxfp4", 0.2, False, True),  # E = 1024
    (32, 64, 128, 64, 8, 2, "bf16", 0.1, True, True),     # k = 64
    (2000, 64, 12, 1, 3, 3, "bf16", 0.0, False, False),   # k = 1, 8 slot workgroups
    (77, 384, 32, 5, 4, 7, "fp8", 0.3, False, True),
    (257, 256, 16, 8, 4, 1, "fp8", 0.0, False, True),     # 2056 pairs: 2 count tiles, tiled
    (4096, 256, 64, 6, 8, 128, "bf16", 0.0, True, True),  # 13 count tiles, tiled
    (700, 6144, 8, 3, 4, 2, "bf16", 0.1, False, True),    # 3 slabs: a workgroup straddles two tiles
    (5000, 64, 4, 1, 2, 1, "bf16", 0.0, True, False),     # k = 1: 2048-token tiles
    (100, 128, 64, 64, 8, 2, "bf16", 0.1, False, True),   # k = 64: 32-token tiles
    (300, 256, 1024, 8, 64, 1, "mxfp4", 0.1, False, True),  # 2 x 1024 = 2048 entries: the most tiled
    (600, 256, 1024, 8, 64, 3, "bf16", 0.0, False, True),   # 3 x 1024 entries: separate launches
    (5000, 128, 256, 8, 8, 16, "fp8", 0.05, True, True),   # separate, 20 tiles x 256, 16-row pads
    (3000, 384, 32, 5, 4, 7, "fp8", 0.3, True, True),     # tiled, quantised workgroup order
    (2500, 1024, 128, 8, 8, 128, "mxfp4", 0.05, True, False),  # tiled, 128-row pads
    (3000, 128, 100, 4, 5, 3, "bf16", 0.1, False, True),  # tiled, E = 100 (does not divide 256)
    (4000, 128, 12, 2, 3, 1, "fp8", 0.0, True, False),    # tiled, E = 12
    (150, 128, 257, 8, 257, 2, "bf16", 0.1, False, True),  # E = 257: the scan spans two waves
    (1000, 128, 260, 4, 4, 2, "fp8", 0.1, True, True),    # tiled, E = 260
    # one launch without padding: a workgroup counts the keys below its own
    # pairs while (own pairs) x (key registers) <= 512, else the plan in LDS
    (200, 64, 1024, 8, 64, 1, "bf16", 0.1, False, True),   # E = 1024: the widest keys
    (227, 96, 64, 9, 8, 1, "mxfp4", 0.05, True, True),     # 36 own pairs x 8 registers
    (228, 64, 64, 9, 8, 1, "bf16", 0.0, False, False),     # the same, no tail
    (64, 2048, 16, 4, 4, 1, "bf16", 0.5, False, True),     # half masked, 4 waves a token
    (1, 4096, 8, 8, 2, 1, "fp8", 0.0, True, True),         # one token, 8 waves
    (30, 64, 128, 64, 8, 1, "bf16", 0.1, False, True),     # 256 own pairs x 8: plan in LDS
    (31, 64, 128, 16, 8, 1, "mxfp4", 0.0, True, True),     # 64 own pairs x 4 registers
    (4, 7168, 256, 8, 8, 1, "mxfp4", 0.0, False, False),   # 32 pairs: one key register
    (9, 8200, 32, 4, 4, 1, "bf16", 0.1, True, True),       # 5 slabs: 2 workgroups a token, 3 idle waves
    (256, 7168, 256, 8, 8, 1, "fp8", 0.0, False, True),    # 2048 pairs counted, 14 slabs a token
    (2048, 64, 32, 1, 4, 1, "bf16", 0.1, False, False),    # k = 1, 2048 tokens: 8 key registers, 4 tokens a workgroup
]


@pytest.mark.parametrize("idx", range(len(SHAPES)),
                         ids=[f"n{c[0]}_h{c[1]}_e{c[2]}_k{c[3]}_{c[6]}" for c in SHAPES])
def test_plan_and_dispatch_shapes(moe, idx):
    n, h, e, k, ep, a, fmt, masked, gated, zero_tail = SHAPES[idx]
    say(f"[plan+dispatch] N={n} H={h} E={e} k={k} EP={ep} A={a} {fmt} masked={masked} "
        f"gated={gated} zero_tail={zero_tail}")
    rng = np.random.default_rng(700 + idx)
    ids, wts = random_routing(rng, n, e, k, masked_frac=masked)
    x = random_bf16(rng, (n, h), scale=float(rng.choice([1e-3, 1.0, 40.0])))
    check_pd(moe, ids=ids, hidden=x, e=e, ep=ep, a=a, fmt=fmt, gates=wts if gated else None,
             zero_tail=zero_tail)


def test_plan_and_dispatch_nvfp4_shapes(moe):
    rng = np.random.default_rng(44)
    for n, h, e, k, ep, a, gs in ((128, 256, 32, 8, 4, 2, 3.0), (40, 64, 8, 3, 2, 5, 0.01),
                                  (300, 96, 64, 6, 8, 1, 400.0), (1500, 96, 64, 6, 8, 2, 7.0),
                                  (70, 1536, 64, 8, 8, 1, 5.0), (16, 7168, 256, 8, 8, 1, 336.0)):
        say(f"[plan+dispatch] nvfp4 N={n} H={h} E={e} k={k} A={a} gs={gs}")
        ids, _ = random_routing(rng, n, e, k, masked_frac=0.1)
        check_pd(moe, ids=ids, hidden=random_bf16(rng, (n, h)), e=e, ep=ep, a=a, fmt="nvfp4",
                 gs=gs)


def test_plan_and_dispatch_faults_and_empty(moe):
    rng = np.random.default_rng(45)
    n, k, e = 300, 4, 16
    ids, _ = random_routing(rng, n, e, k)
    ids[n - 1, 3] = ids[n - 1, 0]  # repeated ID in the last token
    ids[n - 2, 1] = 16             # past E
    ids[5, 2] = -4                 # below -1
    say("[plan+dispatch] DUP, BAD and CAPACITY in one launch")
    got, pl = check_pd(moe, ids=ids, hidden=random_bf16(rng, (n, 64)), e=e, ep=4, a=2,
                       fmt="bf16", cap=100)
    assert got["status"] == 1 | 2 | 4
    say("[plan+dispatch] DUP, BAD and CAPACITY, tiled (two count tiles)")
    n = 1000
    ids, _ = random_routing(rng, n, e, k)
    ids[n - 1, 2] = ids[n - 1, 1]
    ids[700, 0] = 99
    ids[3, 3] = -2
    got, pl = check_pd(moe, ids=ids, hidden=random_bf16(rng, (n, 64)), e=e, ep=4, a=2,
                       fmt="bf16", cap=900)
    assert got["status"] == 1 | 2 | 4
    say("[plan+dispatch] DUP, BAD and CAPACITY in one launch without padding")
    n = 200
    ids, _ = random_routing(rng, n, e, k)
    ids[n - 1, 3] = ids[n - 1, 2]
    ids[0, 0] = 16
    ids[77, 1] = -9
    got, pl = check_pd(moe, ids=ids, hidden=random_bf16(rng, (n, 64)), e=e, ep=4, a=1,
                       fmt="bf16", cap=150)
    assert got["status"] == 1 | 2 | 4
    say("[plan+dispatch] N = 0 without padding, with a zero tail")
    check_pd(moe, ids=np.zeros((0, 2), np.int32), hidden=np.zeros((0, 64), np.uint16), e=4,
             ep=2, a=1, fmt="bf16", cap=0)
    say("[plan+dispatch] every pair masked, no padding")
    check_pd(moe, ids=np.full((40, 5), -1, np.int32), hidden=random_bf16(rng, (40, 128)), e=6,
             ep=3, a=1, fmt="fp8")
    say("[plan+dispatch] N = 0 with pad rows and a zero tail")
    check_pd(moe, ids=np.zeros((0, 2), np.int32), hidden=np.zeros((0, 64), np.uint16), e=4,
             ep=2, a=3, fmt="bf16", cap=0)
    say("[plan+dispatch] every pair masked")
    check_pd(moe, ids=np.full((50, 3), -1, np.int32), hidden=random_bf16(rng, (50, 128)), e=6,
             ep=3, a=4, fmt="mxfp4")
