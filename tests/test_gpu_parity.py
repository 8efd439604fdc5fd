"""GPU parity: libmoe's HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact on every plan array, on packed rows (bf16 bits, E4M3 codes,
fp32 scales, E2M1 nibbles, E8M0 bytes) and on pad/tail rows; combine within
one bf16 ulp (and, by construction of both sides, bit-exact).  Inputs come
from the seeded generators only; expected values only from ``oracle``.
"""

import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import (WORKLOADS, make_inputs, random_bf16,
                                            random_routing)

pytestmark = pytest.mark.gpu

from gpu_helpers import (SENTINEL, assert_combine_close, assert_rows_are_tokens, say,
                         to_dev_bf16, u16)


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def run_path(moe, *, ids, weights, hidden, e, ep, a, fmt, cap=None, expert_out=None,
             zero_tail=True, stream=None, halves=False):
    """plan + dispatch + combine on the GPU; identity experts if expert_out is None.
    halves: the plan and dispatch as moe_plan_and_dispatch_begin + _end (the
    calls bench.py times) instead of moe_dispatch_plan + moe_dispatch."""
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
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(weights).cuda()
    out = torch.full((n, h), 7.0, dtype=torch.bfloat16, device="cuda")
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        if halves:
            moe.moe_plan_and_dispatch_begin(p, ids_d, plan)
            moe.moe_plan_and_dispatch_end(p, ids_d, plan, x_d, payload, scales)
        else:
            moe.moe_dispatch_plan(p, ids_d, plan)
            moe.moe_dispatch(p, plan, x_d, payload, scales)
        if expert_out is None:
            assert fmt == "bf16"
            y_d = payload
        else:
            y_d = to_dev_bf16(expert_out)
        moe.moe_combine(p, plan, y_d, w_d, out)
    torch.cuda.synchronize()
    res = dict(
        expert_counts=plan.expert_counts.cpu().numpy(),
        expert_offsets=plan.expert_offsets.cpu().numpy(),
        dest_counts=plan.dest_counts.cpu().numpy(),
        rank_table=plan.rank_table.cpu().numpy().view(np.uint32),
        slot=plan.slot.cpu().numpy(),
        packed_src=plan.packed_src.cpu().numpy()[:moe.moe_max_rows(p)],
        status=int(plan.status.cpu().numpy().view(np.uint32)[0]),
        payload=payload.view(torch.uint8).cpu().numpy(),
        scales=None if scales is None else scales.view(torch.uint8).cpu().numpy(),
        out=u16(out),
    )
    return res


def assert_plan_equal(got, ref):
    for key in ("expert_counts", "expert_offsets", "dest_counts", "rank_table", "slot",
                "packed_src"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["status"] == ref["status"]


def payload_bytes_ref(fmt, x, pl, zero_tail):
    pay, sc = oracle.dispatch(fmt, x, pl, zero_tail=zero_tail)
    return pay.view(np.uint8).reshape(pay.shape[0], -1), \
        (None if sc is None else sc.view(np.uint8).reshape(sc.shape[0], -1))


def check_full(moe, *, ids, weights, hidden, e, ep, a, fmt, cap=None, expert_out=None,
               zero_tail=True, stream=None, halves=False):
    n, k = ids.shape
    h = hidden.shape[1]
    if cap is None:
        cap = n * min(k, e // ep)
    got = run_path(moe, ids=ids, weights=weights, hidden=hidden, e=e, ep=ep, a=a, fmt=fmt,
                   cap=cap, expert_out=expert_out, zero_tail=zero_tail, stream=stream,
                   halves=halves)
    pl = oracle.plan(ids, e, ep, a, cap, h)
    assert_plan_equal(got, pl)
    pay, sc = payload_bytes_ref(fmt, hidden, pl, zero_tail=True)
    ru = pl["r_used"]
    gp = got["payload"].reshape(pay.shape[0], -1)
    assert np.array_equal(gp[:ru], pay[:ru])
    if zero_tail:
        assert np.array_equal(gp[ru:], pay[ru:])
    else:
        assert np.all(gp[ru:] == SENTINEL)
    if sc is not None:
        gs = got["scales"].reshape(sc.shape[0], -1)
        assert np.array_equal(gs[:ru], sc[:ru])
        if zero_tail:
            assert np.array_equal(gs[ru:], sc[ru:])
        else:
            assert np.all(gs[ru:] == SENTINEL)
    y = pay.view(np.uint16) if expert_out is None else expert_out
    ref_out = oracle.combine(pl["slot"], weights, y)
    nonexact = assert_combine_close(got["out"], ref_out)
    return got, pl, nonexact


# ------------------------------------------------------------ workloads ---

SMALL = ["tiny_bf16_n128", "uniform_bf16_n4096", "zipf_bf16_n16384", "decode_mxfp4_n128"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_full_parity(moe, name):
    """Every output of the full-size workload, element by element."""
    w = WORKLOADS[name]
    say(f"[parity] {name}: {w.describe()}")
    r_max = oracle.max_rows(w.n, w.k, w.e, w.a)
    inp = make_inputs(w, seed=0, expert_rows=r_max)
    got, pl, nonexact = check_full(moe, ids=inp["ids"], weights=inp["weights"],
                                   hidden=inp["hidden"], e=w.e, ep=w.ep, a=w.a, fmt=w.fmt,
                                   cap=w.capacity, expert_out=inp.get("expert_out"),
                                   zero_tail=True)
    assert got["status"] == 0
    assert nonexact == 0, f"{nonexact} combine outputs differ by one ulp"
    if w.experts == "identity":
        x = inp["hidden"]
        negz = x == 0x8000
        assert np.array_equal(got["out"][~negz], x[~negz])


@pytest.mark.parametrize("name", SMALL)
def test_workload_full_parity_bench_calls(moe, name):
    """The same, through the calls and flags bench.py times: the plan and the
    dispatch as moe_plan_and_dispatch_begin + _end (one launch, tiled or
    separate by size), no zero tail (rows past R_used keep their bytes)."""
    w = WORKLOADS[name]
    p = moe.problem(w.n, w.h, w.k, w.e, w.ep, recv_capacity=w.capacity, pad_multiple=w.a,
                    fmt=w.fmt)
    mode = moe.moe_plan_and_dispatch_mode(p)
    say(f"[parity halves] {name}: {w.describe()}; mode {mode}")
    r_max = oracle.max_rows(w.n, w.k, w.e, w.a)
    inp = make_inputs(w, seed=0, expert_rows=r_max)
    got, pl, nonexact = check_full(moe, ids=inp["ids"], weights=inp["weights"],
                                   hidden=inp["hidden"], e=w.e, ep=w.ep, a=w.a, fmt=w.fmt,
                                   cap=w.capacity, expert_out=inp.get("expert_out"),
                                   zero_tail=False, halves=True)
    assert got["status"] == 0
    assert nonexact == 0, f"{nonexact} combine outputs differ by one ulp"
    if name == "uniform_bf16_n4096":
        assert mode == moe.PD_TILED


@pytest.mark.parametrize("halves", [False, True], ids=["three_calls", "bench_calls"])
def test_fp8_workload_full_parity(moe, halves):
    """FP8 1x128 workload at full size (N=8192, H=7168, E=256, k=8, EP=32):
    the whole plan, every packed row and scale row (the oracle encodes each
    token once; row r must hold the encoding of token packed_src[r]) and
    every combine output; through the three calls, and through the calls and
    flags bench.py times (moe_plan_and_dispatch_begin + _end, no zero tail:
    rows past R_used keep their bytes)."""
    w = WORKLOADS["fp8_b128_n8192"]
    say(f"[parity] {w.name}: {w.describe()}; halves={halves}")
    r_max = oracle.max_rows(w.n, w.k, w.e, w.a)
    inp = make_inputs(w, seed=0, expert_rows=r_max)
    got = run_path(moe, ids=inp["ids"], weights=inp["weights"], hidden=inp["hidden"], e=w.e,
                   ep=w.ep, a=w.a, fmt="fp8", cap=w.capacity, expert_out=inp["expert_out"],
                   zero_tail=not halves, halves=halves)
    pl = oracle.plan(inp["ids"], w.e, w.ep, w.a, w.capacity, w.h)
    assert_plan_equal(got, pl)
    assert got["status"] == 0
    enc, enc_sc = oracle.encode_rows("fp8", inp["hidden"])
    ru = pl["r_used"]
    pay = got["payload"].reshape(r_max, w.h)
    sc = got["scales"].reshape(r_max, -1)
    assert_rows_are_tokens(pay[:ru], sc[:ru], enc, enc_sc, pl["packed_src"][:ru])
    if halves:
        assert np.all(pay[ru:] == SENTINEL) and np.all(sc[ru:] == SENTINEL)
    else:
        assert not np.any(pay[ru:]) and not np.any(sc[ru:])
    ref = oracle.combine(pl["slot"], inp["weights"], inp["expert_out"])
    assert assert_combine_close(got["out"], ref) == 0


# ----------------------------------------------------------- fuzz shapes ---

FUZZ = [
    # n, h, e, k, ep, a, fmt, masked
    (1, 8, 1, 1, 1, 1, "bf16", 0.0),
    (3, 136, 5, 3, 5, 2, "bf16", 0.0),
    (777, 520, 16, 5, 4, 3, "bf16", 0.1),
    (2049, 384, 64, 7, 8, 16, "fp8", 0.05),
    (300, 1152, 32, 2, 2, 1, "fp8", 0.0),
    (5000, 256, 256, 8, 32, 128, "bf16", 0.0),
    (1000, 96, 1024, 16, 64, 4, "mxfp4", 0.2),
    (4097, 160, 12, 12, 3, 1, "mxfp4", 0.0),
    (600, 2112, 128, 9, 16, 8, "bf16", 0.3),
    (64, 7168, 256, 8, 8, 1, "mxfp4", 0.0),
    (260, 128, 2, 2, 1, 5, "fp8", 0.5),
    (3840, 64, 64, 8, 8, 128, "bf16", 0.0),    # 15 count tiles of whole tokens
    (32000, 64, 8, 1, 8, 1, "bf16", 0.1),      # k=1: 16 tiles of 2048 pairs
    (1500, 64, 1024, 6, 64, 2, "bf16", 0.1),   # E=1024 over 5 tiles (expert passes)
    (200, 64, 128, 64, 8, 2, "bf16", 0.1),     # k=64, the largest top-k: every lane a slot
    (70, 256, 64, 64, 4, 1, "fp8", 0.0),       # k=E=64
    (40, 65536, 16, 4, 4, 1, "bf16", 0.0),     # H=65536: 32 slabs per token
    (24, 16384, 8, 2, 2, 3, "fp8", 0.0),       # H=16384: 32 FP8 slabs per token
]


@pytest.mark.parametrize("idx", range(len(FUZZ)),
                         ids=[f"{c[6]}-n{c[0]}-h{c[1]}-e{c[2]}-k{c[3]}" for c in FUZZ])
def test_fuzz_shapes(moe, idx):
    n, h, e, k, ep, a, fmt, masked = FUZZ[idx]
    say(f"[fuzz] n={n} h={h} e={e} k={k} ep={ep} a={a} {fmt} masked={masked}")
    rng = np.random.default_rng(1000 + idx)
    ids, w = random_routing(rng, n, e, k, masked_frac=masked)
    x = random_bf16(rng, (n, h))
    y = None
    if fmt != "bf16":
        y = random_bf16(rng, (oracle.max_rows(n, k, e, a), h))
    for zero_tail in (True, False):
        check_full(moe, ids=ids, weights=w, hidden=x, e=e, ep=ep, a=a, fmt=fmt,
                   expert_out=y, zero_tail=zero_tail)


# ------------------------------------------------------------- edge cases ---

def test_empty_problem(moe):
    say("[edge] N=0")
    ids = np.zeros((0, 2), np.int32)
    got = run_path(moe, ids=ids, weights=np.zeros((0, 2), np.float32),
                   hidden=np.zeros((0, 64), np.uint16), e=4, ep=2, a=3, fmt="bf16", cap=0)
    ref = oracle.plan(ids, 4, 2, 3, 0, 64)
    assert_plan_equal(got, ref)
    assert np.all(got["payload"] == 0)  # zero tail covers the whole pad-only buffer


def test_all_masked_and_one_expert(moe):
    say("[edge] all masked / one expert / k=E / L=1")
    rng = np.random.default_rng(9)
    x = random_bf16(rng, (50, 64))
    w = np.full((50, 3), 1 / 3, np.float32)
    got, _, _ = check_full(moe, ids=np.full((50, 3), -1, np.int32), weights=w, hidden=x,
                           e=4, ep=4, a=2, fmt="bf16")
    assert np.all(got["out"] == 0)
    check_full(moe, ids=np.zeros((3000, 1), np.int32), weights=np.ones((3000, 1), np.float32),
               hidden=random_bf16(rng, (3000, 64)), e=8, ep=8, a=128, fmt="bf16")
    ids = np.tile(np.arange(6, dtype=np.int32), (40, 1))
    check_full(moe, ids=ids, weights=np.full((40, 6), 1 / 6, np.float32),
               hidden=random_bf16(rng, (40, 256)), e=6, ep=3, a=1, fmt="fp8",
               expert_out=random_bf16(rng, (240, 256)))


def test_fault_bits(moe):
    say("[edge] bad / duplicate ids, capacity")
    rng = np.random.default_rng(10)
    n, k, e = 3000, 4, 16
    ids, w = random_routing(rng, n, e, k)
    ids[5, 1] = 99          # out of range
    ids[7, 0] = -5          # out of range
    ids[11, 2] = ids[11, 0]  # repeated within a token
    got, pl, _ = check_full(moe, ids=ids, weights=w, hidden=random_bf16(rng, (n, 64)), e=e,
                            ep=4, a=1, fmt="bf16", cap=10)
    assert got["status"] == 1 | 2 | 4 == pl["status"]


def test_fault_bits_far_from_block_zero(moe):
    """Faults only in the last tokens: the block that writes the status word
    must report pairs of a count tile it does not place itself."""
    n = 8000
    say(f"[edge] bad / duplicate ids in the last tokens, n={n}")
    rng = np.random.default_rng(11)
    k, e = 4, 16
    ids, w = random_routing(rng, n, e, k)
    for bits, edit in ((2, lambda a: a.__setitem__((n - 1, 3), a[n - 1, 1])),
                       (1, lambda a: a.__setitem__((n - 2, 2), 16))):
        bad = ids.copy()
        edit(bad)
        got, pl, _ = check_full(moe, ids=bad, weights=w, hidden=random_bf16(rng, (n, 64)), e=e,
                                ep=4, a=2, fmt="bf16")
        assert got["status"] == bits == pl["status"]


def test_extreme_values(moe):
    say("[edge] zero / subnormal / huge blocks")
    rng = np.random.default_rng(12)
    n, h = 64, 512
    x = random_bf16(rng, (n, h))
    x[0, :] = 0x0000
    x[1, :] = 0x8000                       # -0 everywhere
    x[2, :128] = 0x0001                    # bf16 subnormals
    x[2, 128:160] = 0x8003
    x[3, :] = 0x7F7F                       # largest finite bf16
    x[4, ::2] = 0xFF7F
    x[5, :] = random_bf16(rng, (1, h), scale=1e-38)[0]  # near the fp32 subnormal range
    x[6, :] = random_bf16(rng, (1, h), scale=1e30)[0]
    ids, w = random_routing(rng, n, 8, 2)
    for fmt in ("fp8", "mxfp4"):
        y = random_bf16(rng, (oracle.max_rows(n, 2, 8, 1), h))
        check_full(moe, ids=ids, weights=w, hidden=x, e=8, ep=2, a=1, fmt=fmt, expert_out=y)
    # bf16 identity round trip with huge values stays finite and exact
    ids2, w2 = random_routing(rng, n, 8, 1)
    check_full(moe, ids=ids2, weights=np.ones((n, 1), np.float32), hidden=x, e=8, ep=2, a=1,
               fmt="bf16")


def test_deterministic_and_side_stream(moe):
    say("[edge] determinism, side stream")
    w = WORKLOADS["zipf_bf16_n16384"]
    inp = make_inputs(w, seed=1)
    runs = [run_path(moe, ids=inp["ids"], weights=inp["weights"], hidden=inp["hidden"],
                     e=w.e, ep=w.ep, a=w.a, fmt="bf16", cap=w.capacity,
                     stream=torch.cuda.Stream() if i == 2 else None) for i in range(3)]
    for r in runs[1:]:
        for key in ("slot", "packed_src", "rank_table", "payload", "out"):
            assert np.array_equal(r[key], runs[0][key]), key


def test_fp8_every_block_maximum(moe):
    """One 1x128 block for every positive finite bf16 block maximum (0x0001 ..
    0x7F7F, so both sides of the fast-quotient threshold), the other values
    random bf16 magnitudes up to it with random signs; every code and scale
    against the oracle."""
    say("[edge] fp8: every bf16 block maximum")
    rng = np.random.default_rng(77)
    amax = np.arange(1, 0x7F80, dtype=np.uint32)
    nb = -(-amax.size // 8) * 8
    amax = np.concatenate([amax, np.zeros(nb - amax.size, np.uint32)])  # zero blocks pad
    mags = np.minimum((rng.random((nb, 128)) * (amax[:, None] + 1)).astype(np.uint32), amax[:, None])
    signs = rng.integers(0, 2, (nb, 128)).astype(np.uint32) << 15
    blocks = (mags | signs).astype(np.uint16)
    pos = rng.integers(0, 128, nb)
    blocks[np.arange(nb), pos] = (amax | (rng.integers(0, 2, nb).astype(np.uint32) << 15)).astype(np.uint16)
    x = np.ascontiguousarray(blocks.reshape(-1, 1024))
    n = x.shape[0]
    ids = np.zeros((n, 1), np.int32)
    w = np.ones((n, 1), np.float32)
    y = random_bf16(rng, (n, 1024))
    check_full(moe, ids=ids, weights=w, hidden=x, e=1, ep=1, a=1, fmt="fp8", expert_out=y)


def test_graph_capture_replays_match_eager(moe):
    """The three calls captured in one HIP graph and replayed several times,
    with eager work and synchronisation between replays: every replay must
    reproduce the eager outputs (the plan clears nothing with memset nodes)."""
    say("[graph] capture plan + dispatch + combine, replay 4 times")
    w = WORKLOADS["decode_mxfp4_n128"]
    r_max = oracle.max_rows(w.n, w.k, w.e, w.a)
    inp = make_inputs(w, seed=3, expert_rows=r_max)
    p = moe.problem(w.n, w.h, w.k, w.e, w.ep, pad_multiple=w.a, fmt=w.fmt, zero_tail=True)
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    x = to_dev_bf16(inp["hidden"])
    ids = torch.from_numpy(inp["ids"]).cuda()
    wts = torch.from_numpy(inp["weights"]).cuda()
    y = to_dev_bf16(inp["expert_out"])
    out = torch.empty((w.n, w.h), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.moe_dispatch_plan(p, ids, plan)
        moe.moe_dispatch(p, plan, x, payload, scales)
        moe.moe_combine(p, plan, y, wts, out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (plan.slot, plan.packed_src, payload, scales, out)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        step()
    for it in range(4):
        for t in (plan.slot, plan.packed_src, out):
            t.fill_(-3)
        payload.view(torch.uint8).fill_(0xEE)
        scales.fill_(0xEE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (plan.slot, plan.packed_src, payload, scales, out)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), it
    pl = oracle.plan(inp["ids"], w.e, w.ep, w.a, w.capacity, w.h)
    assert np.array_equal(plan.slot.cpu().numpy(), pl["slot"])


def test_largest_buffer_the_table_allows(moe):
    """N = 131071, H = 4096, E = 128, k = 8, A = 1: R_max * H = 4,294,934,528,
    the largest element count below 2^32 that the uint32 table allows (one
    more token is refused), a payload of 8.6 GB, so row byte offsets run far
    past 4 GiB.  The whole plan against the oracle; the packed rows of 4096
    sampled rows (the last ones included) against the oracle's encoding of
    their tokens; every combine output through the identity round trip
    (weights summing to 1, so combine(dispatch(x)) is x bit for bit)."""
    n, h, e, k, ep = 131071, 4096, 128, 8, 16
    assert moe.moe_check_problem(moe.problem(n + 1, h, k, e, ep)) == moe.MOE_EOVERFLOW
    p = moe.problem(n, h, k, e, ep)
    r_max = moe.moe_max_rows(p)
    assert r_max * h == 4294934528 < 1 << 32
    say(f"[edge] largest buffer: N={n} H={h} E={e} k={k}, R_max={r_max}, "
        f"payload {r_max * h * 2 / 1e9:.1f} GB")
    rng = np.random.default_rng(2026)
    ids, w = random_routing(rng, n, e, k)
    x = random_bf16(rng, (n, h))
    plan = moe.alloc_plan(p)
    payload, _ = moe.alloc_payload(p)
    x_d = to_dev_bf16(x)
    ids_d = torch.from_numpy(ids).cuda()
    out = torch.empty_like(x_d)
    moe.moe_plan_and_dispatch_begin(p, ids_d, plan)
    moe.moe_plan_and_dispatch_end(p, ids_d, plan, x_d, payload, None)
    moe.moe_combine(p, plan, payload, torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    pl = oracle.plan(ids, e, ep, 1, n * min(k, e // ep), h)
    assert plan.read_status() == pl["status"] == 0
    for key in ("expert_counts", "expert_offsets", "dest_counts", "slot", "packed_src"):
        assert np.array_equal(getattr(plan, key).cpu().numpy(), pl[key]), key
    rows = np.unique(np.concatenate([np.arange(8), r_max - 1 - np.arange(64),
                                     rng.choice(r_max, 4024, replace=False)]))
    got = u16(payload[torch.from_numpy(rows).cuda()])
    enc, _ = oracle.encode_rows("bf16", x[pl["packed_src"][rows]])
    assert np.array_equal(got, enc)
    negz = x_d.view(torch.int16) == -32768  # -0 comes back as +0
    same = (out.view(torch.int16) == x_d.view(torch.int16)) | (negz & (out.view(torch.int16) == 0))
    assert bool(same.all())
