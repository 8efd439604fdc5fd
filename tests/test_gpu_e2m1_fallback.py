"""The E2M1 encoders' software rule, end to end on the GPU.

The MX-FP4 and NVFP4 encoders convert their quotients with gfx950's E2M1
instruction.  It equals the software rule (round to nearest even, saturate at
6) on every fp32 input but NaN, which it saturates to +-6, so a wave whose
block maxima hold a NaN (or whose gate is not finite) encodes all of its
blocks with the software rule instead.  Non-finite inputs are outside the
contract, but the finite blocks of such a wave are not: here some waves get
one NaN, other blocks hold exact E2M1 rounding ties, and every finite block
of every packed row (codes and scale) must equal the oracle's encoding of its
token.  Blocks are independent (one scale per 32 or 16 values), so a NaN
block does not change the oracle's encoding of its neighbours.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_topk_ids_amd.workloads import random_bf16, random_routing
from gpu_helpers import say, to_dev_bf16

pytestmark = pytest.mark.gpu

N, H, E, K, EP = 96, 7168, 8, 2, 2
SLAB = 512          # values a dispatch wave encodes
NAN = 0x7FC0
# bf16 patterns of E2M1 midpoints under a block maximum of 6 (scale exponent
# 0 for MX; for NVFP4 under gs = 1 the scale is E4M3(1.0), also exact)
TIES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def inputs(block):
    """Hidden rows with NaNs in some waves' slabs and tie blocks in others,
    and a mask of the blocks that hold a NaN."""
    rng = np.random.default_rng(31)
    x = random_bf16(rng, (N, H))
    nb = H // block
    # tie blocks: a 6 (block maximum) and midpoints with random signs
    for t in range(N):
        for b in rng.choice(nb, 24, replace=False):
            v = rng.choice(TIES, block) * rng.choice([-1.0, 1.0], block)
            v[rng.integers(block)] = 6.0
            x[t, b * block:(b + 1) * block] = bf16_bits(v)
    nan_block = np.zeros((N, nb), bool)
    for t in range(0, N, 2):          # every other token: NaNs in a third of its slabs
        for s in range(H // SLAB):
            if (t + s) % 3 == 0:
                c = s * SLAB + int(rng.integers(SLAB))
                x[t, c] = NAN
                nan_block[t, c // block] = True
    ids, w = random_routing(rng, N, E, K)
    return x, ids, w, nan_block


def compare_finite_blocks(got_pay, got_sc, exp_pay, exp_sc, nan_block, block):
    """Rows [M, bytes]: codes (block/2 bytes a block) and scales (one byte or
    none per block) of every block outside nan_block."""
    cb = block // 2
    ok = ~nan_block
    gp = got_pay.reshape(got_pay.shape[0], -1, cb)
    ep = exp_pay.reshape(exp_pay.shape[0], -1, cb)
    diff = np.any(gp != ep, axis=2) & ok
    assert not diff.any(), f"codes differ in (row, block) {np.argwhere(diff)[:8].tolist()}"
    gs = got_sc.reshape(got_sc.shape[0], -1)
    es = exp_sc.reshape(exp_sc.shape[0], -1)
    diff = (gs != es) & ok
    assert not diff.any(), f"scales differ in (row, block) {np.argwhere(diff)[:8].tolist()}"


def dispatch(moe, fmt, x, ids, w=None, one_launch=False):
    p = moe.problem(N, H, K, E, EP, fmt=fmt)
    plan = moe.alloc_plan(p)
    payload, scales = moe.alloc_payload(p)
    ids_d, x_d = torch.from_numpy(ids).cuda(), to_dev_bf16(x)
    gs = torch.tensor([1.0], dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    w_d = None if w is None else torch.from_numpy(w).cuda()
    if one_launch:
        moe.moe_plan_and_dispatch(p, ids_d, plan, x_d, payload, scales, topk_weights=w_d,
                                  input_scale=gs)
    else:
        moe.moe_dispatch_plan(p, ids_d, plan)
        if fmt == "nvfp4":
            moe.moe_dispatch_scaled(p, plan, x_d, gs, payload, scales)
        elif w is not None:
            moe.moe_dispatch_gated(p, plan, x_d, w_d, payload, scales)
        else:
            moe.moe_dispatch(p, plan, x_d, payload, scales)
    torch.cuda.synchronize()
    return (plan.slot.cpu().numpy(), payload.view(torch.uint8).cpu().numpy(),
            scales.view(torch.uint8).cpu().numpy())


@pytest.mark.parametrize("one_launch", [False, True], ids=["three_calls", "one_launch"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_finite_blocks_of_nan_waves(moe, fmt, one_launch):
    block = 32 if fmt == "mxfp4" else 16
    say(f"[e2m1 fallback] {fmt} one_launch={one_launch}")
    x, ids, _, nan_block = inputs(block)
    if fmt == "mxfp4":
        enc, enc_sc = oracle.encode_rows("mxfp4", x)
    else:
        enc, enc_sc = oracle.encode_rows_nvfp4(x, 1.0)
    slot, pay, sc = dispatch(moe, fmt, x, ids, one_launch=one_launch)
    rows = slot.reshape(-1)
    tok = np.repeat(np.arange(N), K)
    live = rows >= 0
    assert live.all()
    compare_finite_blocks(pay[rows], sc[rows], enc.view(np.uint8)[tok], enc_sc.view(np.uint8)[tok],
                          nan_block[tok], block)
    # the NaN waves took the software rule: they exist, and hold ties
    assert nan_block.any(axis=1).sum() == N // 2


@pytest.mark.parametrize("one_launch", [False, True], ids=["three_calls", "one_launch"])
def test_finite_blocks_of_nan_waves_gated(moe, one_launch):
    """Gated MX-FP4: each copy encodes fl32(w * x) on its own."""
    say(f"[e2m1 fallback] gated mxfp4 one_launch={one_launch}")
    x, ids, w, nan_block = inputs(32)
    slot, pay, sc = dispatch(moe, "mxfp4", x, ids, w=w, one_launch=one_launch)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    rows = slot.reshape(-1)
    tok = np.repeat(np.arange(N), K)
    v = (w.reshape(-1)[:, None] * xf[tok]).astype(np.float32)  # one fp32 product a value
    with np.errstate(invalid="ignore"):
        enc, enc_sc = oracle.encode_rows_f32("mxfp4", v)
    compare_finite_blocks(pay[rows], sc[rows], enc.view(np.uint8), enc_sc.view(np.uint8),
                          nan_block[tok], 32)
