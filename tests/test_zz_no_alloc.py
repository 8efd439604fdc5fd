"""GPU: moe_plan_and_dispatch_noalloc (the plan's workspace in the library's
static device scratch) against moe_plan_and_dispatch with a caller
workspace, byte for byte, on two calls in a row, the second with a smaller
problem.  (Its refusal of a problem past the scratch is a host check, in
test_abi.py.)"""
import numpy as np
import pytest
import torch

from combine_topk_ids_amd.workloads import random_bf16, random_routing
from gpu_helpers import SENTINEL, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


def _outputs(moe, p, ids, x, gates, gs, noalloc):
    plan = moe.alloc_plan(p)
    for t in (plan.expert_counts, plan.expert_offsets, plan.dest_counts, plan.rank_table,
              plan.slot, plan.packed_src, plan.status):
        t.fill_(-7)
    payload, scales = moe.alloc_payload(p)
    payload.view(torch.uint8).fill_(SENTINEL)
    if scales is not None:
        scales.view(torch.uint8).fill_(SENTINEL)
    if noalloc:
        moe.moe_plan_and_dispatch_noalloc(p, ids, plan, x, payload, scales, topk_weights=gates,
                                          input_scale=gs)
    else:
        moe.moe_plan_and_dispatch(p, ids, plan, x, payload, scales, topk_weights=gates,
                                  input_scale=gs)
    torch.cuda.synchronize()
    out = [plan.expert_counts, plan.expert_offsets, plan.dest_counts, plan.rank_table, plan.slot,
           plan.packed_src, plan.status, payload]
    if scales is not None:
        out.append(scales)
    return [t.view(torch.uint8).cpu().numpy() for t in out]


# (N, H, E, k, EP, A, format, gated): a problem of 64 count tiles (its plan's
# kernels, then the dispatch), then a smaller tiled one (the counting kernel,
# then one launch) that reuses the scratch the first call left behind
CALLS = [
    (16384, 512, 128, 8, 16, 128, "bf16", False),
    (3000, 1024, 16, 4, 4, 8, "fp8", True),
]


def test_noalloc_matches_the_workspace_call_twice(moe):
    for i, (n, h, e, k, ep, a, fmt, gated) in enumerate(CALLS):
        p = moe.problem(n, h, k, e, ep, pad_multiple=a, fmt=fmt)
        mode = moe.moe_plan_and_dispatch_mode(p)
        ws = moe.moe_workspace_bytes(p)
        say(f"[noalloc] call {i}: N={n} H={h} E={e} k={k} EP={ep} A={a} {fmt} gated={gated} "
            f"mode={mode} workspace={ws} B")
        assert 0 < ws <= moe.NOALLOC_SCRATCH_BYTES
        rng = np.random.default_rng(500 + i)
        ids_np, w_np = random_routing(rng, n, e, k, masked_frac=0.05)
        ids = torch.from_numpy(ids_np).cuda()
        x = to_dev_bf16(random_bf16(rng, (n, h)))
        gates = torch.from_numpy(w_np).cuda() if gated else None
        ref = _outputs(moe, p, ids, x, gates, None, noalloc=False)
        got = _outputs(moe, p, ids, x, gates, None, noalloc=True)
        for j, (a_, b_) in enumerate(zip(ref, got)):
            assert np.array_equal(a_, b_), (i, j)
        assert int(ref[6].view(np.uint32)[0]) == 0
