"""The C-ABI library loads, exports every symbol include/moe.h declares, and
validates arguments on the host (no GPU work: every call here returns before
anything is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def moe():
    from combine_topk_ids_amd import _build
    if not os.path.exists(_build.LIB):
        _build.build(force=False)
    import combine_topk_ids_amd.moe as m
    return m


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports(moe):
    assert declared_symbols() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol(moe):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(moe_\w+)$", out, re.M))
    assert set(declared_symbols()) <= exported
    # nothing else leaks out of the library's namespace
    assert exported == set(declared_symbols())


def test_sizes_match_the_closed_form(moe):
    import oracle
    for (n, h, k, e, ep, a, fmt) in [(128, 256, 2, 8, 4, 1, "bf16"),
                                     (4096, 4096, 6, 64, 8, 128, "bf16"),
                                     (8192, 7168, 8, 256, 32, 1, "fp8"),
                                     (16384, 4096, 8, 128, 16, 128, "bf16"),
                                     (128, 7168, 8, 256, 8, 1, "mxfp4"),
                                     (0, 64, 3, 5, 5, 7, "bf16")]:
        p = moe.problem(n, h, k, e, ep, pad_multiple=a, fmt=fmt)
        assert moe.moe_check_problem(p) == 0
        assert moe.moe_max_rows(p) == oracle.max_rows(n, k, e, a)
        pb = {"bf16": 2 * h, "fp8": h, "mxfp4": h // 2}[fmt]
        sb = {"bf16": 0, "fp8": 4 * (h // 128), "mxfp4": h // 32}[fmt]
        assert moe.moe_payload_row_bytes(p) == pb
        assert moe.moe_scale_row_bytes(p) == sb
        assert moe.moe_workspace_bytes(p) % 256 == 0


@pytest.mark.parametrize("field,value,code", [
    ("n_tokens", -1, -1), ("hidden", 0, -1), ("hidden", 12, -1), ("top_k", 0, -1),
    ("top_k", 9, -1), ("n_experts", 0, -1), ("n_experts", 1025, -1), ("ep", 3, -1),
    ("ep", 0, -1), ("pad_multiple", 0, -1), ("recv_capacity", -5, -1), ("fmt", 4, -1),
    ("flags", 2, -1), ("n_tokens", 1 << 30, -3),
])
def test_invalid_problems_rejected(moe, field, value, code):
    p = moe.problem(64, 256, 2, 8, 4)
    setattr(p, field, value)
    assert moe.moe_check_problem(p) == code
    assert moe.lib.moe_max_rows(ctypes.byref(p)) == code
    pl = moe.Plan()
    assert moe.lib.moe_dispatch_plan(ctypes.byref(p), None, ctypes.byref(pl), None, None) == code
    assert moe.lib.moe_dispatch(ctypes.byref(p), ctypes.byref(pl), None, None, None, None) == code
    assert moe.lib.moe_combine(ctypes.byref(p), ctypes.byref(pl), None, None, None, None) == code


def test_format_divisibility(moe):
    assert moe.moe_check_problem(moe.problem(4, 64, 1, 2, 1, fmt="fp8")) == -1
    assert moe.moe_check_problem(moe.problem(4, 128, 1, 2, 1, fmt="fp8")) == 0
    assert moe.moe_check_problem(moe.problem(4, 48, 1, 2, 1, fmt="mxfp4")) == -1
    assert moe.moe_check_problem(moe.problem(4, 96, 1, 2, 1, fmt="mxfp4")) == 0


def test_element_overflow_rejected(moe):
    # R_max * H must stay below 2^32 for the uint32 element table
    p = moe.problem(70000, 8192, 8, 64, 8)
    assert moe.moe_check_problem(p) == -3


def test_null_and_misaligned_pointers_rejected(moe):
    p = moe.problem(64, 256, 2, 8, 4)
    fake = 1 << 20  # never dereferenced: every call below fails its checks first
    full = moe.Plan(*([fake] * 7))
    # a null plan field
    part = moe.Plan(*([fake] * 6 + [0]))
    assert moe.lib.moe_dispatch_plan(ctypes.byref(p), fake, ctypes.byref(part), None, None) == -1
    # null ids with N*k > 0
    assert moe.lib.moe_dispatch_plan(ctypes.byref(p), None, ctypes.byref(full), None, None) == -1
    # misaligned ids
    assert moe.lib.moe_dispatch_plan(ctypes.byref(p), fake + 2, ctypes.byref(full), None, None) == -2
    # scales given for bf16, missing for fp8
    assert moe.lib.moe_dispatch(ctypes.byref(p), ctypes.byref(full), fake, fake, fake, None) == -1
    p8 = moe.problem(64, 256, 2, 8, 4, fmt="fp8")
    assert moe.lib.moe_dispatch(ctypes.byref(p8), ctypes.byref(full), fake, fake, None, None) == -1
    # rows must be 16-byte aligned
    assert moe.lib.moe_dispatch(ctypes.byref(p), ctypes.byref(full), fake + 8, fake, None, None) == -2
    assert moe.lib.moe_combine(ctypes.byref(p), ctypes.byref(full), fake, fake, fake + 4, None) == -2
    assert moe.lib.moe_combine(ctypes.byref(p), ctypes.byref(full), None, fake, fake, None) == -1


def test_plan_and_dispatch_rejections(moe):
    """Every call below fails its checks before anything is launched."""
    ref = ctypes.byref
    fake = 1 << 20
    full = moe.Plan(*([fake] * 7))
    p = moe.problem(64, 256, 2, 8, 4)
    call = moe.lib.moe_plan_and_dispatch
    # a global scale only with NVFP4, where it is required and gates are not
    assert call(ref(p), fake, ref(full), fake, None, fake, fake, None, None, None) == -1
    pn = moe.problem(64, 256, 2, 8, 4, fmt="nvfp4")
    assert call(ref(pn), fake, ref(full), fake, None, None, fake, fake, None, None) == -1
    assert call(ref(pn), fake, ref(full), fake, fake, fake, fake, fake, None, None) == -1
    # null plan field, null ids, null hidden, scales for bf16
    part = moe.Plan(*([fake] * 6 + [0]))
    assert call(ref(p), fake, ref(part), fake, None, None, fake, None, None, None) == -1
    assert call(ref(p), None, ref(full), fake, None, None, fake, None, None, None) == -1
    assert call(ref(p), fake, ref(full), None, None, None, fake, None, None, None) == -1
    assert call(ref(p), fake, ref(full), fake, None, None, fake, fake, None, None) == -1
    # misaligned rows, IDs and gates
    assert call(ref(p), fake, ref(full), fake + 8, None, None, fake, None, None, None) == -2
    assert call(ref(p), fake + 2, ref(full), fake, None, None, fake, None, None, None) == -2
    assert call(ref(p), fake, ref(full), fake, fake + 2, None, fake, None, None, None) == -2
    # a problem past one launch needs the plan workspace
    big = moe.problem(16384, 4096, 8, 128, 16, pad_multiple=128)
    assert call(ref(big), fake, ref(full), fake, None, None, fake, None, None, None) == -1


def test_plan_and_dispatch_halves_reject_as_the_whole(moe):
    """_begin checks the plan's arguments, _end those of the whole call; each
    call below fails before anything is launched."""
    ref = ctypes.byref
    fake = 1 << 20
    full = moe.Plan(*([fake] * 7))
    part = moe.Plan(*([fake] * 6 + [0]))
    p = moe.problem(64, 256, 2, 8, 4)
    big = moe.problem(4096, 4096, 6, 64, 8)  # tiled: needs the workspace
    begin, end = moe.lib.moe_plan_and_dispatch_begin, moe.lib.moe_plan_and_dispatch_end
    assert begin(None, fake, ref(full), None, None) == -1
    assert begin(ref(p), fake, ref(part), None, None) == -1
    assert begin(ref(p), None, ref(full), None, None) == -1
    assert begin(ref(p), fake + 2, ref(full), None, None) == -2
    assert begin(ref(big), fake, ref(full), None, None) == -1
    assert begin(ref(big), fake, ref(full), fake + 64, None) == -2
    # end: the plan's checks, then the dispatch's
    assert end(ref(p), fake, ref(part), fake, None, None, fake, None, None, None) == -1
    assert end(ref(big), fake, ref(full), fake, None, None, fake, None, None, None) == -1
    assert end(ref(p), fake, ref(full), None, None, None, fake, None, None, None) == -1
    assert end(ref(p), fake, ref(full), fake, None, fake, fake, None, None, None) == -1
    assert end(ref(p), fake, ref(full), fake, None, None, fake, fake, None, None) == -1
    assert end(ref(p), fake, ref(full), fake + 8, None, None, fake, None, None, None) == -2
    pn = moe.problem(64, 256, 2, 8, 4, fmt="nvfp4")
    assert end(ref(pn), fake, ref(full), fake, None, None, fake, fake, None, None) == -1
    assert end(ref(pn), fake, ref(full), fake, fake, fake, fake, fake, None, None) == -1


def test_plan_and_dispatch_mode(moe):
    """One launch up to 2048 pairs; tiled while (count tiles of
    floor(2048 / k) tokens) x E <= 2048; the plan's kernels then the
    dispatch otherwise.  A fixed expert capacity takes the same modes."""
    one, tiled, sep = moe.PD_ONE_LAUNCH, moe.PD_TILED, moe.PD_SEPARATE
    mode = moe.moe_plan_and_dispatch_mode
    assert mode(moe.problem(0, 64, 2, 4, 2)) == one
    assert mode(moe.problem(256, 7168, 8, 256, 8)) == one             # 2048 pairs
    assert mode(moe.problem(257, 7168, 8, 256, 8)) == tiled           # 2 tiles x 256
    assert mode(moe.problem(4096, 4096, 6, 64, 8)) == tiled           # 13 tiles x 64
    assert mode(moe.problem(300, 256, 8, 1024, 64)) == tiled          # 2 x 1024 = 2048
    assert mode(moe.problem(513, 256, 8, 1024, 64)) == sep            # 3 x 1024
    assert mode(moe.problem(2048 * 8, 64, 1, 8, 2)) == tiled          # k = 1: 8 tiles x 8
    assert mode(moe.problem(8192, 7168, 8, 256, 8)) == sep            # 32 x 256
    assert mode(moe.problem(16384, 4096, 8, 128, 16)) == sep          # 64 x 128
    assert mode(moe.problem(100, 256, 4, 8, 2, expert_capacity=60)) == one
    assert mode(moe.problem(4096, 4096, 6, 64, 8, expert_capacity=384)) == tiled
    assert mode(moe.problem(8192, 7168, 8, 256, 8, expert_capacity=320)) == sep
    bad = moe.problem(64, 256, 2, 8, 4)
    bad.hidden = 7
    assert moe.lib.moe_plan_and_dispatch_mode(ctypes.byref(bad)) == -1


def test_workspace_required_only_for_multi_tile_plans(moe):
    small = moe.problem(128, 7168, 8, 256, 8)          # 1024 pairs: one block
    big = moe.problem(16384, 4096, 8, 128, 16, pad_multiple=128)
    assert moe.moe_workspace_bytes(small) == 0
    assert moe.moe_workspace_bytes(big) > 0
    full = moe.Plan(*([1 << 20] * 7))
    assert moe.lib.moe_dispatch_plan(ctypes.byref(big), 1 << 20, ctypes.byref(full), None, None) == -1


def test_strerror(moe):
    for c in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(moe.strerror(c), str) and moe.strerror(c)


# ---- exchange across EP simulated ranks --------------------------------------

def test_exchange_checks(moe):
    ok = moe.problem(4096, 4096, 6, 64, 8, recv_capacity=30720)
    assert moe.moe_check_exchange(ok) == 0
    assert moe.moe_exchange_workspace_bytes(ok) % 256 == 0
    assert moe.moe_exchange_workspace_bytes(ok) > 0
    # source-major receive buffers carry no per-expert padding
    assert moe.moe_check_exchange(moe.problem(64, 256, 2, 8, 4, recv_capacity=64,
                                              pad_multiple=2)) == -1
    # EP * C receive rows must fit int32
    assert moe.moe_check_exchange(moe.problem(64, 256, 2, 8, 4, recv_capacity=1 << 30)) == -3
    # EP * N * k * H must fit the uint32 element table
    assert moe.moe_check_exchange(moe.problem(16384, 4096, 8, 64, 8, recv_capacity=1)) == -3
    # a problem the single-rank checks reject is rejected here too
    bad = moe.problem(64, 12, 2, 8, 4, recv_capacity=8)
    assert moe.moe_check_exchange(bad) == -1
    assert moe.moe_exchange_workspace_bytes(bad) == 0
    x = moe.Exchange()
    for p, code in ((bad, -1), (moe.problem(64, 256, 2, 8, 4, recv_capacity=8, pad_multiple=3), -1)):
        assert moe.lib.moe_exchange_plan(ctypes.byref(p), None, ctypes.byref(x), None, None) == code
        assert moe.lib.moe_exchange_dispatch(ctypes.byref(p), ctypes.byref(x), None, None, None,
                                             None) == code
        assert moe.lib.moe_exchange_combine(ctypes.byref(p), ctypes.byref(x), None, None, None,
                                            None) == code


def test_exchange_null_and_misaligned_pointers_rejected(moe):
    p = moe.problem(64, 256, 2, 8, 4, recv_capacity=64)
    fake = 1 << 20
    full = moe.Exchange(*([fake] * 8))
    part = moe.Exchange(*([fake] * 7 + [0]))  # no status array
    ref = ctypes.byref
    assert moe.lib.moe_exchange_plan(ref(p), fake, ref(part), fake, None) == -1
    assert moe.lib.moe_exchange_plan(ref(p), fake, ref(full), None, None) == -1   # no workspace
    assert moe.lib.moe_exchange_plan(ref(p), None, ref(full), fake, None) == -1   # no ids
    assert moe.lib.moe_exchange_plan(ref(p), fake, ref(full), fake + 64, None) == -2
    assert moe.lib.moe_exchange_plan(ref(p), fake + 1, ref(full), fake, None) == -2
    assert moe.lib.moe_exchange_dispatch(ref(p), ref(full), fake, fake, fake, None) == -1
    assert moe.lib.moe_exchange_dispatch(ref(p), ref(full), fake + 8, fake, None, None) == -2
    p8 = moe.problem(64, 256, 2, 8, 4, recv_capacity=64, fmt="fp8")
    assert moe.lib.moe_exchange_dispatch(ref(p8), ref(full), fake, fake, None, None) == -1
    assert moe.lib.moe_exchange_combine(ref(p), ref(full), fake, fake, fake + 2, None) == -2
    assert moe.lib.moe_exchange_combine(ref(p), ref(full), None, fake, fake, None) == -1


# ---- gates at dispatch, dense routing map -------------------------------------

def test_gated_and_map_entry_points_check_arguments(moe):
    ref = ctypes.byref
    fake = 1 << 20
    p = moe.problem(64, 256, 2, 8, 4)
    full = moe.Plan(*([fake] * 7))
    # gates are required by the gated dispatch (and only there)
    assert moe.lib.moe_dispatch_gated(ref(p), ref(full), fake, None, fake, None, None) == -1
    assert moe.lib.moe_dispatch_gated(ref(p), ref(full), fake, fake + 2, fake, None, None) == -2
    assert moe.lib.moe_dispatch_gated(ref(p), ref(full), fake, fake, fake, fake, None) == -1
    bad = moe.problem(64, 12, 2, 8, 4)
    assert moe.lib.moe_dispatch_gated(ref(bad), ref(full), fake, fake, fake, None, None) == -1
    px = moe.problem(64, 256, 2, 8, 4, recv_capacity=64)
    fx = moe.Exchange(*([fake] * 8))
    assert moe.lib.moe_exchange_dispatch_gated(ref(px), ref(fx), fake, None, fake, None, None) == -1
    assert moe.lib.moe_exchange_dispatch_gated(ref(px), ref(fx), fake, fake + 1, fake, None, None) == -2
    # routing map
    assert moe.moe_map_workspace_bytes(p) % 256 == 0 and moe.moe_map_workspace_bytes(p) > 0
    assert moe.moe_map_workspace_bytes(moe.problem(0, 256, 2, 8, 4)) == 0
    assert moe.lib.moe_routing_map_to_topk(ref(p), fake, None, fake, None, None, fake, None) == -1
    assert moe.lib.moe_routing_map_to_topk(ref(p), None, None, fake, None, fake, fake, None) == -1
    assert moe.lib.moe_routing_map_to_topk(ref(p), fake, None, fake, None, fake, None, None) == -1
    assert moe.lib.moe_routing_map_to_topk(ref(p), fake, fake + 2, fake, None, fake, fake, None) == -2
    assert moe.lib.moe_routing_map_to_topk(ref(p), fake, None, fake, None, fake, fake + 16, None) == -2
    assert moe.lib.moe_routing_map_to_topk(ref(bad), fake, None, fake, None, fake, fake, None) == -1


# ---- fixed expert capacity ------------------------------------------------------

def test_expert_capacity_sizes_and_checks(moe):
    import oracle
    for n, k, e, cf in [(4096, 6, 64, 1.25), (10, 3, 4, 0.5), (100, 1, 1, 0.0), (7, 2, 5, 2.0)]:
        assert moe.moe_expert_capacity(n, k, e, cf) == oracle.expert_capacity(n, k, e, cf)
    assert moe.lib.moe_expert_capacity(10, 0, 4, 1.0) == -1
    assert moe.lib.moe_expert_capacity(10, 2, 4, -1.0) == -1
    assert moe.lib.moe_expert_capacity(1 << 40, 64, 1, 1.0) == -3
    p = moe.problem(4096, 4096, 6, 64, 8, expert_capacity=480)
    assert moe.moe_check_problem(p) == 0
    assert moe.moe_max_rows(p) == 64 * 480
    # a fixed capacity replaces per-expert padding
    assert moe.moe_check_problem(moe.problem(64, 256, 2, 8, 4, pad_multiple=2,
                                             expert_capacity=8)) == -1
    assert moe.moe_check_problem(moe.problem(64, 256, 2, 8, 4, expert_capacity=-1)) == -1
    # E*cap + N*k must fit int32
    assert moe.moe_check_problem(moe.problem(64, 8, 2, 1024, 4, expert_capacity=1 << 21)) == -3
    # no fixed capacity in the exchange
    assert moe.moe_check_exchange(moe.problem(64, 256, 2, 8, 4, recv_capacity=64,
                                              expert_capacity=8)) == -1


# ---- NVFP4 ------------------------------------------------------------------------

def test_nvfp4_sizes_and_entry_points(moe):
    ref = ctypes.byref
    fake = 1 << 20
    p = moe.problem(64, 256, 2, 8, 4, fmt="nvfp4")
    assert moe.moe_check_problem(p) == 0
    assert moe.moe_payload_row_bytes(p) == 128 and moe.moe_scale_row_bytes(p) == 16
    assert moe.moe_check_problem(moe.problem(64, 48, 2, 8, 4, fmt="nvfp4")) == -1  # H % 32
    full = moe.Plan(*([fake] * 7))
    # the plain and gated dispatches cannot carry the global scale
    assert moe.lib.moe_dispatch(ref(p), ref(full), fake, fake, fake, None) == -1
    assert moe.lib.moe_dispatch_gated(ref(p), ref(full), fake, fake, fake, fake, None) == -1
    # the scaled dispatch needs NVFP4, the scale pointer and the scale rows
    assert moe.lib.moe_dispatch_scaled(ref(p), ref(full), fake, None, fake, fake, None) == -1
    assert moe.lib.moe_dispatch_scaled(ref(p), ref(full), fake, fake, fake, None, None) == -1
    assert moe.lib.moe_dispatch_scaled(ref(p), ref(full), fake, fake + 2, fake, fake, None) == -2
    pb = moe.problem(64, 256, 2, 8, 4)
    assert moe.lib.moe_dispatch_scaled(ref(pb), ref(full), fake, fake, fake, None, None) == -1
    px = moe.problem(64, 256, 2, 8, 4, recv_capacity=64, fmt="nvfp4")
    fx = moe.Exchange(*([fake] * 8))
    assert moe.lib.moe_exchange_dispatch(ref(px), ref(fx), fake, fake, fake, None) == -1
    assert moe.lib.moe_exchange_dispatch_scaled(ref(px), ref(fx), fake, None, fake, fake, None) == -1
    assert moe.lib.moe_exchange_dispatch_scaled(ref(px), ref(fx), fake, fake, fake, None, None) == -1


def test_noalloc_refuses_a_problem_past_its_scratch(moe):
    """moe_plan_and_dispatch_noalloc returns MOE_ESCRATCH, before any launch,
    for a problem whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES (E = 1024
    and 274 count tiles: 274 * 1025 * 4 bytes), and rejects an invalid
    problem as every entry point does."""
    p = moe.problem(70000, 64, 8, 1024, 8)
    assert moe.moe_workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the size check fails first
    plan = moe.Plan(*([fake] * 7))
    call = moe.lib.moe_plan_and_dispatch_noalloc
    rc = call(ctypes.byref(p), fake, ctypes.byref(plan), fake, None, None, fake, None, None)
    assert rc == moe.MOE_ESCRATCH == -5
    assert "scratch" in moe.strerror(rc)
    bad = moe.problem(64, 12, 2, 8, 4)
    assert call(ctypes.byref(bad), fake, ctypes.byref(plan), fake, None, None, fake, None,
                None) == moe.MOE_EINVAL
