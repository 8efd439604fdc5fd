"""Exhaustive checks of the blockwise-FP8 device path on the GPU.

The dispatch kernel replaces the correctly rounded quotient x / s by a
reciprocal with one fused correction (for block maxima >= 2^-103) and the
software E4M3 rounding by gfx950's conversion instruction.  These tests run
test-support kernels (tests/kernels/fp8_path_check.hip, compiled against the
library's own device header) over every input those shortcuts can meet:
every (block maximum, value) pair of bf16 numbers, and every fp32 value below
the E4M3 saturation midpoint.  The end-to-end FP8 parity against the CPU
oracle is in test_gpu_parity.py.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from conftest import ROOT

pytestmark = pytest.mark.gpu

LIB = os.path.join(ROOT, "tests", "kernels", "libfp8_path_check.so")


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe  # noqa: F401  (HIP runtime through torch)
    assert os.path.exists(LIB), f"{LIB} is not built (run __graft_entry__.build())"
    h = ctypes.CDLL(LIB)
    for fn in (h.fp8_quotient_check, h.fp8_convert_check, h.fp4_convert_check):
        fn.argtypes = [ctypes.c_void_p] * 3
        fn.restype = ctypes.c_int
    return h


def run(fn):
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda")
    rec = torch.zeros(24, dtype=torch.int32, device="cuda")
    assert fn(cnt.data_ptr(), rec.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    r = rec.cpu().numpy().view(np.uint32).reshape(8, 3)
    return int(c[0]), int(c[1]), [[hex(v) for v in row] for row in r[:min(int(c[2]), 8)]]


def test_fast_quotient_codes_match_ieee_division(lib):
    tested, bad, examples = run(lib.fp8_quotient_check)
    print(f"[fp8] (block max, value) bf16 pairs tested: {tested}, mismatches: {bad}", flush=True)
    assert tested == 1065402238  # all pairs |x| <= amax, amax in (0, max finite]
    assert bad == 0, examples


def test_hw_e4m3_conversion_matches_software_rule(lib):
    tested, bad, examples = run(lib.fp8_convert_check)
    print(f"[fp8] fp32 values |v| < 464 tested: {tested}, mismatches: {bad}", flush=True)
    assert tested == 2278555648
    assert bad == 0, examples


def test_hw_e2m1_conversion_matches_software_rule(lib):
    """gfx950's packed E2M1 conversion against the software rule, for every
    fp32 bit pattern but NaN (and its negation) in each destination byte; a
    NaN saturates to +-6 in hardware (the library's encoders take the
    software rule for a wave that holds one)."""
    cnt = torch.zeros(4, dtype=torch.int64, device="cuda")
    rec = torch.zeros(24, dtype=torch.int32, device="cuda")
    assert lib.fp4_convert_check(cnt.data_ptr(), rec.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    tested, bad, nrec, nan_other = (int(v) for v in cnt.cpu().numpy())
    recs = rec.cpu().numpy().view(np.uint32).reshape(8, 3)[:min(nrec, 8)]
    print(f"[fp4] fp32 values tested: {tested}, mismatches: {bad}", flush=True)
    assert tested == (1 << 32) - 2 * ((1 << 23) - 1)   # every pattern but the NaNs
    assert bad == 0, [[hex(v) for v in row] for row in recs]
    assert nan_other == 0
