"""Host-side checks of bench.py: the algorithmic byte counts it divides by
the measured time, the row sizes of each format, and the one-GPU guard.

The byte formulas follow the hot-path measurement definition: the plan
reads the IDs and writes slot and packed_src; the dispatch reads every token
row once and writes every packed row in use; the combine reads slot,
weights, one expert row per kept pair and writes the output.  The expected
values are worked out by hand from the workload sizes below.
"""
import os
import subprocess
import sys

import bench
from combine_topk_ids_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_row_bytes_per_format():
    h = 7168
    assert bench.row_bytes("bf16", h) == 14336
    assert bench.row_bytes("fp8", h) == 7168 + 56 * 4      # codes + one fp32 per 128
    assert bench.row_bytes("mxfp4", h) == 3584 + 224       # nibbles + one byte per 32
    assert bench.row_bytes("nvfp4", h) == 3584 + 448       # nibbles + one byte per 16


def test_uniform_step_bytes():
    """N=4096, H=4096, k=6, E=64, A=128: R_used = 28,928, R_max = 32,704."""
    w = WORKLOADS["uniform_bf16_n4096"]
    b = bench.step_bytes(w, 28928, 32704)
    nk = 4096 * 6
    assert b["plan"] == 4 * nk + 4 * nk + 4 * 32704 == 327424
    assert b["dispatch"] == 2 * 4096 * 4096 + 28928 * 8192 == 270532608
    assert b["combine"] == 8 * nk + 2 * 4096 * nk + 2 * 4096 * 4096 == 235077632
    assert b["total"] == b["plan"] + b["dispatch"] + b["combine"]


def test_fp8_step_bytes():
    """N=8192, H=7168, k=8, E=256, A=1: every packed row is live."""
    w = WORKLOADS["fp8_b128_n8192"]
    nk = 8192 * 8
    b = bench.step_bytes(w, nk, nk)
    assert b["dispatch"] == 2 * 8192 * 7168 + nk * 7392
    assert b["combine"] == 8 * nk + 2 * 7168 * nk + 2 * 8192 * 7168


def test_exchange_and_capacity_step_bytes():
    """Exchange: every receive row is written (live, then zero rows), the
    combine reads the kept rows.  Fixed capacity: E*cap rows written, the
    combine reads the kept pairs."""
    w = WORKLOADS["exchange_bf16_ep8_n4096"]
    rows = w.ep * w.capacity
    b = bench.step_bytes(w, 100000, rows)
    t, nk = w.tokens, w.tokens * w.k
    assert b["dispatch"] == 2 * t * w.h + rows * 2 * w.h
    assert b["combine"] == 8 * nk + 2 * w.h * 100000 + 2 * t * w.h
    c = WORKLOADS["capacity_bf16_n4096"]
    b = bench.step_bytes(c, 384 * c.e, 384 * c.e, kept=24077)
    assert b["dispatch"] == 2 * c.n * c.h + 384 * c.e * 2 * c.h
    assert b["combine"] == 8 * c.n * c.k + 2 * c.h * 24077 + 2 * c.n * c.h


def test_buffer_rows():
    w = WORKLOADS["uniform_bf16_n4096"]
    assert bench.buffer_rows(w) == 4096 * 6 + 64 * 127
    assert bench.buffer_rows(w, expert_cap=384) == 64 * 384
    x = WORKLOADS["exchange_bf16_ep8_n4096"]
    assert bench.buffer_rows(x) == x.ep * x.capacity


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_paths_name_their_dispatch_kernel():
    """The roofline names the kernel of the dispatch call on either path."""
    for cls in (bench.Path, bench.ExchangePath):
        assert callable(getattr(cls, "dispatch_kernel", None)), cls.__name__


def test_gated_map_step_bytes():
    """Gates at dispatch, routing given as a dense map (N=4096, E=64, k=6,
    A=128): the plan also reads the map (N*E bytes) and the kept
    probabilities and writes IDs and gates; the dispatch reads the gates;
    the combine reads no weights."""
    w = WORKLOADS["gated_map_bf16_n4096"]
    b = bench.step_bytes(w, 28928, 32704)
    nk = 4096 * 6
    assert b["plan"] == 4 * nk + 4 * nk + 4 * 32704 + 4096 * 64 + 3 * 4 * nk
    assert b["dispatch"] == 2 * 4096 * 4096 + 28928 * 8192 + 4 * nk
    assert b["combine"] == 4 * nk + 2 * 4096 * nk + 2 * 4096 * 4096
