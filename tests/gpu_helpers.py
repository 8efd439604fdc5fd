"""Helpers shared by the GPU parity tests (no tests here)."""
import sys

import numpy as np
import torch

SENTINEL = 0x5A  # byte written into outputs before a run, to catch rows left unwritten


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def assert_combine_close(got, ref):
    """At most one bf16 ulp apart everywhere; returns how many differ at all."""
    g = got.astype(np.int32)
    r = ref.astype(np.int32)

    def ordered(v):  # sign-magnitude bits onto a line, so ulps subtract
        return np.where(v & 0x8000, -(v & 0x7FFF), v & 0x7FFF)
    d = np.abs(ordered(g) - ordered(r))
    assert d.max(initial=0) <= 1, f"max ulp diff {d.max()}"
    return int((d != 0).sum())
