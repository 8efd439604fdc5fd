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


def assert_rows_are_tokens(got_pay, got_sc, enc, enc_sc, src, chunk=4096):
    """Every packed row r against the oracle in gather form: row r holds the
    oracle's encoding of token src[r] (each token encoded once, enc[t] /
    enc_sc[t]), or zero bytes where src[r] < 0.  got_pay / got_sc: uint8
    [rows, row bytes]; enc / enc_sc: the oracle's rows of every token, any
    dtype (compared as bytes)."""
    enc = enc.view(np.uint8).reshape(enc.shape[0], -1)
    enc_sc = None if enc_sc is None else enc_sc.view(np.uint8).reshape(enc_sc.shape[0], -1)
    rows = got_pay.shape[0]
    assert src.shape[0] == rows
    for r0 in range(0, rows, chunk):
        s = src[r0:r0 + chunk]
        live = s >= 0
        gp = got_pay[r0:r0 + chunk]
        bad = np.nonzero(np.any(gp[live] != enc[s[live]], axis=1))[0]
        assert bad.size == 0, f"payload rows {(r0 + np.nonzero(live)[0][bad])[:8]} differ"
        assert not np.any(gp[~live]), f"zero rows in {r0}..{r0 + chunk} are not zero"
        if enc_sc is not None:
            gs = got_sc[r0:r0 + chunk]
            bad = np.nonzero(np.any(gs[live] != enc_sc[s[live]], axis=1))[0]
            assert bad.size == 0, f"scale rows {(r0 + np.nonzero(live)[0][bad])[:8]} differ"
            assert not np.any(gs[~live]), f"zero scale rows in {r0}..{r0 + chunk} are not zero"
