"""Seeded synthetic inputs for MoE dispatch/combine.

This module only draws random inputs (router logits, the top-k choice and gate
weights a router would hand over, hidden rows, expert outputs).  It holds none
of the dispatch/combine arithmetic; both the HIP path and the CPU oracle take
its arrays as given.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, drawn in
this order):

1. router logits ``float32 [N, E]``: N(0, 1); for the skewed workload
   ``log p_e + 0.5 * N(0, 1)`` with ``p_e`` proportional to ``(e+1)^-1.2``
   (Zipf popularity, expert 0 most popular);
2. hidden ``[N, H]``: N(0, 1) in float32, rounded to bf16;
3. expert outputs ``[rows, H]`` (only workloads with non-identity experts):
   N(0, 1) in float32, rounded to bf16.

Workloads with ``ranks`` > 1 stand for that many simulated ranks holding N
tokens each; their logits, hidden rows and expert outputs are drawn the same
way for all ``ranks * N`` tokens at once (rank s owns tokens s*N .. s*N+N-1).

Top-k: the k largest logits per token, ties to the lower expert index, IDs in
descending-logit order.  Gate weights: softmax over all E logits in float64,
keep the top-k probabilities, renormalise them to sum 1, cast to float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int            # tokens
    h: int            # hidden size
    e: int            # experts
    k: int            # top-k
    ep: int           # simulated destination ranks
    a: int            # per-expert pad multiple
    fmt: str          # "bf16" | "fp8" | "mxfp4"
    routing: str      # "softmax" | "zipf"
    experts: str      # "identity" (expert output = dispatched rows) | "random"
    recv_capacity: int | None = None  # None: dropless (all tokens) * min(k, E/EP)
    ranks: int = 1    # simulated source ranks, N tokens each (exchange workloads: EP)
    capacity_factor: float | None = None  # fixed per-expert capacity from this factor
    input_scale: float = 1.0    # NVFP4 global encode scale handed to the dispatch
    gated: bool = False         # gates applied at dispatch, unweighted combine
    routing_input: str = "topk"  # "topk" | "map": dense multihot map + probabilities

    @property
    def l(self) -> int:
        return self.e // self.ep

    @property
    def tokens(self) -> int:
        """Tokens over all simulated source ranks."""
        return self.n * self.ranks

    @property
    def exchange(self) -> bool:
        return self.ranks > 1

    @property
    def capacity(self) -> int:
        if self.recv_capacity is not None:
            return self.recv_capacity
        return self.tokens * min(self.k, self.l)

    def describe(self) -> str:
        head = f"{self.ranks} ranks x " if self.exchange else ""
        tail = f", C={self.capacity} rows per receive buffer" if self.exchange else ""
        if self.capacity_factor is not None:
            tail += f", expert capacity factor {self.capacity_factor}"
        if self.gated:
            tail += ", gates applied at dispatch"
        if self.routing_input == "map":
            tail += ", routing given as a dense multihot map with dense probabilities"
        return (f"{head}N={self.n} H={self.h} E={self.e} k={self.k} EP={self.ep} "
                f"A={self.a} {self.fmt} {self.routing} routing, "
                f"{self.experts} experts{tail}")


WORKLOADS = {
    w.name: w
    for w in [
        # plumbing case
        Workload("tiny_bf16_n128", n=128, h=256, e=8, k=2, ep=4, a=1,
                 fmt="bf16", routing="softmax", experts="identity",
                 recv_capacity=256),
        # near-uniform prefill, 128-row expert alignment
        Workload("uniform_bf16_n4096", n=4096, h=4096, e=64, k=6, ep=8,
                 a=128, fmt="bf16", routing="softmax", experts="identity"),
        # blockwise FP8 dispatch, bf16 expert outputs
        Workload("fp8_b128_n8192", n=8192, h=7168, e=256, k=8, ep=32, a=1,
                 fmt="fp8", routing="softmax", experts="random"),
        # Zipf-skewed routing, 128-row padding
        Workload("zipf_bf16_n16384", n=16384, h=4096, e=128, k=8, ep=16,
                 a=128, fmt="bf16", routing="zipf", experts="identity"),
        # decode-sized MX-FP4 dispatch
        Workload("decode_mxfp4_n128", n=128, h=7168, e=256, k=8, ep=8, a=1,
                 fmt="mxfp4", routing="softmax", experts="random"),
        # NVFP4 dispatch (global encode scale 448 * 6 / 8: blocks of N(0,1)
        # rows keep their E4M3 scales below saturation for |x| up to 8)
        Workload("nvfp4_b16_n8192", n=8192, h=7168, e=256, k=8, ep=32, a=1,
                 fmt="nvfp4", routing="softmax", experts="random", input_scale=336.0),
        Workload("decode_nvfp4_n128", n=128, h=7168, e=256, k=8, ep=8, a=1,
                 fmt="nvfp4", routing="softmax", experts="random", input_scale=336.0),
        # fixed per-expert capacity (factor 1.0: experts above the mean drop)
        Workload("capacity_bf16_n4096", n=4096, h=4096, e=64, k=6, ep=8, a=1,
                 fmt="bf16", routing="softmax", experts="identity",
                 capacity_factor=1.0),
        Workload("capacity_fp8_n8192", n=8192, h=7168, e=256, k=8, ep=32, a=1,
                 fmt="fp8", routing="softmax", experts="random", capacity_factor=1.25),
        # exchange across 8 simulated ranks of the uniform prefill share;
        # receive buffers of 1.25 * N * k rows (the mean receive is N * k)
        Workload("exchange_bf16_ep8_n4096", n=4096, h=4096, e=64, k=6, ep=8,
                 a=1, fmt="bf16", routing="softmax", experts="identity",
                 recv_capacity=30720, ranks=8),
        # exchange of FP8 rows across 4 simulated ranks
        Workload("exchange_fp8_ep4_n2048", n=2048, h=7168, e=256, k=8, ep=4,
                 a=1, fmt="fp8", routing="softmax", experts="random",
                 recv_capacity=20480, ranks=4),
        # the uniform prefill share with the routing handed over as a dense
        # multihot map and dense probabilities (converted to top-k on the
        # device), gates applied at dispatch, unweighted combine
        Workload("gated_map_bf16_n4096", n=4096, h=4096, e=64, k=6, ep=8,
                 a=128, fmt="bf16", routing="softmax", experts="identity",
                 gated=True, routing_input="map"),
        # decode-sized exchange across 8 simulated ranks
        Workload("exchange_mxfp4_ep8_n128", n=128, h=7168, e=256, k=8, ep=8,
                 a=1, fmt="mxfp4", routing="softmax", experts="random",
                 recv_capacity=1280, ranks=8),
    ]
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest even) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def router(rng: np.random.Generator, w: Workload):
    """Draw logits and return (topk_ids int32 [T,k], weights float32 [T,k]),
    T = ranks * N tokens."""
    if w.routing == "softmax":
        logits = rng.standard_normal((w.tokens, w.e), dtype=np.float32)
    elif w.routing == "zipf":
        pop = (np.arange(1, w.e + 1, dtype=np.float64)) ** -1.2
        pop /= pop.sum()
        noise = rng.standard_normal((w.tokens, w.e), dtype=np.float32)
        logits = (np.log(pop)[None, :] + 0.5 * noise.astype(np.float64))
        logits = logits.astype(np.float32)
    else:
        raise ValueError(w.routing)
    order = np.argsort(-logits, axis=1, kind="stable")[:, : w.k]
    ids = order.astype(np.int32)
    l64 = logits.astype(np.float64)
    l64 -= l64.max(axis=1, keepdims=True)
    p = np.exp(l64)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, order, axis=1)
    sel /= sel.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(ids), np.ascontiguousarray(sel.astype(np.float32))


def make_inputs(w: Workload, seed: int = 0, expert_rows: int | None = None):
    """All inputs of one workload.

    Returns a dict with ``ids`` (int32 [T,k]), ``weights`` (float32 [T,k]),
    ``hidden`` (uint16 bf16 bits [T,H]), T = ranks * N, and, for random experts,
    ``expert_out`` (uint16 bf16 bits [expert_rows, H]).  Workloads whose
    routing is handed over as a dense map also get ``map`` (uint8 [T,E], 1
    where a token routes to an expert) and ``probs`` (float32 [T,E], the
    token's gate weight for those experts, 0 elsewhere): the same routing in
    the multihot form, nothing drawn.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ids, weights = router(rng, w)
    hidden = to_bf16_bits(rng.standard_normal((w.tokens, w.h), dtype=np.float32))
    out = dict(ids=ids, weights=weights, hidden=hidden)
    if w.experts == "random":
        if expert_rows is None:
            raise ValueError("random experts need expert_rows")
        out["expert_out"] = to_bf16_bits(
            rng.standard_normal((expert_rows, w.h), dtype=np.float32))
    if w.routing_input == "map":
        m = np.zeros((w.tokens, w.e), np.uint8)
        probs = np.zeros((w.tokens, w.e), np.float32)
        rows = np.arange(w.tokens)[:, None]
        m[rows, ids] = 1
        probs[rows, ids] = weights
        out["map"], out["probs"] = m, probs
    return out


def random_routing(rng: np.random.Generator, n: int, e: int, k: int,
                   masked_frac: float = 0.0):
    """Unique random expert IDs per token (optionally some slots masked -1)
    and positive weights summing to 1 per token."""
    keys = rng.random((n, e))
    ids = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    if masked_frac > 0:
        m = rng.random((n, k)) < masked_frac
        ids[m] = -1
    wts = rng.random((n, k)) + 0.05
    wts /= wts.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(ids), np.ascontiguousarray(wts.astype(np.float32))


def random_bf16(rng: np.random.Generator, shape, scale: float = 1.0):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
