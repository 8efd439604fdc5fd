"""CPU oracle for MoE token dispatch and combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain C, built
with gcc, no fast-math) through ctypes and numpy; it shares no code with the
HIP library and never imports it.

Every function here is argument marshalling around the C routines, whose
header comment lists the passages each step follows.  Formats:

* ``"bf16"``  payload ``uint16 [R_max, H]``, no scales;
* ``"fp8"``   payload ``uint8 [R_max, H]`` (OCP E4M3 codes), scales
  ``float32 [R_max, H/128]``;
* ``"mxfp4"`` payload ``uint8 [R_max, H/2]`` (two E2M1 codes a byte, element
  2m in the low nibble), scales ``uint8 [R_max, H/32]`` (E8M0 exponents).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# A separately built copy to load instead (the sanitizer test builds one with
# address and undefined-behaviour checks and runs the pins against it).
PREBUILT = os.environ.get("ORACLE_PREBUILT_LIB")

FMT = {"bf16": 0, "fp8": 1, "mxfp4": 2}
BAD_ID, DUP_ID, CAPACITY, MAP_OVERFLOW, DROPPED = 1, 2, 4, 8, 16

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it."""
    if PREBUILT:
        return PREBUILT
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
             "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if PREBUILT:
            lib = ctypes.CDLL(PREBUILT)
        else:
            if not os.path.exists(LIB):
                build(force=False)
            lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_max_rows.restype = i64
        lib.oracle_max_rows.argtypes = [i64, i32, i32, i32]
        lib.oracle_plan.restype = None
        lib.oracle_plan.argtypes = [i64, i32, i32, i32, i32, i64, i64] + [p] * 8
        lib.oracle_expert_capacity.restype = i64
        lib.oracle_expert_capacity.argtypes = [i64, i32, i32, ctypes.c_double]
        lib.oracle_capacity_plan.restype = None
        lib.oracle_capacity_plan.argtypes = [i64, i32, i32, i32, i64, i64, i64] + [p] * 8
        lib.oracle_encode_row_nvfp4.restype = None
        lib.oracle_encode_row_nvfp4.argtypes = [i64, p, ctypes.c_float, p, p]
        lib.oracle_dispatch_nvfp4.restype = None
        lib.oracle_dispatch_nvfp4.argtypes = [i64, i64, i64, p, p, ctypes.c_float, p, p, i32]
        lib.oracle_exchange_plan.restype = None
        lib.oracle_exchange_plan.argtypes = [i64, i32, i32, i32, i64, i64] + [p] * 9
        lib.oracle_encode_rows.restype = None
        lib.oracle_encode_rows.argtypes = [i32, i64, i64, p, p, p]
        lib.oracle_encode_row.restype = None
        lib.oracle_encode_row.argtypes = [i32, i64, p, p, p]
        lib.oracle_encode_row_f32.restype = None
        lib.oracle_encode_row_f32.argtypes = [i32, i64, p, p, p]
        lib.oracle_dispatch_gated.restype = None
        lib.oracle_dispatch_gated.argtypes = [i32, i64, i32, i64, i64, i64, p, p, p, p, p, i32]
        lib.oracle_routing_map_to_topk.restype = None
        lib.oracle_routing_map_to_topk.argtypes = [i64, i32, i32, p, p, p, p, p]
        lib.oracle_dispatch.restype = None
        lib.oracle_dispatch.argtypes = [i32, i64, i64, i64, p, p, p, p, i32]
        lib.oracle_combine.restype = None
        lib.oracle_combine.argtypes = [i64, i32, i64, p, p, p, p]
        for name in ("oracle_f32_to_bf16_array", "oracle_e4m3_encode_array",
                     "oracle_e2m1_encode_array"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [p, p, i64]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [i32]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [i32]
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_threads.restype = i32
        lib.oracle_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check_rows(idx: np.ndarray, n_rows: int, what: str) -> None:
    """The C loops index an array of n_rows rows by idx (-1 skips)."""
    if idx.size and (int(idx.max()) >= n_rows or int(idx.min()) < -1):
        raise ValueError(f"{what} holds {int(idx.min())}..{int(idx.max())}, outside -1..{n_rows - 1}")


def _check_buf(a: np.ndarray, shape, dtype, what: str) -> None:
    """A caller-given output array the C loop writes whole."""
    if a.shape != tuple(shape) or a.dtype != np.dtype(dtype) or not a.flags.c_contiguous:
        raise ValueError(f"{what} must be a contiguous {np.dtype(dtype)} array of shape "
                         f"{tuple(shape)}, not {a.dtype} {a.shape}")


def set_threads(n: int) -> None:
    """Threads the oracle's row loops may use (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def threads() -> int:
    return int(_load().oracle_threads())


def max_rows(n: int, k: int, e: int, a: int) -> int:
    """R_max = N*k + E*(A-1)."""
    return int(_load().oracle_max_rows(n, k, e, a))


def payload_shape(fmt: str, r_max: int, h: int):
    """(payload dtype, payload shape, scale dtype or None, scale shape)."""
    if fmt == "bf16":
        return np.uint16, (r_max, h), None, (r_max, 0)
    if fmt == "fp8":
        return np.uint8, (r_max, h), np.float32, (r_max, h // 128)
    if fmt == "mxfp4":
        return np.uint8, (r_max, h // 2), np.uint8, (r_max, h // 32)
    raise ValueError(fmt)


def plan(ids: np.ndarray, n_experts: int, ep: int, pad_multiple: int,
         recv_capacity: int, hidden: int) -> dict:
    """Counts, padded offsets, (4, EP) table, slots and packed sources.

    ``ids`` is ``int32 [N, k]`` with -1 for a masked slot.
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, k = ids.shape
    e = n_experts
    r_max = max_rows(n, k, e, pad_multiple)
    out = dict(
        expert_counts=np.zeros(e, np.int32),
        expert_offsets=np.zeros(e + 1, np.int32),
        dest_counts=np.zeros(ep, np.int32),
        rank_table=np.zeros((4, ep), np.uint32),
        slot=np.zeros((n, k), np.int32),
        packed_src=np.zeros(max(r_max, 0), np.int32),
        status=np.zeros(1, np.uint32),
    )
    _load().oracle_plan(n, k, e, ep, pad_multiple, recv_capacity, hidden,
                        _ptr(ids), _ptr(out["expert_counts"]),
                        _ptr(out["expert_offsets"]), _ptr(out["dest_counts"]),
                        _ptr(out["rank_table"]), _ptr(out["slot"]),
                        _ptr(out["packed_src"]), _ptr(out["status"]))
    out["r_max"] = r_max
    out["r_used"] = int(out["expert_offsets"][e])
    out["status"] = int(out["status"][0])
    return out


def expert_capacity(n: int, k: int, e: int, cf: float) -> int:
    """ceil(cf * N * k / E)."""
    return int(_load().oracle_expert_capacity(n, k, e, cf))


def capacity_plan(ids: np.ndarray, n_experts: int, ep: int, expert_cap: int,
                  recv_capacity: int, hidden: int) -> dict:
    """Plan of the fixed-capacity layout: expert e owns rows e*cap ..
    e*cap+cap-1; pairs past an expert's capacity are dropped."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, k = ids.shape
    e = n_experts
    r_max = e * expert_cap
    out = dict(
        expert_counts=np.zeros(e, np.int32),
        expert_offsets=np.zeros(e + 1, np.int32),
        dest_counts=np.zeros(ep, np.int32),
        rank_table=np.zeros((4, ep), np.uint32),
        slot=np.zeros((n, k), np.int32),
        packed_src=np.zeros(max(r_max, 0), np.int32),
        status=np.zeros(1, np.uint32),
    )
    _load().oracle_capacity_plan(n, k, e, ep, recv_capacity, hidden, expert_cap, _ptr(ids),
                                 _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
                                 _ptr(out["dest_counts"]), _ptr(out["rank_table"]),
                                 _ptr(out["slot"]), _ptr(out["packed_src"]), _ptr(out["status"]))
    out["r_max"] = r_max
    out["r_used"] = r_max
    out["status"] = int(out["status"][0])
    return out


def exchange_plan(ids: np.ndarray, n_experts: int, recv_capacity: int,
                  hidden: int) -> dict:
    """Receive-side plan for EP simulated ranks.

    ``ids`` is ``int32 [EP, N, k]``: rank s routes its own N tokens.  Returns
    the count matrix each rank sends, per-rank send counts, what each rank
    receives per source and local expert, the (4, EP) table of every rank,
    and the receive row of every pair (``d * C + i`` into the stacked receive
    buffers ``[EP, C]``) with its inverse ``recv_src`` (``s * N + t``).
    """
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    ep, n, k = ids.shape
    e = n_experts
    cap = recv_capacity
    out = dict(
        expert_counts=np.zeros((ep, e), np.int32),
        send_counts=np.zeros((ep, ep), np.int32),
        recv_expert_counts=np.zeros((ep, ep, e // ep), np.int32),
        recv_rows=np.zeros(ep, np.int32),
        rank_table=np.zeros((ep, 4, ep), np.uint32),
        recv_slot=np.zeros((ep, n, k), np.int32),
        recv_src=np.zeros((ep, cap), np.int32),
        status=np.zeros(ep, np.uint32),
    )
    _load().oracle_exchange_plan(n, k, e, ep, cap, hidden, _ptr(ids),
                                 _ptr(out["expert_counts"]), _ptr(out["send_counts"]),
                                 _ptr(out["recv_expert_counts"]), _ptr(out["recv_rows"]),
                                 _ptr(out["rank_table"]), _ptr(out["recv_slot"]),
                                 _ptr(out["recv_src"]), _ptr(out["status"]))
    return out


def exchange_dispatch(fmt: str, x: np.ndarray, xp: dict, payload=None, scales=None):
    """Every receive buffer, whole: row ``d*C + i`` holds the encoded row of
    global token ``recv_src[d, i]`` of the stacked ``x [EP*N, H]``, or zero
    bytes.  Returns ``(payload [EP*C, ...], scales [EP*C, ...] or None)``."""
    ep, cap = xp["recv_src"].shape
    src = np.ascontiguousarray(xp["recv_src"].reshape(-1))
    pl = dict(packed_src=src, r_max=ep * cap, r_used=ep * cap)
    return dispatch(fmt, x, pl, zero_tail=True, payload=payload, scales=scales)


def encode_rows(fmt: str, x: np.ndarray):
    """Encode whole hidden rows ``uint16 [M, H]``: (payload rows, scale rows)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m, h = x.shape
    pdt, pshape, sdt, sshape = payload_shape(fmt, m, h)
    pay = np.zeros(pshape, pdt)
    sc = np.zeros(sshape, sdt if sdt is not None else np.uint8)
    _load().oracle_encode_rows(FMT[fmt], m, h, _ptr(x), _ptr(pay),
                               _ptr(sc) if sdt is not None else None)
    return pay, (sc if sdt is not None else None)


def dispatch(fmt: str, x: np.ndarray, pl: dict, zero_tail: bool = True,
             payload: np.ndarray | None = None, scales: np.ndarray | None = None):
    """Packed payload and scales for the whole buffer (gather form).

    Rows past R_used are zero when ``zero_tail``; otherwise they keep what the
    given ``payload``/``scales`` arrays held (zeros if none are given).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    h = x.shape[1]
    r_max = pl["r_max"]
    src = np.ascontiguousarray(pl["packed_src"], dtype=np.int32)
    if src.size < r_max:
        raise ValueError(f"packed_src has {src.size} rows, fewer than R_max = {r_max}")
    _check_rows(src[:r_max], x.shape[0], "packed_src")
    pdt, pshape, sdt, sshape = payload_shape(fmt, r_max, h)
    if payload is None:
        payload = np.zeros(pshape, pdt)
    _check_buf(payload, pshape, pdt, "payload")
    if scales is None:
        scales = np.zeros(sshape, sdt if sdt is not None else np.uint8)
    elif sdt is not None:
        _check_buf(scales, sshape, sdt, "scales")
    _load().oracle_dispatch(FMT[fmt], h, r_max, pl["r_used"],
                            _ptr(src), _ptr(x), _ptr(payload),
                            _ptr(scales), int(zero_tail))
    return payload, (scales if sdt is not None else None)


def dispatch_gated(fmt: str, x: np.ndarray, pl: dict, w: np.ndarray, zero_tail: bool = True,
                   payload: np.ndarray | None = None, scales: np.ndarray | None = None):
    """Packed payload and scales when every copy carries its gate: row
    slot[t, j] holds encode(fl32(w[t, j] * x[t])) (scatter form)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    slot = np.ascontiguousarray(pl["slot"], dtype=np.int32)
    n, h = x.shape
    k = slot.shape[1]
    r_max = pl["r_max"]
    if slot.shape[0] != n or w.shape != slot.shape:
        raise ValueError(f"slot {slot.shape} and gates {w.shape} must both be [{n}, k]")
    _check_rows(slot, r_max, "slot")
    pdt, pshape, sdt, sshape = payload_shape(fmt, r_max, h)
    if payload is None:
        payload = np.zeros(pshape, pdt)
    _check_buf(payload, pshape, pdt, "payload")
    if scales is None:
        scales = np.zeros(sshape, sdt if sdt is not None else np.uint8)
    elif sdt is not None:
        _check_buf(scales, sshape, sdt, "scales")
    _load().oracle_dispatch_gated(FMT[fmt], n, k, h, r_max, pl["r_used"], _ptr(slot), _ptr(w),
                                  _ptr(x), _ptr(payload), _ptr(scales), int(zero_tail))
    return payload, (scales if sdt is not None else None)


def encode_rows_f32(fmt: str, v: np.ndarray):
    """Encode rows of fp32 values ``[M, H]``: (payload rows, scale rows)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    m, h = v.shape
    pdt, pshape, sdt, sshape = payload_shape(fmt, m, h)
    pay = np.zeros(pshape, pdt)
    sc = np.zeros(sshape, sdt if sdt is not None else np.uint8)
    lib = _load()
    for i in range(m):
        lib.oracle_encode_row_f32(FMT[fmt], h, ctypes.c_void_p(v[i].ctypes.data),
                                  ctypes.c_void_p(pay[i].ctypes.data),
                                  ctypes.c_void_p(sc[i].ctypes.data) if sdt is not None else None)
    return pay, (sc if sdt is not None else None)


def routing_map_to_topk(routing_map: np.ndarray, probs: np.ndarray | None, k: int):
    """Multihot map ``[N, E]`` (nonzero = routed) and dense probabilities
    ``[N, E]`` (or None) -> (ids int32 [N, k], weights float32 [N, k],
    status)."""
    m = np.ascontiguousarray(routing_map != 0, dtype=np.uint8)
    n, e = m.shape
    pr = None if probs is None else np.ascontiguousarray(probs, dtype=np.float32)
    if pr is not None and pr.shape != m.shape:
        raise ValueError(f"probs {pr.shape} must match the map {m.shape}")
    ids = np.zeros((n, k), np.int32)
    w = np.zeros((n, k), np.float32)
    st = np.zeros(1, np.uint32)
    _load().oracle_routing_map_to_topk(n, e, k, _ptr(m), None if pr is None else _ptr(pr),
                                       _ptr(ids), _ptr(w), _ptr(st))
    return ids, w, int(st[0])


def encode_rows_nvfp4(x: np.ndarray, gs: float):
    """NVFP4 rows of bf16 ``x [M, H]`` with global encode scale ``gs``:
    (payload uint8 [M, H/2], scales uint8 [M, H/16] of E4M3 codes)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m, h = x.shape
    pay = np.zeros((m, h // 2), np.uint8)
    sc = np.zeros((m, h // 16), np.uint8)
    lib = _load()
    for i in range(m):
        lib.oracle_encode_row_nvfp4(h, ctypes.c_void_p(x[i].ctypes.data), float(gs),
                                    ctypes.c_void_p(pay[i].ctypes.data),
                                    ctypes.c_void_p(sc[i].ctypes.data))
    return pay, sc


def dispatch_nvfp4(x: np.ndarray, pl: dict, gs: float, zero_tail: bool = True):
    """Gather-form NVFP4 dispatch over the plan's packed rows."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    h = x.shape[1]
    r_max = pl["r_max"]
    src = np.ascontiguousarray(pl["packed_src"], dtype=np.int32)
    if src.size < r_max:
        raise ValueError(f"packed_src has {src.size} rows, fewer than R_max = {r_max}")
    _check_rows(src[:r_max], x.shape[0], "packed_src")
    pay = np.zeros((r_max, h // 2), np.uint8)
    sc = np.zeros((r_max, h // 16), np.uint8)
    _load().oracle_dispatch_nvfp4(h, r_max, pl["r_used"], _ptr(src),
                                  _ptr(x), float(gs), _ptr(pay), _ptr(sc), int(zero_tail))
    return pay, sc


def combine(slot: np.ndarray, w: np.ndarray | None, y: np.ndarray) -> np.ndarray:
    """``out uint16 [N, H]`` (bf16 bits) from ``slot [N,k]``, ``w f32 [N,k]``
    (None: every weight 1, the unweighted sum after a gated dispatch) and
    expert outputs ``y uint16 [rows, H]``."""
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    y = np.ascontiguousarray(y, dtype=np.uint16)
    n, k = slot.shape
    h = y.shape[1]
    # the C loop indexes y by slot: reject rows it does not have
    if slot.size and slot.max() >= y.shape[0]:
        raise ValueError(f"slot {int(slot.max())} names a row past the {y.shape[0]} rows of y")
    out = np.zeros((n, h), np.uint16)
    wp = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        if w.shape != slot.shape:
            raise ValueError(f"weights {w.shape} do not match slot {slot.shape}")
        wp = _ptr(w)
    _load().oracle_combine(n, k, h, _ptr(slot), wp, _ptr(y), _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.zeros(a.shape, np.uint16)
    _load().oracle_f32_to_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_encode(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.zeros(a.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(a), _ptr(out), a.size)
    return out


def e2m1_encode(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.zeros(a.shape, np.uint8)
    _load().oracle_e2m1_encode_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_value(code: int) -> float:
    """Value of a non-negative E4M3 code 0..126."""
    return float(_load().oracle_e4m3_value(code))


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(code))
