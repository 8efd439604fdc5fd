"""ctypes binding of libmoe (HIP, gfx950): MoE dispatch plan, dispatch, combine.

Argument marshalling only: every step of the path runs in libmoe's kernels.
PyTorch supplies device memory (tensors' ``data_ptr()``) and the stream
(``torch.cuda.current_stream()``).  The C ABI, with the meaning, layout and
error behaviour of every argument, is ``include/moe.h``; the functions here
carry the same names.

Importing this module loads ``libmoe.so`` and fails loudly if it has not been
built (``python -m combine_topk_ids_amd._build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch  # first: libmoe then binds to the HIP runtime torch has loaded

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EOVERFLOW, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 1 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STATUS_BAD_ID, STATUS_DUP_ID, STATUS_CAPACITY, STATUS_MAP_OVERFLOW, STATUS_DROPPED = 1, 2, 4, 8, 16
STATUS_BAD_PLAN = 32
FMT = {"bf16": 0, "fp8": 1, "mxfp4": 2, "nvfp4": 3}
FLAG_ZERO_TAIL = 1
# how moe_plan_and_dispatch runs a problem (moe_plan_and_dispatch_mode)
PD_ONE_LAUNCH, PD_TILED, PD_SEPARATE = 1, 2, 3

# every symbol include/moe.h declares
EXPORTS = ("moe_check_problem", "moe_max_rows", "moe_expert_capacity", "moe_payload_row_bytes",
           "moe_scale_row_bytes", "moe_workspace_bytes", "moe_dispatch_plan",
           "moe_dispatch", "moe_dispatch_scaled", "moe_dispatch_gated", "moe_plan_and_dispatch",
           "moe_plan_and_dispatch_mode", "moe_plan_and_dispatch_begin",
           "moe_plan_and_dispatch_end", "moe_combine",
           "moe_check_exchange", "moe_exchange_workspace_bytes", "moe_exchange_plan",
           "moe_exchange_dispatch", "moe_exchange_dispatch_scaled", "moe_exchange_dispatch_gated",
           "moe_exchange_combine", "moe_map_workspace_bytes",
           "moe_routing_map_to_topk", "moe_plan_and_dispatch_noalloc", "moe_strerror")


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} (code {code})")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("ep", ctypes.c_int32), ("recv_capacity", ctypes.c_int64),
                ("pad_multiple", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("expert_capacity", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "expert_counts", "expert_offsets", "dest_counts", "rank_table", "slot",
        "packed_src", "status")]


class Exchange(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "expert_counts", "send_counts", "recv_expert_counts", "recv_rows", "rank_table",
        "recv_slot", "recv_src", "status")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m combine_topk_ids_amd._build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, V = ctypes.POINTER(Problem), ctypes.c_void_p
    sig = {
        "moe_check_problem": (ctypes.c_int, [P]),
        "moe_max_rows": (ctypes.c_int64, [P]),
        "moe_expert_capacity": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_double]),
        "moe_payload_row_bytes": (ctypes.c_int64, [P]),
        "moe_scale_row_bytes": (ctypes.c_int64, [P]),
        "moe_workspace_bytes": (ctypes.c_size_t, [P]),
        "moe_dispatch_plan": (ctypes.c_int, [P, V, ctypes.POINTER(Plan), V, V]),
        "moe_dispatch": (ctypes.c_int, [P, ctypes.POINTER(Plan), V, V, V, V]),
        "moe_dispatch_gated": (ctypes.c_int, [P, ctypes.POINTER(Plan), V, V, V, V, V]),
        "moe_plan_and_dispatch": (ctypes.c_int, [P, V, ctypes.POINTER(Plan), V, V, V, V, V, V, V]),
        "moe_plan_and_dispatch_mode": (ctypes.c_int, [P]),
        "moe_plan_and_dispatch_begin": (ctypes.c_int, [P, V, ctypes.POINTER(Plan), V, V]),
        "moe_plan_and_dispatch_end": (ctypes.c_int, [P, V, ctypes.POINTER(Plan), V, V, V, V, V, V, V]),
        "moe_plan_and_dispatch_noalloc": (ctypes.c_int, [P, V, ctypes.POINTER(Plan), V, V, V, V, V, V]),
        "moe_dispatch_scaled": (ctypes.c_int, [P, ctypes.POINTER(Plan), V, V, V, V, V]),
        "moe_exchange_dispatch_scaled": (ctypes.c_int, [P, ctypes.POINTER(Exchange), V, V, V, V, V]),
        "moe_combine": (ctypes.c_int, [P, ctypes.POINTER(Plan), V, V, V, V]),
        "moe_check_exchange": (ctypes.c_int, [P]),
        "moe_exchange_workspace_bytes": (ctypes.c_size_t, [P]),
        "moe_exchange_plan": (ctypes.c_int, [P, V, ctypes.POINTER(Exchange), V, V]),
        "moe_exchange_dispatch": (ctypes.c_int, [P, ctypes.POINTER(Exchange), V, V, V, V]),
        "moe_exchange_dispatch_gated": (ctypes.c_int, [P, ctypes.POINTER(Exchange), V, V, V, V, V]),
        "moe_exchange_combine": (ctypes.c_int, [P, ctypes.POINTER(Exchange), V, V, V, V]),
        "moe_map_workspace_bytes": (ctypes.c_size_t, [P]),
        "moe_routing_map_to_topk": (ctypes.c_int, [P, V, V, V, V, V, V, V]),
        "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def strerror(code: int) -> str:
    return lib.moe_strerror(code).decode()


def problem(n_tokens: int, hidden: int, top_k: int, n_experts: int, ep: int,
            recv_capacity: int | None = None, pad_multiple: int = 1,
            fmt: str = "bf16", zero_tail: bool = False, expert_capacity: int = 0) -> Problem:
    """Build a moe_problem; recv_capacity None means the dropless bound;
    expert_capacity > 0 selects the fixed-capacity [E][cap] layout."""
    if recv_capacity is None:
        recv_capacity = n_tokens * min(top_k, n_experts // max(ep, 1))
    return Problem(n_tokens, hidden, top_k, n_experts, ep, recv_capacity,
                   pad_multiple, FMT[fmt], FLAG_ZERO_TAIL if zero_tail else 0, expert_capacity)


def moe_expert_capacity(n_tokens: int, top_k: int, n_experts: int, capacity_factor: float) -> int:
    """ceil(capacity_factor * N * k / E)."""
    return _checked(lib.moe_expert_capacity(n_tokens, top_k, n_experts, float(capacity_factor)),
                    "moe_expert_capacity")


def _checked(value: int, where: str) -> int:
    if value < 0:
        raise MoeError(value, where)
    return int(value)


def moe_check_problem(p: Problem) -> int:
    return int(lib.moe_check_problem(ctypes.byref(p)))


def moe_max_rows(p: Problem) -> int:
    return _checked(lib.moe_max_rows(ctypes.byref(p)), "moe_max_rows")


def moe_payload_row_bytes(p: Problem) -> int:
    return _checked(lib.moe_payload_row_bytes(ctypes.byref(p)), "moe_payload_row_bytes")


def moe_scale_row_bytes(p: Problem) -> int:
    return _checked(lib.moe_scale_row_bytes(ctypes.byref(p)), "moe_scale_row_bytes")


def moe_workspace_bytes(p: Problem) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(p)))


_SIZES: dict = {}


def _sizes(p: Problem):
    """(R_max, payload row bytes, scale row bytes, workspace bytes), cached per
    problem value (the C library stays the source of these numbers)."""
    key = (p.n_tokens, p.hidden, p.top_k, p.n_experts, p.ep, p.recv_capacity,
           p.pad_multiple, p.fmt, p.flags, p.expert_capacity)
    v = _SIZES.get(key)
    if v is None:
        v = (moe_max_rows(p), moe_payload_row_bytes(p), moe_scale_row_bytes(p),
             moe_workspace_bytes(p))
        if len(_SIZES) > 4096:
            _SIZES.clear()
        _SIZES[key] = v
    return v


@dataclasses.dataclass(frozen=True)
class PlanBuffers:
    """Device tensors a plan is written to, plus the plan kernels' workspace."""
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    dest_counts: torch.Tensor
    rank_table: torch.Tensor
    slot: torch.Tensor
    packed_src: torch.Tensor
    status: torch.Tensor
    workspace: torch.Tensor

    def as_struct(self) -> Plan:
        """The moe_plan struct (device pointers); built once per buffer set."""
        st = self.__dict__.get("_struct")
        if st is None:
            st = Plan(*(getattr(self, f).data_ptr() for f, _ in Plan._fields_))
            self.__dict__["_struct"] = st
        return st

    def read_status(self) -> int:
        """Synchronises the current stream and returns the status bits."""
        return int(self.status.item())


def alloc_plan(p: Problem, device="cuda") -> PlanBuffers:
    r_max = moe_max_rows(p)
    i32 = dict(dtype=torch.int32, device=device)
    return PlanBuffers(
        expert_counts=torch.empty(p.n_experts, **i32),
        expert_offsets=torch.empty(p.n_experts + 1, **i32),
        dest_counts=torch.empty(p.ep, **i32),
        rank_table=torch.empty((4, p.ep), **i32),  # uint32 bits in int32 storage
        slot=torch.empty((p.n_tokens, p.top_k), **i32),
        packed_src=torch.empty(max(r_max, 1), **i32),
        status=torch.empty(1, **i32),
        workspace=torch.empty(max(moe_workspace_bytes(p), 256), dtype=torch.uint8,
                              device=device),
    )


def alloc_payload(p: Problem, device="cuda"):
    """(payload, scales) device tensors of R_max rows for p.fmt."""
    r_max = moe_max_rows(p)
    h = p.hidden
    if p.fmt == FMT["bf16"]:
        return torch.empty((r_max, h), dtype=torch.bfloat16, device=device), None
    if p.fmt == FMT["fp8"]:
        return (torch.empty((r_max, h), dtype=torch.uint8, device=device),
                torch.empty((r_max, h // 128), dtype=torch.float32, device=device))
    if p.fmt == FMT["nvfp4"]:
        return (torch.empty((r_max, h // 2), dtype=torch.uint8, device=device),
                torch.empty((r_max, h // 16), dtype=torch.uint8, device=device))
    return (torch.empty((r_max, h // 2), dtype=torch.uint8, device=device),
            torch.empty((r_max, h // 32), dtype=torch.uint8, device=device))


def _dev(t: torch.Tensor | None, name: str, dtypes, numel: int | None = None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    """Raw hipStream_t of `stream`, or of torch's current stream (which is the
    capture stream inside torch.cuda.graph)."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_PAYLOAD = (torch.bfloat16, torch.int16, torch.uint16, torch.uint8, torch.float8_e4m3fn)


def moe_dispatch_plan(p: Problem, topk_ids: torch.Tensor, plan: PlanBuffers, stream=None) -> None:
    r_max, _, _, ws = _sizes(p)
    npairs = p.n_tokens * p.top_k
    ids = _dev(topk_ids, "topk_ids", (torch.int32,), npairs)
    _dev(plan.slot, "plan.slot", (torch.int32,), npairs)
    _dev(plan.packed_src, "plan.packed_src", (torch.int32,), r_max)
    _dev(plan.workspace, "plan.workspace", (torch.uint8,), ws)
    rc = lib.moe_dispatch_plan(ctypes.byref(p), ids, ctypes.byref(plan.as_struct()),
                               plan.workspace.data_ptr(), _stream(stream))
    _checked(rc, "moe_dispatch_plan")


def moe_dispatch(p: Problem, plan: PlanBuffers, hidden: torch.Tensor, payload: torch.Tensor,
                 scales: torch.Tensor | None, stream=None) -> None:
    r_max, pb, sb, _ = _sizes(p)
    x = _dev(hidden, "hidden", _BF16, p.n_tokens * p.hidden)
    if payload.numel() * payload.element_size() < r_max * pb:
        raise ValueError("payload is smaller than R_max rows")
    if scales is not None and scales.numel() * scales.element_size() < r_max * sb:
        raise ValueError("scales is smaller than R_max rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.float32, torch.uint8))
    rc = lib.moe_dispatch(ctypes.byref(p), ctypes.byref(plan.as_struct()), x, pay, sc or None,
                          _stream(stream))
    _checked(rc, "moe_dispatch")


def moe_dispatch_scaled(p: Problem, plan: PlanBuffers, hidden: torch.Tensor,
                        input_scale: torch.Tensor, payload: torch.Tensor, scales: torch.Tensor,
                        stream=None) -> None:
    """NVFP4 dispatch; input_scale: device float32 tensor holding the global
    encode scale."""
    r_max, pb, sb, _ = _sizes(p)
    x = _dev(hidden, "hidden", _BF16, p.n_tokens * p.hidden)
    gs = _dev(input_scale, "input_scale", (torch.float32,), 1)
    if payload.numel() * payload.element_size() < r_max * pb:
        raise ValueError("payload is smaller than R_max rows")
    if scales.numel() * scales.element_size() < r_max * sb:
        raise ValueError("scales is smaller than R_max rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.uint8,))
    rc = lib.moe_dispatch_scaled(ctypes.byref(p), ctypes.byref(plan.as_struct()), x, gs, pay, sc,
                                 _stream(stream))
    _checked(rc, "moe_dispatch_scaled")


def moe_dispatch_gated(p: Problem, plan: PlanBuffers, hidden: torch.Tensor,
                       topk_weights: torch.Tensor, payload: torch.Tensor,
                       scales: torch.Tensor | None, stream=None) -> None:
    r_max, pb, sb, _ = _sizes(p)
    x = _dev(hidden, "hidden", _BF16, p.n_tokens * p.hidden)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), p.n_tokens * p.top_k)
    if payload.numel() * payload.element_size() < r_max * pb:
        raise ValueError("payload is smaller than R_max rows")
    if scales is not None and scales.numel() * scales.element_size() < r_max * sb:
        raise ValueError("scales is smaller than R_max rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.float32, torch.uint8))
    rc = lib.moe_dispatch_gated(ctypes.byref(p), ctypes.byref(plan.as_struct()), x, w, pay,
                                sc or None, _stream(stream))
    _checked(rc, "moe_dispatch_gated")


def _pd_args(p: Problem, topk_ids, plan: PlanBuffers, hidden, payload, scales, topk_weights,
             input_scale, need_workspace=True):
    r_max, pb, sb, ws = _sizes(p)
    npairs = p.n_tokens * p.top_k
    ids = _dev(topk_ids, "topk_ids", (torch.int32,), npairs)
    _dev(plan.slot, "plan.slot", (torch.int32,), npairs)
    _dev(plan.packed_src, "plan.packed_src", (torch.int32,), r_max)
    if need_workspace:
        _dev(plan.workspace, "plan.workspace", (torch.uint8,), ws)
    x = _dev(hidden, "hidden", _BF16, p.n_tokens * p.hidden)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), npairs) or None
    gs = _dev(input_scale, "input_scale", (torch.float32,), 1) or None
    if payload.numel() * payload.element_size() < r_max * pb:
        raise ValueError("payload is smaller than R_max rows")
    if scales is not None and scales.numel() * scales.element_size() < r_max * sb:
        raise ValueError("scales is smaller than R_max rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.float32, torch.uint8))
    return (ctypes.byref(p), ids, ctypes.byref(plan.as_struct()), x, w, gs, pay, sc or None,
            plan.workspace.data_ptr())


def moe_plan_and_dispatch(p: Problem, topk_ids: torch.Tensor, plan: PlanBuffers,
                          hidden: torch.Tensor, payload: torch.Tensor, scales: torch.Tensor | None,
                          topk_weights: torch.Tensor | None = None,
                          input_scale: torch.Tensor | None = None, stream=None) -> None:
    """moe_dispatch_plan then moe_dispatch (or the gated dispatch with
    topk_weights, or the NVFP4 dispatch with input_scale), in one or two
    launches (moe_plan_and_dispatch_mode) where the problem allows."""
    args = _pd_args(p, topk_ids, plan, hidden, payload, scales, topk_weights, input_scale)
    _checked(lib.moe_plan_and_dispatch(*args, _stream(stream)), "moe_plan_and_dispatch")


def moe_plan_and_dispatch_noalloc(p: Problem, topk_ids: torch.Tensor, plan: PlanBuffers,
                                  hidden: torch.Tensor, payload: torch.Tensor,
                                  scales: torch.Tensor | None,
                                  topk_weights: torch.Tensor | None = None,
                                  input_scale: torch.Tensor | None = None, stream=None) -> None:
    """moe_plan_and_dispatch with the plan's workspace in the library's static
    device scratch (plan.workspace is not used); raises MoeError with
    MOE_ESCRATCH for problems whose workspace exceeds NOALLOC_SCRATCH_BYTES."""
    args = _pd_args(p, topk_ids, plan, hidden, payload, scales, topk_weights, input_scale,
                    need_workspace=False)
    _checked(lib.moe_plan_and_dispatch_noalloc(*args[:-1], _stream(stream)),
             "moe_plan_and_dispatch_noalloc")


def moe_plan_and_dispatch_mode(p: Problem) -> int:
    """PD_ONE_LAUNCH, PD_TILED or PD_SEPARATE."""
    return _checked(lib.moe_plan_and_dispatch_mode(ctypes.byref(p)),
                    "moe_plan_and_dispatch_mode")


def moe_plan_and_dispatch_begin(p: Problem, topk_ids: torch.Tensor, plan: PlanBuffers,
                                stream=None) -> None:
    """The launches of moe_plan_and_dispatch that need only topk_ids."""
    r_max, _, _, ws = _sizes(p)
    npairs = p.n_tokens * p.top_k
    ids = _dev(topk_ids, "topk_ids", (torch.int32,), npairs)
    _dev(plan.slot, "plan.slot", (torch.int32,), npairs)
    _dev(plan.packed_src, "plan.packed_src", (torch.int32,), r_max)
    _dev(plan.workspace, "plan.workspace", (torch.uint8,), ws)
    rc = lib.moe_plan_and_dispatch_begin(ctypes.byref(p), ids, ctypes.byref(plan.as_struct()),
                                         plan.workspace.data_ptr(), _stream(stream))
    _checked(rc, "moe_plan_and_dispatch_begin")


def moe_plan_and_dispatch_end(p: Problem, topk_ids: torch.Tensor, plan: PlanBuffers,
                              hidden: torch.Tensor, payload: torch.Tensor,
                              scales: torch.Tensor | None, topk_weights: torch.Tensor | None = None,
                              input_scale: torch.Tensor | None = None, stream=None) -> None:
    """The launch of moe_plan_and_dispatch that writes the payload, after
    moe_plan_and_dispatch_begin on the same stream."""
    args = _pd_args(p, topk_ids, plan, hidden, payload, scales, topk_weights, input_scale)
    _checked(lib.moe_plan_and_dispatch_end(*args, _stream(stream)), "moe_plan_and_dispatch_end")


def moe_combine(p: Problem, plan: PlanBuffers, expert_out: torch.Tensor,
                topk_weights: torch.Tensor | None, out: torch.Tensor, stream=None) -> None:
    """topk_weights None: weights of 1 (after a gated dispatch)."""
    r_max = _sizes(p)[0]
    y = _dev(expert_out, "expert_out", _BF16, r_max * p.hidden)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), p.n_tokens * p.top_k) or None
    o = _dev(out, "out", _BF16, p.n_tokens * p.hidden)
    rc = lib.moe_combine(ctypes.byref(p), ctypes.byref(plan.as_struct()), y, w, o,
                         _stream(stream))
    _checked(rc, "moe_combine")


# ---- exchange across EP simulated ranks ---------------------------------------

def moe_check_exchange(p: Problem) -> int:
    return int(lib.moe_check_exchange(ctypes.byref(p)))


def moe_exchange_workspace_bytes(p: Problem) -> int:
    return int(lib.moe_exchange_workspace_bytes(ctypes.byref(p)))


@dataclasses.dataclass(frozen=True)
class ExchangeBuffers:
    """Device tensors an exchange plan is written to, plus its workspace."""
    expert_counts: torch.Tensor
    send_counts: torch.Tensor
    recv_expert_counts: torch.Tensor
    recv_rows: torch.Tensor
    rank_table: torch.Tensor
    recv_slot: torch.Tensor
    recv_src: torch.Tensor
    status: torch.Tensor
    workspace: torch.Tensor

    def as_struct(self) -> Exchange:
        st = self.__dict__.get("_struct")
        if st is None:
            st = Exchange(*(getattr(self, f).data_ptr() for f, _ in Exchange._fields_))
            self.__dict__["_struct"] = st
        return st


def alloc_exchange(p: Problem, device="cuda") -> ExchangeBuffers:
    """Buffers of an exchange over p.ep ranks of p.n_tokens tokens each."""
    ep, e = p.ep, p.n_experts
    i32 = dict(dtype=torch.int32, device=device)
    ws = moe_exchange_workspace_bytes(p)
    if ws == 0:
        raise MoeError(moe_check_exchange(p), "alloc_exchange")
    return ExchangeBuffers(
        expert_counts=torch.empty((ep, e), **i32),
        send_counts=torch.empty((ep, ep), **i32),
        recv_expert_counts=torch.empty((ep, ep, e // ep), **i32),
        recv_rows=torch.empty(ep, **i32),
        rank_table=torch.empty((ep, 4, ep), **i32),  # uint32 bits in int32 storage
        recv_slot=torch.empty((ep, p.n_tokens, p.top_k), **i32),
        recv_src=torch.empty((ep, max(p.recv_capacity, 1)), **i32),
        status=torch.empty(ep, **i32),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device),
    )


def alloc_recv_payload(p: Problem, device="cuda"):
    """(payload, scales) device tensors of EP * C receive rows for p.fmt."""
    rows = p.ep * p.recv_capacity
    h = p.hidden
    if p.fmt == FMT["bf16"]:
        return torch.empty((rows, h), dtype=torch.bfloat16, device=device), None
    if p.fmt == FMT["fp8"]:
        return (torch.empty((rows, h), dtype=torch.uint8, device=device),
                torch.empty((rows, h // 128), dtype=torch.float32, device=device))
    if p.fmt == FMT["nvfp4"]:
        return (torch.empty((rows, h // 2), dtype=torch.uint8, device=device),
                torch.empty((rows, h // 16), dtype=torch.uint8, device=device))
    return (torch.empty((rows, h // 2), dtype=torch.uint8, device=device),
            torch.empty((rows, h // 32), dtype=torch.uint8, device=device))


def moe_exchange_plan(p: Problem, topk_ids: torch.Tensor, x: ExchangeBuffers, stream=None) -> None:
    tokens = p.ep * p.n_tokens
    ids = _dev(topk_ids, "topk_ids", (torch.int32,), tokens * p.top_k)
    _dev(x.recv_slot, "recv_slot", (torch.int32,), tokens * p.top_k)
    _dev(x.recv_src, "recv_src", (torch.int32,), p.ep * p.recv_capacity)
    _dev(x.workspace, "workspace", (torch.uint8,), moe_exchange_workspace_bytes(p))
    rc = lib.moe_exchange_plan(ctypes.byref(p), ids, ctypes.byref(x.as_struct()),
                               x.workspace.data_ptr(), _stream(stream))
    _checked(rc, "moe_exchange_plan")


def moe_exchange_dispatch(p: Problem, x: ExchangeBuffers, hidden: torch.Tensor,
                          payload: torch.Tensor, scales: torch.Tensor | None, stream=None) -> None:
    _, pb, sb, _ = _sizes(p)
    rows = p.ep * p.recv_capacity
    h = _dev(hidden, "hidden", _BF16, p.ep * p.n_tokens * p.hidden)
    if payload.numel() * payload.element_size() < rows * pb:
        raise ValueError("payload is smaller than EP * C rows")
    if scales is not None and scales.numel() * scales.element_size() < rows * sb:
        raise ValueError("scales is smaller than EP * C rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.float32, torch.uint8))
    rc = lib.moe_exchange_dispatch(ctypes.byref(p), ctypes.byref(x.as_struct()), h, pay,
                                   sc or None, _stream(stream))
    _checked(rc, "moe_exchange_dispatch")


def moe_exchange_dispatch_scaled(p: Problem, x: ExchangeBuffers, hidden: torch.Tensor,
                                 input_scale: torch.Tensor, payload: torch.Tensor,
                                 scales: torch.Tensor, stream=None) -> None:
    _, pb, sb, _ = _sizes(p)
    rows = p.ep * p.recv_capacity
    h = _dev(hidden, "hidden", _BF16, p.ep * p.n_tokens * p.hidden)
    gs = _dev(input_scale, "input_scale", (torch.float32,), 1)
    if payload.numel() * payload.element_size() < rows * pb:
        raise ValueError("payload is smaller than EP * C rows")
    if scales.numel() * scales.element_size() < rows * sb:
        raise ValueError("scales is smaller than EP * C rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.uint8,))
    rc = lib.moe_exchange_dispatch_scaled(ctypes.byref(p), ctypes.byref(x.as_struct()), h, gs, pay,
                                          sc, _stream(stream))
    _checked(rc, "moe_exchange_dispatch_scaled")


def moe_exchange_dispatch_gated(p: Problem, x: ExchangeBuffers, hidden: torch.Tensor,
                                topk_weights: torch.Tensor, payload: torch.Tensor,
                                scales: torch.Tensor | None, stream=None) -> None:
    _, pb, sb, _ = _sizes(p)
    rows = p.ep * p.recv_capacity
    h = _dev(hidden, "hidden", _BF16, p.ep * p.n_tokens * p.hidden)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), p.ep * p.n_tokens * p.top_k)
    if payload.numel() * payload.element_size() < rows * pb:
        raise ValueError("payload is smaller than EP * C rows")
    if scales is not None and scales.numel() * scales.element_size() < rows * sb:
        raise ValueError("scales is smaller than EP * C rows")
    pay = _dev(payload, "payload", _PAYLOAD)
    sc = _dev(scales, "scales", (torch.float32, torch.uint8))
    rc = lib.moe_exchange_dispatch_gated(ctypes.byref(p), ctypes.byref(x.as_struct()), h, w, pay,
                                         sc or None, _stream(stream))
    _checked(rc, "moe_exchange_dispatch_gated")


def moe_exchange_combine(p: Problem, x: ExchangeBuffers, expert_out: torch.Tensor,
                         topk_weights: torch.Tensor | None, out: torch.Tensor, stream=None) -> None:
    """topk_weights None: weights of 1 (after a gated dispatch)."""
    tokens = p.ep * p.n_tokens
    y = _dev(expert_out, "expert_out", _BF16, p.ep * p.recv_capacity * p.hidden)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), tokens * p.top_k) or None
    o = _dev(out, "out", _BF16, tokens * p.hidden)
    rc = lib.moe_exchange_combine(ctypes.byref(p), ctypes.byref(x.as_struct()), y, w, o,
                                  _stream(stream))
    _checked(rc, "moe_exchange_combine")


# ---- dense routing-map input ----------------------------------------------------

def moe_map_workspace_bytes(p: Problem) -> int:
    return int(lib.moe_map_workspace_bytes(ctypes.byref(p)))


def moe_routing_map_to_topk(p: Problem, routing_map: torch.Tensor, probs: torch.Tensor | None,
                            topk_ids: torch.Tensor, topk_weights: torch.Tensor | None,
                            status: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """Multihot map [N, E] (uint8 or bool; nonzero = routed) and optional dense
    probabilities [N, E] -> compact top-k IDs and weights; status[0] gets
    STATUS_MAP_OVERFLOW if a token routes to more than k experts."""
    ne, nk = p.n_tokens * p.n_experts, p.n_tokens * p.top_k
    m = _dev(routing_map, "routing_map", (torch.uint8, torch.bool), ne)
    pr = _dev(probs, "probs", (torch.float32,), ne) or None
    ids = _dev(topk_ids, "topk_ids", (torch.int32,), nk)
    w = _dev(topk_weights, "topk_weights", (torch.float32,), nk) or None
    st = _dev(status, "status", (torch.int32,), 1)
    _dev(workspace, "workspace", (torch.uint8,), moe_map_workspace_bytes(p))
    rc = lib.moe_routing_map_to_topk(ctypes.byref(p), m, pr, ids, w, st, workspace.data_ptr(),
                                     _stream(stream))
    _checked(rc, "moe_routing_map_to_topk")
