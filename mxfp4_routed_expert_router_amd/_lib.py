"""ctypes binding of libmoe_fp4.so.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  If the
native library is missing this module raises at import time; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp4.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP = range(6)
MODE_AUTO, MODE_DECODE, MODE_PREFILL, MODE_PREFILL_MXFP8 = 0, 1, 2, 3
(PATH_DECODE_ONE, PATH_DECODE_FEW, PATH_DECODE_MFMA, PATH_PREFILL,
 PATH_PREFILL_MXFP8) = 1, 2, 3, 4, 5
ACCUMULATE = 1
TENSORS = ("w1", "s1", "w3", "s3", "w2", "s2")


class MoeFp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TENSORS] + [("expert_stride", ctypes.c_int64 * 6)]


class SharedWeightsStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TENSORS] + [("I", ctypes.c_int32)]


class RouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m "
                          f"mxfp4_routed_expert_router_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_fp4_workspace_size.argtypes = [ctypes.POINTER(Dims), I32, ctypes.POINTER(SZ)]
    lib.moe_fp4_route.argtypes = [ctypes.POINTER(Dims), P, ctypes.POINTER(RouteOut), P, SZ, P]
    lib.moe_fp4_route_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(SZ)]
    lib.moe_fp4_plan.argtypes = [ctypes.POINTER(Dims), I32, ctypes.POINTER(I32)]
    lib.moe_fp4_forward_noalloc.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(Weights), P,
                                            I32, I32, P]
    lib.moe_fp4_forward.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(Weights), P, I32,
                                    I32, P, SZ, P]
    lib.moe_fp4_forward_debug.argtypes = lib.moe_fp4_forward.argtypes + [P, ctypes.POINTER(RouteOut)]
    lib.moe_fp4_forward_profiled.argtypes = lib.moe_fp4_forward.argtypes + [P, I32]
    lib.moe_fp4_forward_profiled.restype = ctypes.c_int
    lib.moe_fp4_prenorm_bf16.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P]
    lib.moe_fp4_status_string.argtypes = [I32]
    lib.moe_fp4_quant_mxfp8.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.moe_fp4_router_logits.argtypes = [ctypes.POINTER(Dims), P, P, P, P]
    lib.moe_fp4_forward_routed.argtypes = lib.moe_fp4_forward.argtypes
    lib.moe_fp4_shared_expert.argtypes = [ctypes.POINTER(Dims), P, ctypes.POINTER(SharedWeightsStruct),
                                          P, I32, P, P]
    lib.moe_fp4_forward_shared.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(Weights),
                                           ctypes.POINTER(SharedWeightsStruct), P, I32, I32, P, SZ, P]
    lib.moe_fp4_forward_residual.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(Weights),
                                             I32, P, SZ, P]
    lib.moe_fp4_forward_saliency.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(Weights),
                                             P, P, I32, I32, P, SZ, P]
    lib.moe_fp4_status_string.restype = ctypes.c_char_p
    for f in ("moe_fp4_workspace_size", "moe_fp4_route", "moe_fp4_forward", "moe_fp4_plan",
              "moe_fp4_route_workspace_size", "moe_fp4_forward_noalloc",
              "moe_fp4_forward_debug", "moe_fp4_prenorm_bf16", "moe_fp4_quant_mxfp8",
              "moe_fp4_router_logits", "moe_fp4_forward_routed", "moe_fp4_forward_saliency",
              "moe_fp4_shared_expert", "moe_fp4_forward_shared", "moe_fp4_forward_residual"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.moe_fp4_status_string(status).decode()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(rc: int, what: str):
    if rc != OK:
        raise MoeFp4Error(rc, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


@dataclass
class ExpertWeights:
    """The six checkpoint tensors of E experts (uint8, on the GPU).

    Dense tensors are [E, rows, cols]; `strides` (bytes between experts, per
    tensor) lets the experts live anywhere, e.g. one blob per expert, and then
    the intermediate size `I` must be given."""
    w1: torch.Tensor
    s1: torch.Tensor
    w3: torch.Tensor
    s3: torch.Tensor
    w2: torch.Tensor
    s2: torch.Tensor
    strides: Optional[tuple] = None
    I: Optional[int] = None

    def intermediate(self) -> int:
        if self.I is not None:
            return int(self.I)
        if self.w1.dim() == 3:
            return int(self.w1.shape[1])
        raise ValueError("ExpertWeights: give I= when the tensors are not dense [E, rows, cols]")

    @classmethod
    def from_dict(cls, d: Dict[str, torch.Tensor]) -> "ExpertWeights":
        return cls(**{n: d[n] for n in TENSORS})

    def as_struct(self) -> Weights:
        w = Weights()
        for n in TENSORS:
            t = getattr(self, n)
            if t.dtype != torch.uint8 or t.device.type != "cuda":
                raise TypeError(f"weight tensor {n} must be uint8 on the GPU")
            setattr(w, n, t.data_ptr())
        st = self.strides or (0,) * 6
        for i in range(6):
            w.expert_stride[i] = int(st[i])
        return w


@dataclass
class Route:
    topk_idx: torch.Tensor
    gates: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pairs: torch.Tensor
    pair_slot: torch.Tensor

    @classmethod
    def empty(cls, T: int, E: int, k: int, device) -> "Route":
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                   torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32),
                   torch.empty(T * k, **i32))

    def as_struct(self) -> RouteOut:
        r = RouteOut()
        for n in ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot"):
            setattr(r, n, getattr(self, n).data_ptr())
        return r


def moe_fp4_workspace_size(T: int, H: int, I: int, E: int, k: int, mode: int = MODE_AUTO) -> int:
    n = ctypes.c_size_t()
    _check(_lib.moe_fp4_workspace_size(ctypes.byref(Dims(T, H, I, E, k)), mode, ctypes.byref(n)),
           "moe_fp4_workspace_size")
    return n.value


def moe_fp4_plan(T: int, H: int, I: int, E: int, k: int, mode: int = MODE_AUTO) -> int:
    """The kernel path (PATH_*) moe_fp4_forward takes for these sizes and mode."""
    path = ctypes.c_int()
    _check(_lib.moe_fp4_plan(ctypes.byref(Dims(T, H, I, E, k)), mode, ctypes.byref(path)),
           "moe_fp4_plan")
    return path.value


def moe_fp4_route_workspace_size(T: int, E: int, k: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.moe_fp4_route_workspace_size(ctypes.byref(Dims(T, 0, 0, E, k)), ctypes.byref(n)),
           "moe_fp4_route_workspace_size")
    return n.value


def moe_fp4_route(logits: torch.Tensor, k: int, workspace: Optional[torch.Tensor] = None) -> Route:
    _need(logits, "logits", (torch.float32,), 2)
    T, E = logits.shape
    out = Route.empty(T, E, k, logits.device)
    rs = out.as_struct()
    nws = moe_fp4_route_workspace_size(T, E, k)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=logits.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.moe_fp4_route(ctypes.byref(Dims(T, 0, 0, E, k)), logits.data_ptr(),
                              ctypes.byref(rs), ws_ptr, ws_n, _stream(logits)), "moe_fp4_route")
    return out


def _forward(x, logits, weights: ExpertWeights, k, y, mode, accumulate, workspace, debug):
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(logits, "logits", (torch.float32,), 2)
    T, H = x.shape
    E = logits.shape[0 + 1]
    if logits.shape[0] != T:
        raise ValueError("x and logits disagree on the number of tokens")
    I = weights.intermediate()
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    need = moe_fp4_workspace_size(T, H, I, E, k, mode)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    dims = Dims(T, H, I, E, k)
    ws = weights.as_struct()
    flags = ACCUMULATE if accumulate else 0
    if not debug:
        _check(_lib.moe_fp4_forward(ctypes.byref(dims), x.data_ptr(), logits.data_ptr(),
                                    ctypes.byref(ws), y.data_ptr(), mode, flags,
                                    workspace.data_ptr(), workspace.numel(), _stream(x)),
               "moe_fp4_forward")
        return y
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=x.device)
    route = Route.empty(T, E, k, x.device)
    rs = route.as_struct()
    _check(_lib.moe_fp4_forward_debug(ctypes.byref(dims), x.data_ptr(), logits.data_ptr(),
                                      ctypes.byref(ws), y.data_ptr(), mode, flags,
                                      workspace.data_ptr(), workspace.numel(), _stream(x),
                                      h.data_ptr(), ctypes.byref(rs)), "moe_fp4_forward_debug")
    return y, h, route


def moe_fp4_forward(x: torch.Tensor, logits: torch.Tensor, weights: ExpertWeights, k: int,
                    y: Optional[torch.Tensor] = None, mode: int = MODE_AUTO,
                    accumulate: bool = False, workspace: Optional[torch.Tensor] = None):
    """y [T, H] fp32 = the layer applied to x [T, H] (bf16 bits) routed by logits [T, E]."""
    return _forward(x, logits, weights, k, y, mode, accumulate, workspace, False)


def moe_fp4_forward_debug(x, logits, weights: ExpertWeights, k: int, y=None, mode=MODE_AUTO,
                          accumulate=False, workspace=None):
    """As moe_fp4_forward; also returns h [T*k, I] (bf16, pair order) and the Route."""
    return _forward(x, logits, weights, k, y, mode, accumulate, workspace, True)


class StageEvents:
    """Eight HIP events for moe_fp4_forward_profiled (created with timing on):
    start and end of the kernels of routing, w1/w3, w2 and combine."""

    N = 8

    def __init__(self):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(self.N)]
        for e in self.events:
            e.record()  # materialise the underlying hipEvent_t
        self._arr = (ctypes.c_void_p * self.N)(*[e.cuda_event for e in self.events])

    def stage_ms(self):
        """Kernel ms of routing, w1/w3, w2, combine (after a sync)."""
        ev = self.events
        return [ev[2 * s].elapsed_time(ev[2 * s + 1]) for s in range(4)]

    def span_ms(self):
        """ms from the start of routing to the end of the combine."""
        return self.events[0].elapsed_time(self.events[-1])


def moe_fp4_forward_noalloc(x, logits, weights: ExpertWeights, k: int, y=None, mode=MODE_AUTO,
                            accumulate=False):
    """As moe_fp4_forward with the library's static per-GPU workspace (no
    allocation inside the library; y is allocated here only when not given)."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(logits, "logits", (torch.float32,), 2)
    T, H = x.shape
    E = logits.shape[1]
    I = weights.intermediate()
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    ws = weights.as_struct()
    _check(_lib.moe_fp4_forward_noalloc(
        ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(), logits.data_ptr(), ctypes.byref(ws),
        y.data_ptr(), mode, ACCUMULATE if accumulate else 0, _stream(x)), "moe_fp4_forward_noalloc")
    return y


def moe_fp4_forward_profiled(x, logits, weights: ExpertWeights, k: int, events: StageEvents,
                             y=None, mode=MODE_AUTO, accumulate=False, workspace=None):
    """As moe_fp4_forward, timing the kernels of each stage with `events`."""
    T, H = x.shape
    E = logits.shape[1]
    I = weights.intermediate()
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    need = moe_fp4_workspace_size(T, H, I, E, k, mode)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws = weights.as_struct()
    _check(_lib.moe_fp4_forward_profiled(
        ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(), logits.data_ptr(), ctypes.byref(ws),
        y.data_ptr(), mode, ACCUMULATE if accumulate else 0, workspace.data_ptr(),
        workspace.numel(), _stream(x), events._arr, events.N), "moe_fp4_forward_profiled")
    return y


def moe_fp4_prenorm_bf16(x: torch.Tensor, eps: float = 1e-6,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(x, "x", (torch.float32,), 2)
    T, H = x.shape
    u = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(_lib.moe_fp4_prenorm_bf16(x.data_ptr(), u.data_ptr(), T, H, eps, _stream(x)),
           "moe_fp4_prenorm_bf16")
    return u


def moe_fp4_router_logits(x: torch.Tensor, w_router: torch.Tensor,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Router logits [T, E] fp32 = x [T, H] . w_router [E, H]^T (both bf16)."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(w_router, "w_router", (torch.bfloat16, torch.int16, torch.uint16), 2)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("x and w_router disagree on the hidden size")
    lg = out if out is not None else torch.empty((T, E), dtype=torch.float32, device=x.device)
    _need(lg, "logits", (torch.float32,), 2)
    _check(_lib.moe_fp4_router_logits(ctypes.byref(Dims(T, H, 0, E, 0)), x.data_ptr(),
                                      w_router.data_ptr(), lg.data_ptr(), _stream(x)),
           "moe_fp4_router_logits")
    return lg


def moe_fp4_forward_routed(x: torch.Tensor, w_router: torch.Tensor, weights: ExpertWeights, k: int,
                           y: Optional[torch.Tensor] = None, mode: int = MODE_AUTO,
                           accumulate: bool = False, workspace: Optional[torch.Tensor] = None):
    """As moe_fp4_forward, with the logits computed from x and w_router [E, H] (bf16)."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(w_router, "w_router", (torch.bfloat16, torch.int16, torch.uint16), 2)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("x and w_router disagree on the hidden size")
    I = weights.intermediate()
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    need = moe_fp4_workspace_size(T, H, I, E, k, mode)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws = weights.as_struct()
    _check(_lib.moe_fp4_forward_routed(ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(),
                                       w_router.data_ptr(), ctypes.byref(ws), y.data_ptr(), mode,
                                       ACCUMULATE if accumulate else 0, workspace.data_ptr(),
                                       workspace.numel(), _stream(x)), "moe_fp4_forward_routed")
    return y


def moe_fp4_forward_saliency(x: torch.Tensor, logits: torch.Tensor, weights: ExpertWeights, k: int,
                             saliency: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                             mode: int = MODE_PREFILL, accumulate: bool = False,
                             workspace: Optional[torch.Tensor] = None):
    """As moe_fp4_forward (prefill modes), also adding each expert's saliency --
    sum over its pairs of gate * ||expert output||_2 -- to `saliency` [E] fp32
    (zeros if None).  Returns (y, saliency)."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(logits, "logits", (torch.float32,), 2)
    T, H = x.shape
    E = logits.shape[1]
    I = weights.intermediate()
    if saliency is None:
        saliency = torch.zeros(E, dtype=torch.float32, device=x.device)
    _need(saliency, "saliency", (torch.float32,), 1)
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    run = MODE_PREFILL if mode == MODE_AUTO else mode
    need = moe_fp4_workspace_size(T, H, I, E, k, run)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws = weights.as_struct()
    _check(_lib.moe_fp4_forward_saliency(ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(),
                                         logits.data_ptr(), ctypes.byref(ws), y.data_ptr(),
                                         saliency.data_ptr(), mode, ACCUMULATE if accumulate else 0,
                                         workspace.data_ptr(), workspace.numel(), _stream(x)),
           "moe_fp4_forward_saliency")
    return y, saliency


@dataclass
class SharedWeights:
    """The shared expert's tensors (uint8, on the GPU): w1, w3 [I, H] and w2 [H, I]
    E4M3 codes; s1, s3 [I/32, H/32] and s2 [H/32, I/32] UE8M0 block scales."""
    w1: torch.Tensor
    s1: torch.Tensor
    w3: torch.Tensor
    s3: torch.Tensor
    w2: torch.Tensor
    s2: torch.Tensor

    @classmethod
    def from_dict(cls, d: Dict[str, torch.Tensor]) -> "SharedWeights":
        return cls(**{n: d[n] for n in TENSORS})

    def as_struct(self) -> SharedWeightsStruct:
        sw = SharedWeightsStruct()
        for n in TENSORS:
            t = getattr(self, n)
            if t.dtype != torch.uint8 or t.device.type != "cuda" or not t.is_contiguous():
                raise TypeError(f"shared weight tensor {n} must be contiguous uint8 on the GPU")
            setattr(sw, n, t.data_ptr())
        sw.I = int(self.w1.shape[0])
        return sw


def moe_fp4_shared_expert(x: torch.Tensor, shared: SharedWeights, y: Optional[torch.Tensor] = None,
                          accumulate: bool = False, h: Optional[torch.Tensor] = None):
    """The shared expert alone: y [T, H] (+)= W2 bf16(silu(W1 x) * (W3 x)).
    Returns (y, h) with h [T, I] bf16."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    T, H = x.shape
    I = int(shared.w1.shape[0])
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    if h is None:
        h = torch.empty((T, I), dtype=torch.bfloat16, device=x.device)
    sw = shared.as_struct()
    _check(_lib.moe_fp4_shared_expert(ctypes.byref(Dims(T, H, 0, 0, 0)), x.data_ptr(),
                                      ctypes.byref(sw), y.data_ptr(),
                                      ACCUMULATE if accumulate else 0, h.data_ptr(), _stream(x)),
           "moe_fp4_shared_expert")
    return y, h


def moe_fp4_forward_shared(x: torch.Tensor, logits: torch.Tensor, weights: ExpertWeights,
                           shared: SharedWeights, k: int, y: Optional[torch.Tensor] = None,
                           mode: int = MODE_AUTO, accumulate: bool = False,
                           workspace: Optional[torch.Tensor] = None):
    """The routed layer plus the shared expert: y (+)= sum_j g_j Y_j + W2s h_s."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _need(logits, "logits", (torch.float32,), 2)
    T, H = x.shape
    E = logits.shape[1]
    I = weights.intermediate()
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs y")
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(y, "y", (torch.float32,), 2)
    need = moe_fp4_workspace_size(T, H, I, E, k, mode)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws, sw = weights.as_struct(), shared.as_struct()
    _check(_lib.moe_fp4_forward_shared(ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(),
                                       logits.data_ptr(), ctypes.byref(ws), ctypes.byref(sw),
                                       y.data_ptr(), mode, ACCUMULATE if accumulate else 0,
                                       workspace.data_ptr(), workspace.numel(), _stream(x)),
           "moe_fp4_forward_shared")
    return y


def moe_fp4_forward_residual(x: torch.Tensor, logits: torch.Tensor, weights: ExpertWeights, k: int,
                             mode: int = MODE_AUTO, workspace: Optional[torch.Tensor] = None):
    """One residual layer in place: x [T, H] fp32 += layer(bf16(x / rms(x)))."""
    _need(x, "x", (torch.float32,), 2)
    _need(logits, "logits", (torch.float32,), 2)
    T, H = x.shape
    E = logits.shape[1]
    I = weights.intermediate()
    need = moe_fp4_workspace_size(T, H, I, E, k, mode)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws = weights.as_struct()
    _check(_lib.moe_fp4_forward_residual(ctypes.byref(Dims(T, H, I, E, k)), x.data_ptr(),
                                         logits.data_ptr(), ctypes.byref(ws), mode,
                                         workspace.data_ptr(), workspace.numel(), _stream(x)),
           "moe_fp4_forward_residual")
    return x


def moe_fp4_quant_mxfp8(x: torch.Tensor):
    """MXFP8 quantisation of bf16 rows [rows, K] (blocks of 32 along K):
    returns (E4M3 codes uint8 [rows, K], UE8M0 scales uint8 [rows, K/32])."""
    _need(x, "x", (torch.bfloat16,), 2)
    rows, K = x.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.moe_fp4_quant_mxfp8(x.data_ptr(), rows, K, codes.data_ptr(), scales.data_ptr(),
                                    _stream(x)), "moe_fp4_quant_mxfp8")
    return codes, scales
