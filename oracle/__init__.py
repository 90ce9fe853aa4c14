"""CPU oracle of the routed-expert FP4 MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path never calls it, and it shares no code with the
GPU library: it has its own C implementation (oracle.c), built with gcc, and a
pure-Python scalar version (brute.py) for tiny shapes.

Every function follows the plain definition on the DeepSeek-V4.1-Flash pages
(10100.com page, section on the expert-capacity bottleneck: 6 of 384 experts
per token, w1/w2/w3 in FP4 E2M1 with UE8M0 scales, the byte shapes of each
tensor).  Where the pages are silent the readings stated at the top of
oracle.c apply.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "oracle.c")

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C")


def build(out: str = SO, src: str = SRC) -> str:
    """Compile oracle.c (or `src`, a copy of it: the mutation tests build copies
    with one planted mistake) into a shared library."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stderr}")
    return out


class _ACC(ctypes.Structure):
    """oracle_acc: the accumulation model an h bound is for (see oracle.c)."""
    _fields_ = [("sum", ctypes.c_double), ("prefix", ctypes.c_double), ("block", ctypes.c_int)]


def _acc(acc):
    """None (gamma_H), or (sum, prefix, block)."""
    if acc is None:
        return None
    s, p, b = acc
    return ctypes.byref(_ACC(float(s), float(p), int(b)))


class _OW(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_void_p)) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]


class Oracle:
    """ctypes view of one build of oracle.c."""

    def __init__(self, path: str = SO):
        if path == SO and not os.path.exists(SO):
            build()
        lib = ctypes.CDLL(path)
        lib.oracle_e2m1.restype = ctypes.c_double
        lib.oracle_e2m1.argtypes = [ctypes.c_int]
        lib.oracle_ue8m0.restype = ctypes.c_double
        lib.oracle_ue8m0.argtypes = [ctypes.c_int]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_route.restype = None
        lib.oracle_route.argtypes = [ctypes.c_int] * 3 + [_f32p, _i32p, _f32p]
        lib.oracle_permute.restype = None
        lib.oracle_permute.argtypes = [ctypes.c_int] * 3 + [_i32p] * 5
        lib.oracle_router_logits.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 4
        lib.oracle_router_logits.restype = None
        lib.oracle_saliency.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, _f32p,
                                                              ctypes.POINTER(_OW), ctypes.c_int,
                                                              ctypes.c_void_p, ctypes.c_void_p,
                                                              ctypes.c_int]
        lib.oracle_saliency.restype = ctypes.c_int
        lib.oracle_shared.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 12
        lib.oracle_shared.restype = None
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, _f32p,
                                      ctypes.POINTER(_OW), ctypes.c_int, ctypes.c_void_p,
                                      _f32p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_forward_mx8.restype = ctypes.c_int
        lib.oracle_forward_mx8.argtypes = lib.oracle_forward.argtypes
        lib.oracle_e4m3.restype = ctypes.c_double
        lib.oracle_e4m3.argtypes = [ctypes.c_int]
        lib.oracle_mx8_quant.restype = None
        lib.oracle_mx8_quant.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.oracle_prenorm.restype = None
        lib.oracle_prenorm.argtypes = [ctypes.c_int, ctypes.c_int, _f32p, ctypes.c_double,
                                       ctypes.c_void_p]
        lib.oracle_stack_layer.restype = ctypes.c_int
        lib.oracle_stack_layer.argtypes = [ctypes.c_int] * 5 + [_f32p, _f32p, ctypes.POINTER(_OW)]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib = lib

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        """Threads of the oracle's parallel loops from now on."""
        self.lib.oracle_set_threads(int(n))

    # ---------------------------------------------------------------- formats
    def e2m1(self, code: int) -> float:
        return self.lib.oracle_e2m1(code)

    def ue8m0(self, e: int) -> float:
        return self.lib.oracle_ue8m0(e)

    def to_bf16(self, v: float) -> int:
        return int(self.lib.oracle_double_to_bf16(float(v)))

    # ---------------------------------------------------------------- router
    def route(self, logits: np.ndarray, k: int):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        idx = np.empty((T, k), np.int32)
        g = np.empty((T, k), np.float32)
        self.lib.oracle_route(T, E, k, logits, idx, g)
        return idx, g

    def router_logits(self, x_bits: np.ndarray, w_bits: np.ndarray):
        """Router logits x . wr^T in double for bf16 bits x [T, H] and wr [E, H],
        and the fp32 summation bound of each (see oracle_router_logits)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
        T, H = x_bits.shape
        E = w_bits.shape[0]
        assert w_bits.shape[1] == H
        lg = np.empty((T, E), np.float64)
        b = np.empty((T, E), np.float64)
        self.lib.oracle_router_logits(T, H, E, x_bits.ctypes.data, w_bits.ctypes.data,
                                      lg.ctypes.data, b.ctypes.data)
        return lg, b

    def permute(self, idx: np.ndarray, E: int):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, k = idx.shape
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        sp = np.empty(T * k, np.int32)
        slot = np.empty(T * k, np.int32)
        self.lib.oracle_permute(T, E, k, idx, counts, offsets, sp, slot)
        return counts, offsets, sp, slot

    # ---------------------------------------------------------------- layer
    @staticmethod
    def _weights(experts: Dict[int, Dict[str, np.ndarray]], E: int):
        keep = []
        arrs = {}
        for n in ("w1", "s1", "w3", "s3", "w2", "s2"):
            a = (ctypes.c_void_p * E)()
            for e, t in experts.items():
                buf = np.ascontiguousarray(t[n], dtype=np.uint8)
                keep.append(buf)
                a[e] = buf.ctypes.data
            arrs[n] = a
        ow = _OW(**{n: ctypes.cast(arrs[n], ctypes.POINTER(ctypes.c_void_p)) for n in arrs})
        return ow, (keep, arrs)

    def e4m3(self, code: int) -> float:
        return self.lib.oracle_e4m3(code)

    def mx8_quant(self, v: np.ndarray):
        """MXFP8 blocks of 32 along the last axis: (E4M3 codes uint8, UE8M0 scales uint8)."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        assert v.shape[-1] % 32 == 0
        codes = np.empty(v.shape, np.uint8)
        scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
        self.lib.oracle_mx8_quant(v.size, v.ctypes.data, codes.ctypes.data, scales.ctypes.data)
        return codes, scales

    def forward(self, H: int, I: int, E: int, k: int, x_bits: np.ndarray, logits: np.ndarray,
                experts: Dict[int, Dict[str, np.ndarray]], tokens: Optional[Sequence[int]] = None,
                want_h: bool = False, mx8: bool = False, acc=None):
        """y for the listed tokens (default all).  `experts` maps expert id -> its six
        byte tensors; only experts the router selects for the listed tokens are needed.
        With mx8, x and the bf16 h are quantised to MXFP8 before the matrices that
        read them.  hbound bounds an fp32 evaluation of G and U under the
        accumulation model `acc` = (sum, prefix, block) (None: gamma_H, the
        products summed one by one in any order); see oracle_acc in oracle.c.
        Returns dict(y, idx, gates[, h, hpre, hbound])."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T = x_bits.shape[0]
        assert x_bits.shape == (T, H) and logits.shape == (T, E)
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        n_tok = T if tok is None else len(tok)
        y = np.empty((n_tok, H), np.float32)
        idx = np.empty((T, k), np.int32)
        g = np.empty((T, k), np.float32)
        h = np.zeros((T * k, I), np.uint16) if want_h else None
        hpre = np.zeros((T * k, I), np.float64) if want_h else None
        hbound = np.zeros((T * k, I), np.float64) if want_h else None
        ow, keep = self._weights(experts, E)
        args = (T, H, I, E, k, x_bits.ctypes.data, logits, ctypes.byref(ow), n_tok,
                None if tok is None else tok.ctypes.data, y,
                None if h is None else h.ctypes.data, None if hpre is None else hpre.ctypes.data,
                None if hbound is None else hbound.ctypes.data, idx.ctypes.data, g.ctypes.data)
        rc = (self.lib.oracle_forward_mx8 if mx8 else self.lib.oracle_forward)(*args, _acc(acc))
        del keep
        if rc != 0:
            raise KeyError("the router selected an expert whose weights were not given")
        out = {"y": y, "idx": idx, "gates": g}
        if want_h:
            out["h"], out["hpre"], out["hbound"] = h, hpre, hbound
        return out

    def saliency(self, H: int, I: int, E: int, k: int, x_bits: np.ndarray, logits: np.ndarray,
                 experts: Dict[int, Dict[str, np.ndarray]],
                 expert_list: Optional[Sequence[int]] = None, mx8: bool = False) -> np.ndarray:
        """Saliency of the listed experts (default: all E, and then every expert's
        weights are needed): for expert e, the sum over the pairs (t, j) routed to
        it of g[t][j] * ||Y_(t,j)||_2, Y the expert's output before the gate."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T = x_bits.shape[0]
        assert x_bits.shape == (T, H) and logits.shape == (T, E)
        lst = np.ascontiguousarray(np.arange(E) if expert_list is None else expert_list,
                                   dtype=np.int32)
        sal = np.empty(len(lst), np.float64)
        ow, keep = self._weights(experts, E)
        rc = self.lib.oracle_saliency(T, H, I, E, k, x_bits.ctypes.data, logits, ctypes.byref(ow),
                                      len(lst), lst.ctypes.data, sal.ctypes.data, int(mx8))
        del keep
        if rc != 0:
            raise KeyError("a listed expert's weights were not given")
        return sal

    def shared(self, x_bits: np.ndarray, sw: Dict[str, np.ndarray], want_h: bool = False,
               acc=None):
        """The shared expert's output y_s [T, H] (double) for bf16 bits x [T, H];
        sw holds w1, w3 [I, H] and w2 [H, I] E4M3 bytes with s1, s3 [I/32, H/32]
        and s2 [H/32, I/32] UE8M0 block scales.  With want_h also h (bf16 bits),
        hpre and hbound [T, I] (hbound under the accumulation model `acc`, as in forward)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        T, H = x_bits.shape
        I = sw["w1"].shape[0]
        t = {n: np.ascontiguousarray(sw[n], dtype=np.uint8) for n in ("w1", "s1", "w3", "s3", "w2", "s2")}
        assert t["w1"].shape == (I, H) and t["w3"].shape == (I, H) and t["w2"].shape == (H, I)
        assert t["s1"].shape == (I // 32, H // 32) and t["s2"].shape == (H // 32, I // 32)
        y = np.empty((T, H), np.float64)
        h = np.empty((T, I), np.uint16) if want_h else None
        hp = np.empty((T, I), np.float64) if want_h else None
        hb = np.empty((T, I), np.float64) if want_h else None
        ptr = lambda a: None if a is None else a.ctypes.data
        self.lib.oracle_shared(T, H, I, x_bits.ctypes.data, *(t[n].ctypes.data for n in
                               ("w1", "s1", "w3", "s3", "w2", "s2")), y.ctypes.data, ptr(h),
                               ptr(hp), ptr(hb), _acc(acc))
        out = {"y": y}
        if want_h:
            out["h"], out["hpre"], out["hbound"] = h, hp, hb
        return out

    def prenorm(self, x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        u = np.empty(x.shape, np.uint16)
        self.lib.oracle_prenorm(x.shape[0], x.shape[1], x, eps, u.ctypes.data)
        return u

    def stack_layer(self, I: int, E: int, k: int, x: np.ndarray, logits: np.ndarray,
                    experts: Dict[int, Dict[str, np.ndarray]]) -> np.ndarray:
        """x <- x + moe(prenorm(x)); returns the new x (float32)."""
        x = np.array(x, dtype=np.float32, copy=True, order="C")
        T, H = x.shape
        ow, keep = self._weights(experts, E)
        rc = self.lib.oracle_stack_layer(T, H, I, E, k, x,
                                         np.ascontiguousarray(logits, dtype=np.float32),
                                         ctypes.byref(ow))
        del keep
        if rc != 0:
            raise KeyError("the router selected an expert whose weights were not given")
        return x


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
