"""Seeded synthetic inputs for the FP4 routed-expert MoE layer.

This package is shared by the tests, the benchmark and the oracle's checks.  It
holds input generation only -- none of the MoE arithmetic:

* expert weights: a counter-based SplitMix64 byte stream (see gen_host.c),
  identical on host (C, OpenMP) and device (HIP), so a multi-gigabyte layer is
  made in HBM while the oracle regenerates just the experts it needs;
* activations x: numpy PCG64 N(0,1) draws rounded to bf16 (round to nearest
  even), returned as raw uint16 bit patterns;
* router logits: PCG64 N(0,1) draws plus an optional per-expert Zipf-shaped bias.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Tuple

import numpy as np

from .configs import ZIPF_ALPHA, Workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libsynth_host.so")
DEV_SO = os.path.join(_HERE, "libsynth_dev.so")

# tensor ids of the generator streams
W1, S1, W3, S3, W2, S2 = range(6)
TENSOR_NAMES = ("w1", "s1", "w3", "s3", "w2", "s2")


def tensor_shapes(H: int, I: int) -> Dict[str, Tuple[int, int]]:
    """Per-expert [rows, cols] byte shapes of the six checkpoint tensors."""
    return {"w1": (I, H // 2), "s1": (I, H // 32), "w3": (I, H // 2), "s3": (I, H // 32),
            "w2": (H, I // 2), "s2": (H, I // 32)}


# --------------------------------------------------------------------------- build
def build(verbose: bool = False) -> None:
    """Compile the host and device generator libraries in place."""
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", HOST_SO,
         os.path.join(_HERE, "gen_host.c")],
        ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", DEV_SO, os.path.join(_HERE, "gen_device.hip")],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"synth build failed: {' '.join(c)}\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(c))


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            build()
        lib = ctypes.CDLL(HOST_SO)
        lib.synth_sm64_at.restype = ctypes.c_uint64
        lib.synth_sm64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_stream.restype = ctypes.c_uint64
        lib.synth_stream.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.c_uint32]
        lib.synth_fill.restype = None
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_SO):
            raise RuntimeError(f"{DEV_SO} is not built; run synth.build()")
        lib = ctypes.CDLL(DEV_SO)
        lib.synth_fill_tensor_dev.restype = ctypes.c_int
        lib.synth_fill_tensor_dev.argtypes = [
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
            ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p]
        _dev = lib
    return _dev


def sm64_at(state: int, i: int) -> int:
    return int(_host_lib().synth_sm64_at(state, i))


def stream(seed: int, layer: int, expert: int, tensor: int) -> int:
    return int(_host_lib().synth_stream(seed & (2**64 - 1), layer, expert, tensor))


# --------------------------------------------------------------------------- weights
def expert_host(wl: Workload, layer: int, expert: int) -> Dict[str, np.ndarray]:
    """The six byte tensors of one expert, generated on the host."""
    lib = _host_lib()
    out = {}
    for tid, name in enumerate(TENSOR_NAMES):
        rows, cols = tensor_shapes(wl.H, wl.I)[name]
        a = np.empty((rows, cols), dtype=np.uint8)
        st = lib.synth_stream(wl.weight_seed, layer, expert, tid)
        kind = tid & 1
        lib.synth_fill(a.ctypes.data, 0, a.size, st, kind, wl.scale_lo, wl.scale_hi)
        out[name] = a
    return out


def layer_host(wl: Workload, layer: int = 0, experts=None) -> Dict[str, np.ndarray]:
    """Dense [E, rows, cols] host tensors for the listed experts (default: all)."""
    experts = range(wl.E) if experts is None else experts
    per = [expert_host(wl, layer, e) for e in experts]
    return {n: np.stack([p[n] for p in per]) for n in TENSOR_NAMES}


def layer_device(wl: Workload, layer: int = 0, device="cuda", n_experts: int | None = None):
    """Dense [E, rows, cols] uint8 torch tensors for one layer, generated in HBM."""
    import torch
    E = wl.E if n_experts is None else n_experts
    lib = _dev_lib()
    stream_ptr = torch.cuda.current_stream(device).cuda_stream
    out = {}
    for tid, name in enumerate(TENSOR_NAMES):
        rows, cols = tensor_shapes(wl.H, wl.I)[name]
        t = torch.empty((E, rows, cols), dtype=torch.uint8, device=device)
        rc = lib.synth_fill_tensor_dev(t.data_ptr(), E, rows * cols, rows * cols, wl.weight_seed,
                                       layer, 0, tid, tid & 1, wl.scale_lo, wl.scale_hi, stream_ptr)
        if rc != 0:
            raise RuntimeError(f"synth_fill_tensor_dev failed with hipError {rc}")
        out[name] = t
    return out


# --------------------------------------------------------------------------- activations
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(k) & (2**63 - 1) for k in key]))


def gen_x(wl: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    """x for one step: [T, H] bf16 bit patterns of N(0,1) draws."""
    x = _rng(wl.input_seed, 1, step, layer).standard_normal((wl.T, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def gen_x_f32(wl: Workload, step: int = 0) -> np.ndarray:
    """fp32 residual-stream input x_0 for the layer stack: [T, H] N(0,1)."""
    return _rng(wl.input_seed, 3, step).standard_normal((wl.T, wl.H), dtype=np.float32)


def logit_bias(wl: Workload, layer: int = 0) -> np.ndarray:
    """Per-expert Zipf-shaped bias -alpha*s*ln(r_e), r a seeded permutation of 1..E."""
    if wl.zipf_s == 0.0:
        return np.zeros(wl.E, dtype=np.float64)
    r = 1 + _rng(wl.input_seed, 2, layer).permutation(wl.E)
    return -ZIPF_ALPHA * wl.zipf_s * np.log(r.astype(np.float64))


def gen_router(wl: Workload, layer: int = 0) -> np.ndarray:
    """Router weight for the router-logits step: [E, H] bf16 bit patterns of
    N(0, 1/H) draws, so that logits of N(0,1) activations are about N(0,1)."""
    w = _rng(wl.input_seed, 4, layer).standard_normal((wl.E, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(w * np.float32(1.0 / np.sqrt(wl.H)))


def gen_shared(wl: Workload, layer: int = 0) -> dict:
    """Shared-expert tensors of one layer, intermediate size wl.I: E4M3 codes
    uniform over the 254 non-NaN codes (w1, w3 [I, H], w2 [H, I]) and UE8M0
    32 x 32 block scales uniform in [113, 115] (s1, s3 [I/32, H/32], s2
    [H/32, I/32]), which keeps the projections of N(0,1) activations O(1)."""
    rng = _rng(wl.weight_seed, 5, layer)
    H, I = wl.H, wl.I

    def codes(shape):
        c = rng.integers(0, 254, shape, dtype=np.int32)
        return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)

    def scales(shape):
        return rng.integers(113, 116, shape, dtype=np.int32).astype(np.uint8)

    return {"w1": codes((I, H)), "s1": scales((I // 32, H // 32)),
            "w3": codes((I, H)), "s3": scales((I // 32, H // 32)),
            "w2": codes((H, I)), "s2": scales((H // 32, I // 32))}


def gen_logits(wl: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    """Router logits for one step: [T, E] float32 = N(0,1) noise + per-expert bias."""
    noise = _rng(wl.input_seed, 0, step, layer).standard_normal((wl.T, wl.E), dtype=np.float32)
    return (noise.astype(np.float64) + logit_bias(wl, layer)[None, :]).astype(np.float32)
