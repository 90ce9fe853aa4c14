"""The per-instruction accumulation bounds that the h checks rest on
(tests/accum.py), measured on the GPU.

Each probe runs one instruction of the kind the layer's kernels chain on
inputs chosen to stress its rounding (mixed magnitudes, heavy cancellation, an
accumulator far larger than the products) and compares the fp32 result with
the exact sum of its terms (float64: every term is a product of two short
significands, exact in double).  The largest error seen, relative to the sum of
the terms' absolute values, must stay within the bound the h checks use."""
import ctypes
import os

import numpy as np
import pytest

import accum
from gpu_common import say

pytestmark = pytest.mark.gpu

SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libaccum_probe.so")


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(SO)
    for f in (lib.probe_dot2, lib.probe_mfma_bf16, lib.probe_mfma_scale):
        f.restype = ctypes.c_int
    return lib


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(v):
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bf16(rng, shape, span):
    v = rng.standard_normal(shape) * np.ldexp(1.0, rng.integers(-span, span + 1, shape))
    return bf16_bits(v.astype(np.float32))


def rel_err_u(got, exact, absum):
    got = np.asarray(got, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(absum > 0, np.abs(got - exact) / absum, 0.0)
    return float(r.max()) / accum.U


def breakdown(name, got, exact, psum, cabs, pmax, classes):
    """Print the largest error of each input class relative to several scales:
    the terms' absolute sum, the largest term, and the exact result."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        for cname, sel in classes.items():
            e = err[sel]
            a = np.nanmax(np.where((psum + cabs)[sel] > 0, e / (psum + cabs)[sel], 0)) / accum.U
            b = np.nanmax(np.where(np.maximum(pmax, cabs)[sel] > 0, e / np.maximum(pmax, cabs)[sel], 0)) / accum.U
            c = np.nanmax(np.where(np.abs(exact[sel]) > 0, e / np.abs(exact[sel]), 0)) / accum.U
            d = np.nanmax(np.where(psum[sel] > 0, e / psum[sel], 0)) / accum.U
            say(f"    {name} [{cname}]: max err / (sum|p|+|c|) {a:.3f} u, / max(|p|max,|c|) {b:.3f} u, "
                f"/ |exact| {c:.3f} u, / sum|p| {d:.3f} u")


def test_dot2(probe):
    import torch
    rng = np.random.default_rng(101)
    n = 1 << 20
    a = rand_bf16(rng, (n, 2), 6)
    b = rand_bf16(rng, (n, 2), 6)
    p = bf16_val(a) * bf16_val(b)
    c = (rng.standard_normal(n) * np.abs(p).sum(1) * 2.0).astype(np.float32)
    # a third of the cases cancel: c close to -(p0 + p1)
    k = n // 3
    c[:k] = (-(p[:k, 0] + p[:k, 1]) * (1 + rng.standard_normal(k) * 2.0 ** -20)).astype(np.float32)
    # fused or not: 1 + 2^-24 + 2^-24 is 1 + 2^-23 with one rounding, 1 with two
    a[-1] = bf16_bits([1.0, 1.0])
    b[-1] = bf16_bits([2.0 ** -24, 2.0 ** -24])
    c[-1] = 1.0
    d = torch.empty(n, dtype=torch.float32, device="cuda")
    av, bv = a.view(np.uint32).reshape(n), b.view(np.uint32).reshape(n)
    assert probe.probe_dot2(ctypes.c_void_p(_dev(av).data_ptr()), ctypes.c_void_p(_dev(bv).data_ptr()),
                            ctypes.c_void_p(_dev(c).data_ptr()), ctypes.c_void_p(d.data_ptr()), n) == 0
    got = d.cpu().numpy()
    p = bf16_val(a) * bf16_val(b)
    exact = p.sum(1) + c.astype(np.float64)
    absum = np.abs(p).sum(1) + np.abs(c.astype(np.float64))
    e = rel_err_u(got, exact, absum)
    cls = {"cancel": np.arange(n) < k, "random": np.arange(n) >= k}
    breakdown("dot2", got, exact, np.abs(p).sum(1), np.abs(c.astype(np.float64)), np.abs(p).max(1), cls)
    say(f"  v_dot2c_f32_bf16: max error {e:.3f} u of the terms' absolute sum; "
        f"1 + 2^-24 + 2^-24 -> 1 + {(float(got[-1]) - 1.0) / 2.0 ** -24:.0f} * 2^-24")
    assert e <= accum.EPS_DOT2, e


def test_mfma_bf16(probe):
    import torch
    rng = np.random.default_rng(102)
    n = 1 << 13
    A = rand_bf16(rng, (n, 16, 32), 4)
    B = rand_bf16(rng, (n, 32, 16), 4)
    Av, Bv = bf16_val(A), bf16_val(B)
    prod = np.einsum("pik,pkj->pij", Av, Bv)
    absp = np.einsum("pik,pkj->pij", np.abs(Av), np.abs(Bv))
    C = (rng.standard_normal((n, 16, 16)) * absp).astype(np.float32)
    k = n // 3
    C[:k] = (-prod[:k] * (1 + rng.standard_normal((k, 16, 16)) * 2.0 ** -20)).astype(np.float32)
    # an accumulator 2^20 times the products
    C[k:2 * k] = (rng.standard_normal((k, 16, 16)) * absp[k:2 * k] * 2.0 ** 20).astype(np.float32)
    C[n - 64:] = 0.0
    D = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    assert probe.probe_mfma_bf16(ctypes.c_void_p(_dev(A).data_ptr()), ctypes.c_void_p(_dev(B).data_ptr()),
                                 ctypes.c_void_p(_dev(C).data_ptr()), ctypes.c_void_p(D.data_ptr()),
                                 n) == 0
    got = D.cpu().numpy()
    exact = prod + C.astype(np.float64)
    absum = absp + np.abs(C.astype(np.float64))
    e = rel_err_u(got, exact, absum)
    pmax = np.einsum("pik,pkj->pijk", np.abs(Av), np.abs(Bv)).max(-1)
    ids = np.arange(n)[:, None, None] + np.zeros((1, 16, 16), int)
    cls = {"cancel": ids < k, "C=2^20 p": (ids >= k) & (ids < 2 * k), "C~p": (ids >= 2 * k) & (ids < n - 64),
           "C=0": ids >= n - 64}
    breakdown("mfma_bf16", got, exact, absp, np.abs(C.astype(np.float64)), pmax, cls)
    say(f"  v_mfma_f32_16x16x32_bf16: max error {e:.3f} u of the terms' absolute sum")
    assert e <= accum.EPS_MFMA_BF16, e


E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def e4m3_values():
    c = np.arange(256)
    e, m = (c >> 3) & 15, c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where(c & 0x80, -v, v)


def test_mfma_scale(probe):
    import torch
    rng = np.random.default_rng(103)
    n = 1 << 13
    A = rng.integers(0, 256, (n, 16, 64), dtype=np.uint8)
    sa = rng.integers(118, 127, (n, 16, 4), dtype=np.uint8)
    Bc = rng.integers(0, 254, (n, 16, 128))
    Bc = np.where(Bc >= 0x7F, Bc + 1, Bc).astype(np.uint8)          # no NaN codes
    sb = rng.integers(118, 127, (n, 16, 4), dtype=np.uint8)
    codes = np.stack([A & 15, A >> 4], -1).reshape(n, 16, 128)
    Aval = E2M1[codes] * np.repeat(np.ldexp(1.0, sa.astype(np.int64) - 127), 32, axis=2)
    Bval = e4m3_values()[Bc] * np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=2)
    prod = np.einsum("pik,pjk->pij", Aval, Bval)
    absp = np.einsum("pik,pjk->pij", np.abs(Aval), np.abs(Bval))
    C = (rng.standard_normal((n, 16, 16)) * absp * 0.1).astype(np.float32)
    k = n // 3
    C[:k] = (-prod[:k] * (1 + rng.standard_normal((k, 16, 16)) * 2.0 ** -20)).astype(np.float32)
    C[2 * k:] = (rng.standard_normal((n - 2 * k, 16, 16)) * absp[2 * k:] * 2.0 ** 10).astype(np.float32)
    C[n - 64:] = 0.0
    D = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    keep = [_dev(x) for x in (A, sa, Bc, sb, C)]
    args = [ctypes.c_void_p(t.data_ptr()) for t in keep]
    assert probe.probe_mfma_scale(*args, ctypes.c_void_p(D.data_ptr()), n) == 0
    got = D.cpu().numpy()
    exact = prod + C.astype(np.float64)
    absum = absp + np.abs(C.astype(np.float64))
    e = rel_err_u(got, exact, absum)
    pmax = np.einsum("pik,pjk->pijk", np.abs(Aval), np.abs(Bval)).max(-1)
    ids = np.arange(n)[:, None, None] + np.zeros((1, 16, 16), int)
    cls = {"cancel": ids < k, "C~0.1p": (ids >= k) & (ids < 2 * k), "C=2^10 p": (ids >= 2 * k) & (ids < n - 64),
           "C=0": ids >= n - 64}
    breakdown("mfma_scale", got, exact, absp, np.abs(C.astype(np.float64)), pmax, cls)
    say(f"  v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E4M3): max error {e:.1f} u "
        f"(2^{np.log2(max(e, 1e-30)) - 24:.2f}) of the terms' absolute sum")
    assert e <= accum.EPS_MFMA_SCALE, e
