"""Pins of the CPU oracle: checks against facts fixed outside the oracle itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with what the pages, the format specification, a library routine or
hand-computed closed forms fix.  tests/test_oracle.py runs them all on the real
oracle; tests/test_oracle_mutants.py runs them on copies of the oracle with one
planted mistake each and requires that every mistake is caught by some pin.
"""
from __future__ import annotations

import math
import os
import struct

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


def bf16_bits(v: float) -> int:
    """bf16 bit pattern of a value that is exactly representable in bf16."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    assert u & 0xFFFF == 0, v
    return u >> 16


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


# ------------------------------------------------------------------ helpers
def const_expert(H, I, w1, w3, w2, s1=127, s3=127, s2=127):
    """Expert whose every nibble of a tensor holds the same E2M1 code."""
    def nib(code, rows, cols):
        return np.full((rows, cols // 2), code | (code << 4), np.uint8)
    return {"w1": nib(w1, I, H), "s1": np.full((I, H // 32), s1, np.uint8),
            "w3": nib(w3, I, H), "s3": np.full((I, H // 32), s3, np.uint8),
            "w2": nib(w2, H, I), "s2": np.full((H, I // 32), s2, np.uint8)}


def random_expert(rng, H, I, lo=120, hi=124):
    return {"w1": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
            "s1": rng.integers(lo, hi + 1, (I, H // 32), dtype=np.uint8),
            "w3": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
            "s3": rng.integers(lo, hi + 1, (I, H // 32), dtype=np.uint8),
            "w2": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
            "s2": rng.integers(lo, hi + 1, (H, I // 32), dtype=np.uint8)}


def set_nibble(w, r, c, code):
    b = int(w[r, c // 2])
    if c % 2:
        b = (b & 0x0F) | (code << 4)
    else:
        b = (b & 0xF0) | code
    w[r, c // 2] = b


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ formats
def pin_e2m1_table(o):
    """16 codes against the OCP MX v1.0 E2M1 facts (tests/golden/mx_formats.txt)."""
    g = read_golden("mx_formats.txt")
    pos = g["e2m1_positive"]
    for c in range(8):
        assert o.e2m1(c) == pos[c], (c, o.e2m1(c))
        neg = o.e2m1(c + 8)
        assert neg == -pos[c] and math.copysign(1.0, neg) == -1.0, (c + 8, neg)
    vals = [o.e2m1(c) for c in range(16)]
    assert max(vals) == g["e2m1_max_normal"][0]
    assert min(v for v in vals if v >= 1.0) == g["e2m1_min_normal"][0]
    sub = [v for v in vals if 0 < v < 1.0]
    assert max(sub) == g["e2m1_max_subnormal"][0] and min(sub) == g["e2m1_min_subnormal"][0]


def pin_ue8m0(o):
    """All 256 scale bytes against torch's float8_e8m0fnu decode (a library routine)."""
    import torch
    g = read_golden("mx_formats.txt")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    for e in range(256):
        v = o.ue8m0(e)
        r = float(ref[e])
        if e == int(g["e8m0_nan"][0]):
            assert math.isnan(v) and math.isnan(r)
        else:
            assert v == r, (e, v, r)
    assert o.ue8m0(int(g["e8m0_bias"][0])) == 1.0


def pin_bf16_rounding(o):
    """double -> bf16 against the exact rational rounding of brute.to_bf16_bits."""
    rng = np.random.default_rng(7)
    vals = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -40,
            2.0 ** -130, 2.0 ** -133 * 1.5, 2.0 ** -134, 3.3961e38, 3.4e38, -3.4e38, 1e-45,
            0.0, -0.0, 255.5, 256.5, 71.99955]
    vals += list(rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300))
    for v in vals:
        a, b = o.to_bf16(v), brute.to_bf16_bits(v)
        assert a == b, (v, hex(a), hex(b))
    assert o.to_bf16(float("inf")) == 0x7F80 and o.to_bf16(float("-inf")) == 0xFF80
    assert (o.to_bf16(float("nan")) & 0x7F80) == 0x7F80 and (o.to_bf16(float("nan")) & 0x7F)


# ------------------------------------------------------------------ router
def pin_router_vs_sort(o):
    """Top-k = first k of numpy's stable argsort of -logits; gates = scipy softmax."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    T, E, k = 64, 37, 5
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, 3] = lg[:, 20]          # exact ties
    lg[::3, 7] = -0.0
    lg[::3, 2] = 0.0              # -0 vs +0 tie
    lg[5, :] = lg[5, 0]           # a fully tied row
    idx, g = o.route(lg, k)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref)
    sel = np.take_along_axis(lg.astype(np.float64), ref, axis=1)
    assert np.max(np.abs(g - softmax(sel, axis=1))) < 1e-6
    assert np.max(np.abs(g.astype(np.float64).sum(1) - 1.0)) < 1e-6


def pin_router_special(o):
    E = 12
    idx, g = o.route(np.full((2, E), 0.75, np.float32), 4)      # all equal
    assert np.array_equal(idx, np.tile(np.arange(4), (2, 1))) and np.all(g == f32(0.25))
    lg = np.random.default_rng(3).standard_normal((5, E)).astype(np.float32)
    idx, g = o.route(lg, 1)                                     # k = 1
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1)) and np.all(g == 1.0)
    idx, g = o.route(lg, E)                                     # k = E: full order
    assert np.array_equal(idx, np.argsort(-lg, axis=1, kind="stable"))
    z = np.zeros((1, E), np.float32)
    z[0, 0] = -0.0
    z[0, 1] = -1.0
    idx, _ = o.route(z, 3)                                      # -0 ties +0
    assert list(idx[0]) == [0, 2, 3]
    n = np.zeros((1, E), np.float32)
    n[0, 0] = np.nan
    n[0, 5] = -np.inf
    idx, _ = o.route(n, E)                                      # NaN ranks last
    assert idx[0, -1] == 0 and idx[0, -2] == 5


# ------------------------------------------------------------------ permutation
def pin_permute(o):
    """Invariants, plus equality with numpy's stable argsort of the expert ids."""
    rng = np.random.default_rng(5)
    for T, E, k in ((1, 384, 6), (33, 16, 2), (257, 40, 6), (2, 8, 8)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        idx, _ = o.route(lg, k)
        counts, offsets, sp, slot = o.permute(idx, E)
        flat = idx.ravel()
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
        assert np.all(np.diff(offsets) == counts)
        assert np.array_equal(np.sort(sp), np.arange(T * k))
        assert np.array_equal(slot[sp], np.arange(T * k))
        assert np.array_equal(sp, np.argsort(flat, kind="stable"))
        for e in range(E):
            seg = sp[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg // k) > 0)
        assert np.array_equal(np.bincount(sp // k, minlength=T), np.full(T, k))


# ------------------------------------------------------------------ one-hot probes
def pin_probe_w1(o, H=256, I=128, cases=None):
    """A single nonzero w1 nibble fixes G exactly: G[n0] = x[c0]*E2M1(code)*2^(sc-127).

    w3 is all 1.0, so U[n] = sum(x); x has two nonzeros in the byte holding c0, so a
    swapped nibble order, a wrong row/column orientation, a wrong scale index or a
    dropped column all change hpre = silu(G)*U."""
    cases = cases or [(0, 0, 7, 124), (0, 1, 15, 120), (I - 1, H - 1, 1, 130),
                      (I // 2 + 3, 37, 9, 126), (5, 32 * 3 + 17, 6, 121), (I - 2, 32, 3, 140)]
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for n0, c0, code, sc in cases:
        ex = const_expert(H, I, 0, 2, 0)
        set_nibble(ex["w1"], n0, c0, code)
        ex["s1"][n0, c0 // 32] = sc
        x = np.zeros((1, H), np.uint16)
        a, b = 1.5, -0.625
        x[0, c0] = bf16_bits(a)
        x[0, c0 ^ 1] = bf16_bits(b)
        out = o.forward(H, I, 1, 1, x, np.zeros((1, 1), np.float32), {0: ex}, want_h=True)
        val = (-1 if code & 8 else 1) * e2m1[code & 7] * 2.0 ** (sc - 127)
        G = a * val
        U = a + b
        want = G / (1.0 + math.exp(-G)) * U
        hp = out["hpre"][0]
        assert abs(hp[n0] - want) <= 1e-14 * abs(want), (n0, c0, hp[n0], want)
        others = np.delete(hp, n0)
        assert np.all(others == 0.0), (n0, c0)


def pin_probe_w2(o, H=256, I=128, cases=None):
    """A single nonzero w2 nibble at (m0, n0) makes y nonzero only at row m0."""
    cases = cases or [(0, 0, 7, 124), (H - 1, I - 1, 13, 125), (3, 33, 5, 127), (H // 2, 1, 2, 131)]
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for m0, n0, code, sc in cases:
        ex = const_expert(H, I, 2, 2, 0)
        set_nibble(ex["w2"], m0, n0, code)
        ex["s2"][m0, n0 // 32] = sc
        x = np.zeros((1, H), np.uint16)
        a = 1.25
        x[0, 0] = bf16_bits(a)
        out = o.forward(H, I, 1, 1, x, np.zeros((1, 1), np.float32), {0: ex}, want_h=True)
        h0 = brute.bf16_value(brute.to_bf16_bits(a / (1.0 + math.exp(-a)) * a))
        assert np.all(out["h"][0] == brute.to_bf16_bits(h0))
        val = (-1 if code & 8 else 1) * e2m1[code & 7] * 2.0 ** (sc - 127)
        y = out["y"][0]
        assert y[m0] == f32(h0 * val), (m0, n0, y[m0], h0 * val)
        assert np.all(np.delete(y, m0) == 0.0), (m0, n0)


# ------------------------------------------------------------------ closed forms
def pin_closed_form_swiglu(o):
    """Constant-weight experts whose output can be done by hand.

    H = 64, I = 32, x = 3/16 everywhere, two experts, k = 2, logits (0.3, -0.2):
      expert 0: W1 = 1, W3 = 1/2, W2 = 1/4  -> G = 12, U = 6,  silu(G)U = 71.99955 -> h = 72
      expert 1: W1 = 1/2, W3 = -1, W2 = 2   -> G = 6,  U = -12, silu(G)U = -71.8218 -> h = -72
      Y0 = 32*72/4 = 576, Y1 = -32*72*2 = -4608,  y = g0*Y0 + g1*Y1."""
    H, I = 64, 32
    e0 = const_expert(H, I, 2, 1, 2, s2=125)       # 1.0, 0.5, 1.0*2^-2
    e1 = const_expert(H, I, 1, 10, 4)              # 0.5, -1.0, 2.0
    x = np.full((1, H), bf16_bits(0.1875), np.uint16)
    lg = np.array([[0.3, -0.2]], np.float32)
    out = o.forward(H, I, 2, 2, x, lg, {0: e0, 1: e1}, want_h=True)
    l0, l1 = float(lg[0, 0]), float(lg[0, 1])
    g0 = f32(1.0 / (1.0 + math.exp(l1 - l0)))
    g1 = f32(math.exp(l1 - l0) / (1.0 + math.exp(l1 - l0)))
    assert list(out["idx"][0]) == [0, 1] and out["gates"][0, 0] == g0 and out["gates"][0, 1] == g1
    assert np.all(out["h"][0] == bf16_bits(72.0)) and np.all(out["h"][1] == bf16_bits(-72.0))
    want = f32(g0 * 576.0 + g1 * -4608.0)
    assert np.all(out["y"][0] == want), (out["y"][0][:4], want)
    # k = 1 keeps only expert 0, gate exactly 1
    out1 = o.forward(H, I, 2, 1, x, lg, {0: e0, 1: e1})
    assert np.all(out1["y"][0] == 576.0)


def pin_prenorm(o):
    """x = (3, -4, 3, -4, ...): mean(x^2) = 12.5, u = bf16(x / sqrt(12.5 + 1e-6))."""
    H = 64
    x = np.tile(np.array([3.0, -4.0], np.float32), (2, H // 2))
    x[1] *= -2.0
    u = o.prenorm(x)
    r0 = math.sqrt(12.5 + 1e-6)
    r1 = math.sqrt(50.0 + 1e-6)
    assert u[0, 0] == brute.to_bf16_bits(3.0 / r0) and u[0, 1] == brute.to_bf16_bits(-4.0 / r0)
    assert u[1, 0] == brute.to_bf16_bits(-6.0 / r1) and u[1, 1] == brute.to_bf16_bits(8.0 / r1)


# ------------------------------------------------------------------ independent implementations
def pin_brute(o):
    """Bit-equal with the scalar pure-Python version on a tiny random layer."""
    rng = np.random.default_rng(21)
    H, I, E, k, T = 64, 32, 5, 2, 3
    experts = {e: random_expert(rng, H, I) for e in range(E)}
    x = rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out = o.forward(H, I, E, k, x, lg, experts, want_h=True)
    ys, idx, g, hs = brute.forward(H, I, k, x, lg, experts)
    assert np.array_equal(out["idx"], np.array(idx))
    assert np.array_equal(out["gates"], np.array(g, np.float32))
    for p, h in hs.items():
        assert np.array_equal(out["h"][p], np.array(h, np.uint16)), p
    assert np.array_equal(out["y"], np.array(ys, np.float32))


def _dequant(w, s):
    """numpy dequantisation: table lookup + ldexp (for the matmul pin)."""
    g = read_golden("mx_formats.txt")["e2m1_positive"]
    table = np.array(g + [-v for v in g])
    lo = w & 0x0F
    hi = w >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(w.shape[0], -1)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    return table[codes] * sc


def pin_numpy_matmul(o):
    """Against numpy float64 dequantisation + matmul (library GEMM) at a mid shape."""
    rng = np.random.default_rng(33)
    H, I, E, k, T = 256, 96, 7, 3, 5
    experts = {e: random_expert(rng, H, I) for e in range(E)}
    x = rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out = o.forward(H, I, E, k, x, lg, experts, want_h=True)
    xd = bf16_to_f64(x)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = int(out["idx"][t, j])
            W1 = _dequant(experts[e]["w1"], experts[e]["s1"])
            W3 = _dequant(experts[e]["w3"], experts[e]["s3"])
            W2 = _dequant(experts[e]["w2"], experts[e]["s2"])
            G = W1 @ xd[t]
            U = W3 @ xd[t]
            hp = G / (1.0 + np.exp(-G)) * U
            p = t * k + j
            assert np.allclose(out["hpre"][p], hp, rtol=1e-12, atol=1e-12 * np.abs(hp).max())
            Y = W2 @ bf16_to_f64(out["h"][p])
            acc += float(out["gates"][t, j]) * Y
        assert np.allclose(out["y"][t], acc.astype(np.float32), rtol=1e-6, atol=1e-6 * np.abs(acc).max())


# ---------------------------------------------------------------- MXFP8 mode
def _e4m3_values():
    """All finite E4M3 values by code, from the bit fields (sign 7, exponent 6..3
    with bias 7, mantissa 2..0, exponent 0 subnormal), as exact fractions."""
    from fractions import Fraction
    vals = {}
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue  # NaN
        e, m = (c >> 3) & 15, c & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        vals[c] = -v if c & 0x80 else v
    return vals


def _mx8_brute(block):
    """Independent MXFP8 quantiser for one block of 32 (exact rationals, exhaustive
    search over the finite E4M3 codes).  Returns (codes, scale byte)."""
    from fractions import Fraction
    vals = _e4m3_values()
    fr = [Fraction(float(v)) for v in block]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        se = 0
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= amax:
            e += 1
        while Fraction(2) ** e > amax:
            e -= 1
        se = min(254, max(0, e - 8 + 127))
    scale = Fraction(2) ** (se - 127)
    pos = sorted((v, c) for c, v in vals.items() if c < 0x80)  # non-negative values
    codes = []
    for v, f in zip(block, fr):
        r = min(abs(f) / scale, Fraction(448))   # saturate
        best = min(pos, key=lambda vc: (abs(vc[0] - r), vc[1] & 1))  # nearest, ties to even code
        codes.append(best[1] | (0x80 if math.copysign(1.0, float(v)) < 0 else 0))
    return codes, se


def pin_e4m3_table(o):
    """E4M3 decode of all 256 codes against torch's float8_e4m3fn."""
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got, want = o.e4m3(c), float(ref[c])
        assert (math.isnan(got) and math.isnan(want)) or got == want, (hex(c), got, want)


def pin_mx8_quant(o):
    """MXFP8 quantiser against the exhaustive-search version on random blocks of
    mixed magnitudes (signs, subnormal results, exact ties, zeros)."""
    rng = np.random.default_rng(41)
    blocks = []
    for b in range(24):
        v = rng.standard_normal(32) * np.ldexp(1.0, int(rng.integers(-20, 20)))
        v[rng.integers(0, 32, 4)] *= np.ldexp(1.0, -12)   # values far below the block max
        v[rng.integers(0, 32, 2)] = 0.0
        blocks.append(v)
    # ties at several binades: 17 (16 vs 18), 1.0625 (1 vs 1.125), 9*2^-10 (subnormal 4 vs 5)
    t = np.zeros(32)
    t[:6] = [256.0, 17.0, -1.0625, 9 * 2.0 ** -10 * 256, 19.0, -0.0]
    blocks.append(t)
    for v in blocks:
        codes, scales = o.mx8_quant(v)
        want, se = _mx8_brute(v)
        assert int(scales[0]) == se, (int(scales[0]), se)
        assert list(codes) == want, (list(codes), want)


def pin_mx8_special(o):
    """Closed forms: a block whose max is 2^k has scale byte k - 8 + 127 and that
    element is 256 = code 0x78; a max of 511 * 2^k saturates to 448 (0x7E); a
    zero block has byte 0 and zero codes; -0 keeps its sign."""
    for k in (-30, -3, 0, 5, 40):
        v = np.zeros(32)
        v[3] = 2.0 ** k
        v[7] = -(2.0 ** k)
        codes, sc = o.mx8_quant(v)
        assert int(sc[0]) == k - 8 + 127 and codes[3] == 0x78 and codes[7] == 0xF8
        v[5] = 511 * 2.0 ** (k - 8)       # max of the block now: 511 * 2^(k-8) < 2^(k+1)
        codes, sc = o.mx8_quant(v)
        assert int(sc[0]) == k - 8 + 127 and codes[5] == 0x7E
    codes, sc = o.mx8_quant(np.zeros(64))
    assert not codes.any() and not sc.any()
    v = np.zeros(32)
    v[0], v[1] = 1.0, -0.0
    codes, _ = o.mx8_quant(v)
    assert codes[1] == 0x80


def pin_mx8_forward(o):
    """The MXFP8 mode against numpy: x and the bf16 h go through the (pinned)
    quantiser, everything else is float64 dequantisation + matmul."""
    rng = np.random.default_rng(45)
    H, I, E, k, T = 128, 64, 5, 2, 3
    experts = {e: random_expert(rng, H, I) for e in range(E)}
    x = rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out = o.forward(H, I, E, k, x, lg, experts, want_h=True, mx8=True)

    def rt(v):
        c, sc = o.mx8_quant(v)
        d = np.array([o.e4m3(int(q)) for q in c.ravel()]).reshape(c.shape)
        return d * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)

    for t in range(T):
        xq = rt(bf16_to_f64(x[t]))
        acc = np.zeros(H)
        for j in range(k):
            e = int(out["idx"][t, j])
            W1 = _dequant(experts[e]["w1"], experts[e]["s1"])
            W3 = _dequant(experts[e]["w3"], experts[e]["s3"])
            W2 = _dequant(experts[e]["w2"], experts[e]["s2"])
            G, U = W1 @ xq, W3 @ xq
            hp = G / (1.0 + np.exp(-G)) * U
            p = t * k + j
            assert np.allclose(out["hpre"][p], hp, rtol=1e-12, atol=1e-12 * np.abs(hp).max())
            acc += float(out["gates"][t, j]) * (W2 @ rt(bf16_to_f64(out["h"][p])))
        assert np.allclose(out["y"][t], acc.astype(np.float32), rtol=1e-6, atol=1e-6 * np.abs(acc).max())


def pin_router_numpy(o):
    """Router logits against numpy's float64 matmul of the same bf16 values, at
    shapes that are not multiples of anything (T=5, H=224, E=19)."""
    rng = np.random.default_rng(61)
    T, H, E = 5, 224, 19
    x = rand_bf16(rng, (T, H))
    w = rand_bf16(rng, (E, H), scale=1.0 / np.sqrt(H))
    lg, b = o.router_logits(x, w)
    ref = bf16_to_f64(x) @ bf16_to_f64(w).T
    assert np.allclose(lg, ref, rtol=0, atol=1e-12 * np.abs(ref).max()), np.abs(lg - ref).max()
    assert np.all(b > 0)


def pin_router_onehot(o):
    """x a unit vector at column c gives logits[e] = wr[e][c] exactly, for the
    first, a middle and the last column: pins operand orientation and that
    every input is summed."""
    rng = np.random.default_rng(62)
    H, E = 96, 7
    w = rand_bf16(rng, (E, H))
    one = o.to_bf16(1.0)
    for c in (0, 37, H - 1):
        x = np.zeros((1, H), np.uint16)
        x[0, c] = one
        lg, _ = o.router_logits(x, w)
        assert np.array_equal(lg[0], bf16_to_f64(w[:, c])), c


def pin_router_bound(o):
    """Closed form: x and wr all ones give logits = H exactly and the bound
    gamma_H * H, gamma_H = H 2^-24 / (1 - H 2^-24)."""
    H, E = 5120, 3
    one = o.to_bf16(1.0)
    x = np.full((2, H), one, np.uint16)
    w = np.full((E, H), one, np.uint16)
    lg, b = o.router_logits(x, w)
    u = 2.0 ** -24
    assert np.all(lg == H) and np.allclose(b, H * u / (1 - H * u) * H, rtol=1e-15)


def pin_saliency_single(o):
    """k = 1 and one token: the gate is 1, so the saliency of the chosen expert
    is the L2 norm of the layer output y, and every other expert's is 0."""
    rng = np.random.default_rng(71)
    H, I, E = 128, 64, 4
    experts = {e: random_expert(rng, H, I) for e in range(E)}
    x = rand_bf16(rng, (1, H))
    lg = rng.standard_normal((1, E)).astype(np.float32)
    out = o.forward(H, I, E, 1, x, lg, experts)
    sal = o.saliency(H, I, E, 1, x, lg, experts)
    e = int(out["idx"][0, 0])
    assert out["gates"][0, 0] == 1.0
    assert abs(sal[e] - np.linalg.norm(out["y"][0].astype(np.float64))) <= 1e-6 * sal[e]
    assert np.all(np.delete(sal, e) == 0.0)


def pin_saliency_numpy(o):
    """Saliency against numpy float64: each pair's Y from dequantised matrices
    and the oracle's (pinned) bf16 h, its norm, times the gate, summed by expert."""
    rng = np.random.default_rng(72)
    H, I, E, k, T = 96, 64, 5, 2, 7
    experts = {e: random_expert(rng, H, I) for e in range(E)}
    x = rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out = o.forward(H, I, E, k, x, lg, experts, want_h=True)
    sal = o.saliency(H, I, E, k, x, lg, experts)
    ref = np.zeros(E)
    for t in range(T):
        for j in range(k):
            e = int(out["idx"][t, j])
            hv = bf16_to_f64(out["h"][t * k + j])
            Y = _dequant(experts[e]["w2"], experts[e]["s2"]) @ hv
            ref[e] += float(out["gates"][t, j]) * np.linalg.norm(Y)
    assert np.allclose(sal, ref, rtol=1e-12, atol=0), (sal, ref)
    assert np.all(sal[np.setdiff1d(np.arange(E), out["idx"])] == 0.0)


def random_shared(rng, H, I, lo=113, hi=115):
    """Shared-expert tensors: E4M3 codes uniform over the 254 non-NaN codes,
    UE8M0 block scales uniform in [lo, hi]."""
    def codes(shape):
        c = rng.integers(0, 254, shape)
        return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)
    return {"w1": codes((I, H)), "s1": rng.integers(lo, hi + 1, (I // 32, H // 32)).astype(np.uint8),
            "w3": codes((I, H)), "s3": rng.integers(lo, hi + 1, (I // 32, H // 32)).astype(np.uint8),
            "w2": codes((H, I)), "s2": rng.integers(lo, hi + 1, (H // 32, I // 32)).astype(np.uint8)}


def pin_shared_numpy(o):
    """The shared expert against numpy float64: E4M3 values from the (pinned)
    decode table, 32 x 32 block scales expanded with np.kron, matmuls, SwiGLU
    and the oracle's (pinned) bf16 rounding of h.  Non-square block grids
    (H = 96, I = 64) so that a transposed scale index shows."""
    rng = np.random.default_rng(81)
    H, I, T = 96, 64, 3
    sw = random_shared(rng, H, I, 110, 118)
    x = rand_bf16(rng, (T, H))
    out = o.shared(x, sw, want_h=True)
    tab = np.array([o.e4m3(c) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)])
    dq = lambda w, sc: tab[w] * np.kron(np.ldexp(1.0, sc.astype(np.int64) - 127), np.ones((32, 32)))
    W1, W3, W2 = dq(sw["w1"], sw["s1"]), dq(sw["w3"], sw["s3"]), dq(sw["w2"], sw["s2"])
    xf = bf16_to_f64(x)
    G, U = xf @ W1.T, xf @ W3.T
    a = G / (1.0 + np.exp(-G)) * U
    assert np.allclose(out["hpre"], a, rtol=1e-12, atol=1e-300)
    h = np.array([[o.to_bf16(v) for v in row] for row in a], np.uint16)
    assert np.array_equal(out["h"], h)
    y = bf16_to_f64(h) @ W2.T
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


ALL_PINS = [pin_e2m1_table, pin_ue8m0, pin_bf16_rounding, pin_router_vs_sort, pin_router_special,
            pin_permute, pin_probe_w1, pin_probe_w2, pin_closed_form_swiglu, pin_prenorm,
            pin_brute, pin_numpy_matmul, pin_e4m3_table, pin_mx8_quant, pin_mx8_special,
            pin_mx8_forward, pin_router_numpy, pin_router_onehot, pin_router_bound,
            pin_saliency_single, pin_saliency_numpy, pin_shared_numpy]


# ---------------------------------------------------------------- h bound and the stack layer
def _f32_bf16_bits(v32):
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.asarray(v32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _h32(G32, U32):
    """An fp32 evaluation's h: silu(G') U' from the fp32 sums, rounded once to
    fp32 (then to bf16).  One rounding after exact arithmetic is within the
    bound's allowance for the epilogue."""
    G, U = np.asarray(G32, np.float64), np.asarray(U32, np.float64)
    return _f32_bf16_bits((G / (1.0 + np.exp(-G)) * U).astype(np.float32))


def _in_interval(o, hbits, hpre, hbound):
    """Indices where the bf16 value hbits is outside [bf16(hpre - b), bf16(hpre + b)]."""
    lo = bf16_to_f64(np.array([o.to_bf16(v) for v in (hpre - hbound).ravel()], np.uint16))
    hi = bf16_to_f64(np.array([o.to_bf16(v) for v in (hpre + hbound).ravel()], np.uint16))
    got = bf16_to_f64(hbits.ravel())
    return np.nonzero((got < lo) | (got > hi))[0]


def _f32_sum(terms, order):
    """fp32 evaluation of sum(terms) (exact float64 products, last axis) in a
    given order: 'forward' / 'reverse' one by one, 'pairwise' (numpy's float32
    sum), 'sorted' by decreasing magnitude, 'lanes' (lane l of 64 chains its
    32-input groups l, l + 64, ... one product at a time, then a 6-level tree of
    the 64 lane sums, as a wave's DPP reduction), 'blocks' (the inputs in
    ascending groups of 32 whose exact sum is added to an fp32 accumulator with
    one rounding, as an MFMA instruction at best)."""
    t = np.asarray(terms, np.float64)
    t32 = t.astype(np.float32)
    assert np.array_equal(t32.astype(np.float64), t)          # products exact in fp32
    if order == "forward":
        return np.add.accumulate(t32, axis=-1)[..., -1]
    if order == "reverse":
        return np.add.accumulate(t32[..., ::-1], axis=-1)[..., -1]
    if order == "pairwise":
        return t32.sum(axis=-1, dtype=np.float32)
    if order == "sorted":
        idx = np.argsort(-np.abs(t), axis=-1, kind="stable")
        return np.add.accumulate(np.take_along_axis(t32, idx, -1), axis=-1)[..., -1]
    K = t.shape[-1]
    if order == "lanes":
        G = K // 32
        lanes = np.zeros(t.shape[:-1] + (64,), np.float32)
        for g in range(G):
            for j in range(32):
                lanes[..., g % 64] = lanes[..., g % 64] + t32[..., 32 * g + j]
        while lanes.shape[-1] > 1:
            lanes = lanes[..., 0::2] + lanes[..., 1::2]
        return lanes[..., 0]
    if order == "blocks":
        acc = np.zeros(t.shape[:-1], np.float32)
        for g in range(0, K, 32):
            acc = (acc.astype(np.float64) + t[..., g:g + 32].sum(-1)).astype(np.float32)
        return acc
    raise ValueError(order)


_U24 = 2.0 ** -24


def _acc_worst(D):
    return (D * _U24 / (1 - D * _U24), 0.0, 0)


def _acc_blocks(K):
    """The 'blocks' order: N = K/32 additions, each within u of its terms'
    absolute sum; four of them per 128-input block."""
    e = _U24 / (1 - (K // 32) * _U24)
    return (5 * e, 4 * e, 128)


def pin_hbound_sound(o):
    """Soundness of the oracle's h bound: fp32 evaluations of G and U in several
    summation orders, then h rounded to bf16, must lie in [bf16(hpre - b),
    bf16(hpre + b)] with b the oracle's bound for that order's accumulation
    model (gamma_K for any order; the lane-tree depth for 'lanes'; the blocked
    model for 'blocks').  Random rows at H = 2048, half of them with U made
    small by cancellation, so that both terms of the bound matter."""
    rng = np.random.default_rng(91)
    H, I, T = 2048, 48, 3
    ex = random_expert(rng, H, I)
    x = rand_bf16(rng, (T, H))
    W1, W3 = _dequant(ex["w1"], ex["s1"]), _dequant(ex["w3"], ex["s3"])
    xd = bf16_to_f64(x)
    P1 = xd[:, None, :] * W1[None]          # [T, I, H] exact products
    P3 = xd[:, None, :] * W3[None]
    models = {"forward": None, "reverse": None, "pairwise": None, "sorted": None,
              "lanes": _acc_worst(32 * (H // 2048) + 6), "blocks": _acc_blocks(H)}
    for order, acc in models.items():
        out = o.forward(H, I, 1, 1, x, np.zeros((T, 1), np.float32), {0: ex}, want_h=True, acc=acc)
        h32 = _h32(_f32_sum(P1, order), _f32_sum(P3, order))
        bad = _in_interval(o, h32, out["hpre"], out["hbound"])
        assert bad.size == 0, (order, bad[:4])


def _adversarial_rows(K, T):
    """Rows on which fp32 summation errs by almost the worst case.  Token t has
    x_0 = 1 + t/128 and x_c = a = 2^-24 (1 + 2^-7) for c > 0: each added a
    exceeds half an ulp of a running sum in [1, 2), so every addition rounds up
    by almost u.  x2 is x with x_{K-32} = 1.
      row 0 (x):  W1 all 1, W3 = 1 at input 0 only  -> G adversarial, U = x_0
      row 1 (x):  W1 = 1 at input 0 only, W3 all 1  -> U adversarial, G = x_0
      row 2 (x2): W1 = 1 at the first input of every 32-input group, -1 at the
                  group starting at K - 32; W3 as row 0.  Summed in 32-input
                  groups, each group after the first rounds up by almost u and
                  the last one cancels the 1: the accumulated error is of the
                  order of G itself
      row 3 (x2): W1 as row 1; W3 all 1 except -1 at K - 32: U summed one by one
                  errs by almost (K - 33) u and then cancels to t/128 + (K-2) a,
                  so the error is large against U and against the G term of the
                  bound.
    Returns the expert, x and x2."""
    ex = const_expert(K, 32, 0, 0, 0)
    ex["w1"][0, :] = 0x22
    set_nibble(ex["w3"], 0, 0, 2)
    set_nibble(ex["w1"], 1, 0, 2)
    ex["w3"][1, :] = 0x22
    for c in range(0, K, 32):
        set_nibble(ex["w1"], 2, c, 10 if c == K - 32 else 2)
    set_nibble(ex["w3"], 2, 0, 2)
    set_nibble(ex["w1"], 3, 0, 2)
    ex["w3"][3, :] = 0x22
    set_nibble(ex["w3"], 3, K - 32, 10)
    x = np.full((T, K), bf16_bits(2.0 ** -24 * (1 + 2.0 ** -7)), np.uint16)
    x[:, 0] = [bf16_bits(1.0 + t / 128.0) for t in range(T)]
    x2 = x.copy()
    x2[:, K - 32] = bf16_bits(1.0)
    return ex, x, x2


def pin_hbound_adversarial(o):
    """The bound is tight where fp32 summation is at its worst.  Summed one by
    one, rows 0 and 1 stray by more than 99% of gamma_K * sum|p|, and row 3 by
    nearly as much and then cancels; summed in 32-input groups, row 2 strays by
    about (K/32) u, which only the prefix term of the blocked model covers.  h
    crosses bf16 rounding boundaries for some tokens in each case, and every h
    must still be inside the oracle's interval: a bound that dropped the G or
    the U term, the prefix mass, or used a shorter gamma fails here."""
    K, T = 5120, 116
    ex, x, x2 = _adversarial_rows(K, T)
    W1, W3 = _dequant(ex["w1"], ex["s1"]), _dequant(ex["w3"], ex["s3"])
    lg = np.zeros((T, 1), np.float32)
    worst = 0.99 * (K - 1) * _U24 * (1 - 2.0 ** -7)
    for order, acc, xb, rows in (("forward", None, x, (0, 1)), ("forward", None, x2, (3,)),
                                 ("blocks", _acc_blocks(K), x2, (2,))):
        xd = bf16_to_f64(xb)
        P1, P3 = xd[:, None, :] * W1[None], xd[:, None, :] * W3[None]
        out = o.forward(K, 32, 1, 1, xb, lg, {0: ex}, want_h=True, acc=acc)
        G32, U32 = _f32_sum(P1, order), _f32_sum(P3, order)
        h32 = _h32(G32, U32)
        hpre, hb = out["hpre"].reshape(T, 32), out["hbound"].reshape(T, 32)
        for r in rows:
            if r in (0, 1):   # the evaluation is nearly the worst case
                S, S32 = (P1[:, r].sum(-1), G32[:, r]) if r == 0 else (P3[:, r].sum(-1), U32[:, r])
                assert np.all(np.abs(S32 - S) > worst), (r, np.abs(S32 - S).min())
            crossed = _f32_bf16_bits(hpre[:, r].astype(np.float32)) != h32[:, r]
            assert crossed.any(), (order, r)    # the rows have teeth
            bad = _in_interval(o, h32[:, r], hpre[:, r], hb[:, r])
            assert bad.size == 0, (order, r, bad[:4])


def pin_stack_layer(o):
    """One layer of the residual stack in closed form.  x rows are constant
    (3/16 and 3/4), so the pre-norm gives u = bf16(x / sqrt(x^2 + 1e-6)) = 1
    everywhere; with the constant experts of pin_closed_form_swiglu (H = 64,
    I = 32): expert 0 has G = 64, U = 32, h = 2048, Y0 = 32 * 2048 / 4 = 16384;
    expert 1 has G = 32, U = -64, h = bf16(-2048 / (1 + e^-32)) = -2048,
    Y1 = 32 * -2048 * 2 = -131072.  The layer's output is
    x + (g0 * Y0 + g1 * Y1), each sum stored as fp32."""
    H, I = 64, 32
    e0 = const_expert(H, I, 2, 1, 2, s2=125)
    e1 = const_expert(H, I, 1, 10, 4)
    x = np.array([[0.1875] * H, [0.75] * H], np.float32)
    assert np.all(o.prenorm(x) == bf16_bits(1.0))
    lg = np.array([[0.3, -0.2], [-1.0, 0.5]], np.float32)
    out = o.stack_layer(I, 2, 2, x, lg, {0: e0, 1: e1})
    idx, g = o.route(lg, 2)
    for t in range(2):
        Y = {0: 16384.0, 1: -131072.0}
        y = f32(sum(float(g[t, j]) * Y[int(idx[t, j])] for j in range(2)))
        want = f32(float(x[t, 0]) + y)
        assert np.all(out[t] == np.float32(want)), (t, out[t][:2], want)


ALL_PINS += [pin_hbound_sound, pin_hbound_adversarial, pin_stack_layer]
