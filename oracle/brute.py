"""Scalar pure-Python version of the oracle, for tiny shapes only.

TEST INFRASTRUCTURE ONLY.  It is written separately from oracle.c (Python
scalars, Python's sorted(), fractions for the bf16 rounding) so that the two can
be compared; an indexing mistake in one is unlikely to be repeated in the other.
The definition is the same: DeepSeek-V4.1-Flash expert layout (10100.com page,
section on the expert-capacity bottleneck) and the readings at the top of
oracle.c.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def e2m1(code: int) -> float:
    # sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 = subnormal
    sign = -1.0 if code & 8 else 1.0
    exp_field = (code >> 1) & 3
    man = code & 1
    if exp_field == 0:
        return sign * man * 0.5
    return sign * (2.0 ** (exp_field - 1)) * (1 + man / 2)


def ue8m0(e: int) -> float:
    return math.nan if e == 255 else 2.0 ** (e - 127)


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def to_bf16_bits(v: float) -> int:
    """Round a Python float to bf16, nearest with ties to even, exactly (Fractions)."""
    if math.isnan(v):
        return 0x7FC0
    if v == 0.0 or math.isinf(v):
        return struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    # candidates: every bf16 value is a float32 whose low 16 bits are zero
    f32 = struct.unpack("<I", struct.pack("<f", v))[0] if abs(v) < 3.4e38 else None
    if f32 is None:
        return 0xFF80 if v < 0 else 0x7F80
    lo = f32 & 0xFFFF0000
    cands = [lo, lo + 0x10000, lo - 0x10000]
    best = None
    x = Fraction(v)
    for c in cands:
        c &= 0xFFFFFFFF
        cv = struct.unpack("<f", struct.pack("<I", c))[0]
        if math.isnan(cv):
            continue
        if math.isinf(cv):
            # rounding beyond the largest finite bf16 goes to inf
            d = abs(x - Fraction(2) ** 128)
        else:
            d = abs(x - Fraction(cv))
        key = (d, (c >> 16) & 1)  # tie -> even mantissa
        if best is None or key < best[0]:
            best = (key, c >> 16)
    return best[1]


def weight(w, s, r: int, c: int) -> float:
    """Element (row r, input c) of a nibble tensor w[rows][cols/2] with scales s[rows][cols/32]."""
    byte = int(w[r][c // 2])
    code = (byte >> 4) if (c % 2) else (byte & 15)
    return e2m1(code) * ue8m0(int(s[r][c // 32]))


def route(logits, k):
    out_idx, out_g = [], []
    for row in logits:
        vals = [float(v) for v in row]

        def key(e):
            v = vals[e]
            if math.isnan(v):
                return (1, 0.0, e)
            return (0, -(v + 0.0), e)  # +0.0 folds -0 onto +0
        order = sorted(range(len(vals)), key=key)[:k]
        l0 = vals[order[0]]
        ex = [math.exp(vals[e] - l0) for e in order]
        den = sum(ex)
        out_idx.append(order)
        out_g.append([struct.unpack("<f", struct.pack("<f", v / den))[0] for v in ex])
    return out_idx, out_g


def forward(H, I, k, x_bits, logits, experts):
    """y[t][m] for every token, as Python floats rounded to float32 at the end."""
    idx, g = route(logits, k)
    T = len(x_bits)
    ys, hs = [], {}
    for t in range(T):
        x = [bf16_value(int(b)) for b in x_bits[t]]
        acc = [0.0] * H
        for j in range(k):
            W = experts[idx[t][j]]
            h = []
            for n in range(I):
                G = sum(x[c] * weight(W["w1"], W["s1"], n, c) for c in range(H))
                U = sum(x[c] * weight(W["w3"], W["s3"], n, c) for c in range(H))
                a = G / (1.0 + math.exp(-G)) * U
                h.append(to_bf16_bits(a))
            hs[t * k + j] = h
            hv = [bf16_value(b) for b in h]
            for m in range(H):
                Y = sum(hv[n] * weight(W["w2"], W["s2"], m, n) for n in range(I))
                acc[m] += g[t][j] * Y
        ys.append([struct.unpack("<f", struct.pack("<f", v))[0] for v in acc])
    return ys, idx, g, hs
