"""Helpers of the GPU parity tests: moving inputs to the device and comparing
the HIP path with the oracle to the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

# Output tolerance: relative L2 error <= 2e-3 and max |error| <= 2e-2 * RMS(oracle).
REL_L2 = 2e-3
MAX_ABS_RMS = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bits(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_weights(host: dict):
    import torch
    import mxfp4_routed_expert_router_amd as moe
    return moe.ExpertWeights.from_dict({n: torch.from_numpy(np.ascontiguousarray(a)).cuda()
                                        for n, a in host.items()})


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "", max_abs_rms: float = MAX_ABS_RMS):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), what
    d = y_gpu - y_ref
    nref = np.linalg.norm(y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2))
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mx = np.max(np.abs(d)) if d.size else 0.0
    say(f"  {what}: rel_l2={rel:.3e} max_abs/rms={mx / rms if rms else mx:.3e}")
    assert rel <= REL_L2, (what, rel)
    assert mx <= max_abs_rms * rms, (what, mx, rms)
    return rel


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_order(bits):
    """bf16 bit patterns -> integers in value order (adjacent values differ by 1)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _bf16_rne_stats(v):
    """Round doubles to bf16 bit patterns (nearest, ties to even), for the
    interval-width statistics only; the pass/fail decision uses the oracle's
    own rounding."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def check_h(h_gpu: np.ndarray, h_ref: np.ndarray, hpre: np.ndarray, hbound: np.ndarray,
            what: str = "", rel_max: float = None):
    """h is rounded to bf16 at the same point on both sides.  The kernel's value
    before rounding lies within the oracle's bound b of the exact value hpre
    (b from the accumulation model of the kernel family that ran: tests/accum.py),
    and rounding to nearest is monotone, so the GPU's h must lie between
    bf16(hpre - b) and bf16(hpre + b).  Where that interval holds one bf16
    value the GPU must match the oracle exactly, where it holds two, the GPU may
    take the adjacent value.  An exact rule, not a tolerance on a count.
    Prints the mismatch count, the largest distance in bf16 steps and the
    interval widths.  rel_max, where given, also bounds the relative L2
    distance of the GPU's h from the oracle's: a statistical guard for paths
    whose per-element intervals are wide (the MXFP8 mode's)."""
    import oracle
    h_gpu = np.asarray(h_gpu, np.uint16)
    h_ref = np.asarray(h_ref, np.uint16)
    bad = np.nonzero(h_gpu != h_ref)
    n = len(bad[0])
    dist = np.abs(_bf16_order(h_gpu) - _bf16_order(h_ref))
    width = _bf16_order(_bf16_rne_stats(hpre + hbound)) - _bf16_order(_bf16_rne_stats(hpre - hbound)) + 1
    hg, hr = bf16_value(h_gpu), bf16_value(h_ref)
    rel = np.linalg.norm(hg - hr) / max(np.linalg.norm(hr), 1e-300)
    say(f"  {what}: h mismatches {n} of {h_ref.size} (largest {int(dist.max()) if dist.size else 0} "
        f"bf16 steps, rel_l2 {rel:.2e}); interval width median {np.median(width):.0f}, p90 "
        f"{np.percentile(width, 90):.0f}, p99 {np.percentile(width, 99):.0f} values")
    if rel_max is not None:
        assert rel <= rel_max, (what, rel)
    if n == 0:
        return
    o = oracle.get()
    pre, b = hpre[bad], hbound[bad]
    lo = bf16_value(np.array([o.to_bf16(v) for v in pre - b], np.uint16))
    hi = bf16_value(np.array([o.to_bf16(v) for v in pre + b], np.uint16))
    got = bf16_value(h_gpu[bad])
    ok = (got >= lo) & (got <= hi)
    assert np.all(ok), (what, int(np.count_nonzero(~ok)), got[~ok][:4], pre[~ok][:4], b[~ok][:4])


def check_route(route, idx_ref, g_ref, perm_ref, what: str = ""):
    """Routing and permutation bit-exact; gates within 1e-6."""
    counts, offsets, sp, slot = perm_ref
    assert np.array_equal(route.topk_idx.cpu().numpy(), idx_ref), what
    assert np.array_equal(route.counts.cpu().numpy(), counts), what
    assert np.array_equal(route.offsets.cpu().numpy(), offsets), what
    assert np.array_equal(route.sorted_pairs.cpu().numpy(), sp), what
    assert np.array_equal(route.pair_slot.cpu().numpy(), slot), what
    g = route.gates.cpu().numpy()
    assert np.max(np.abs(g.astype(np.float64) - g_ref)) <= 1e-6, (what, np.max(np.abs(g - g_ref)))


def mx8_w2_on_h(orc, experts, idx, gates, h_bits, H, I):
    """The MXFP8 mode's w2 stage applied to the GPU's own h: y[t] = sum_j
    gate[t][j] * W2_e . MXFP8(h[t*k+j]), h in pair order (bf16 bits), quantised
    by the oracle's quantiser; the E4M3 and FP4 values are exact in float64 and
    the products are summed in float64 (experts in parallel threads, added in
    ascending expert order).  Where the GPU's h sits next to an FP8 code
    boundary its code may differ from the one the oracle's h takes, so the
    end-to-end y carries those decisions; against this reference only the w2
    stage's own accumulation remains."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from pins import bf16_to_f64, read_golden
    T, k = idx.shape
    codes, sc = orc.mx8_quant(bf16_to_f64(np.asarray(h_bits, np.uint16)))
    e4 = np.array([orc.e4m3(c) for c in range(256)])
    hq = e4[codes] * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)
    g = read_golden("mx_formats.txt")["e2m1_positive"]
    t16 = np.array(g + [-v for v in g])
    lut = np.stack([t16[np.arange(256) & 15], t16[np.arange(256) >> 4]], axis=-1)  # byte -> 2 values
    flat = idx.ravel()
    gflat = gates.ravel().astype(np.float64)

    def part(e):
        p = np.nonzero(flat == e)[0]
        w2, s2 = experts[int(e)]["w2"], experts[int(e)]["s2"]
        W2 = lut[w2].reshape(H, I) * np.repeat(np.ldexp(1.0, s2.astype(np.int64) - 127), 32, axis=1)
        return p, gflat[p][:, None] * (hq[p] @ W2.T)

    y = np.zeros((T, H))
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        for p, c in ex.map(part, np.unique(flat)):
            y[p // k] += c
    return y
