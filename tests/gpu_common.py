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


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
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
    assert mx <= MAX_ABS_RMS * rms, (what, mx, rms)
    return rel


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_h(h_gpu: np.ndarray, h_ref: np.ndarray, hpre: np.ndarray, hbound: np.ndarray,
            what: str = ""):
    """h is rounded to bf16 at the same point on both sides.  The GPU evaluates
    silu(G)*U in fp32 from fp32 sums, so its value before rounding lies within
    the oracle's bound b of the exact value hpre; rounding to nearest is
    monotone, so the GPU's h must lie between bf16(hpre - b) and bf16(hpre + b).
    Where that interval holds one bf16 value the GPU must match the oracle
    exactly.  This is an exact rule, not a tolerance on a count."""
    import oracle
    h_gpu = np.asarray(h_gpu, np.uint16)
    h_ref = np.asarray(h_ref, np.uint16)
    bad = np.nonzero(h_gpu != h_ref)
    n = len(bad[0])
    say(f"  {what}: h mismatches {n} of {h_ref.size}")
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
