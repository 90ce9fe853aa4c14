"""GPU parity of the MXFP8 prefill mode (activations in OCP MX FP8, FP4 x FP8
scaled MFMA) against the oracle's MXFP8 forward.

The quantiser is compared bit for bit.  x is quantised identically on both
sides, so G and U differ only by accumulation: the scaled FP4 x FP8 matrix
instruction sums its 128 products with less than fp32 precision (measured on
MI355X: at most 2^-13.5 of the block's sum of absolute products), so the h
check takes the oracle's first-order bound with gamma = 2^-12 in place of the
fp32 summation bound.  y is held to the bf16 path's tolerances against the w2
stage applied to the GPU's own h (the FP8 codes of h are a discrete decision,
taken from the same input on both sides), and to its rel-L2 bound end to end."""
import numpy as np
import pytest

import pins
import synth
from synth.configs import PREFILL
from gpu_common import check_h, check_route, check_y, dev_bits, dev_weights, host_bits, say

pytestmark = pytest.mark.gpu

GAMMA_MX = 2.0 ** -12


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


def _bf16_rows(rng, rows, K):
    """bf16 rows with blocks of very different magnitudes, zero blocks, subnormal
    values and exact E4M3 ties."""
    v = rng.standard_normal((rows, K)) * np.ldexp(1.0, rng.integers(-30, 30, (rows, K // 32)).repeat(32, 1))
    v[rng.random((rows, K)) < 0.05] *= 2.0 ** -20
    v[:, :32] = 0.0                                  # a zero block in every row
    if K >= 64:
        v[0, 32:40] = [17.0, -1.0625, 19.0, 256.0, 9 * 2.0 ** -2, -0.0, 3.0, 2.0 ** -133]
    return _to_bits(v)


def _to_bits(v):
    import oracle
    o = oracle.get()
    return np.array([o.to_bf16(float(a)) for a in v.ravel()], np.uint16).reshape(v.shape)


@pytest.mark.parametrize("rows,K", [(3, 64), (17, 256), (64, 5120)])
def test_quant_mxfp8_bitexact(moe, orc, rows, K):
    import torch
    say(f"MXFP8 quantiser rows={rows} K={K}")
    rng = np.random.default_rng(rows * 31 + K)
    x = _bf16_rows(rng, rows, K)
    codes, scales = moe.moe_fp4_quant_mxfp8(dev_bits(x))
    torch.cuda.synchronize()
    ref_c, ref_s = orc.mx8_quant(pins.bf16_to_f64(x))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    c = codes.cpu().numpy()
    bad = np.argwhere(c != ref_c)
    assert bad.size == 0, [(tuple(b), int(c[tuple(b)]), int(ref_c[tuple(b)])) for b in bad[:8]]


def _y_from_h(orc, experts, idx, gates, h_bits, tokens):
    """y of the listed tokens from a given bf16 h (pair order): each pair's h is
    quantised to MXFP8 by the oracle's quantiser, then W2 (float64) and the
    gate-weighted sum.  Used to compare y on the GPU's own h: where the GPU's h
    lies one bf16 ulp from the oracle's (allowed by the h check), the block's
    FP8 codes may differ, and that discrete decision must be taken from the same
    input on both sides."""
    k = idx.shape[1]
    tab = np.array([orc.e4m3(c) for c in range(256)])
    out = []
    for t in tokens:
        acc = np.zeros(experts[int(idx[t, 0])]["w2"].shape[0])
        for j in range(k):
            e = int(idx[t, j])
            hv = pins.bf16_to_f64(h_bits[t * k + j])
            c, sc = orc.mx8_quant(hv)
            hq = tab[c] * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32)
            acc += float(gates[t, j]) * (pins._dequant(experts[e]["w2"], experts[e]["s2"]) @ hq)
        out.append(acc)
    return np.array(out)


def _check_y_mx(y_gpu, y_ref, y_on_gpu_h, what):
    """Full tolerance against y from the GPU's own h; rel-L2 end to end."""
    check_y(y_gpu, y_on_gpu_h, what + " (on the GPU's h)")
    d = np.asarray(y_gpu, np.float64) - np.asarray(y_ref, np.float64)
    rel = np.linalg.norm(d) / np.linalg.norm(np.asarray(y_ref, np.float64))
    say(f"  {what}: end-to-end rel_l2={rel:.3e}")
    assert rel <= 2e-3, (what, rel)


def _forward_mx(moe, orc, T, H, I, E, k, seed):
    import torch
    rng = np.random.default_rng(seed)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True, mx8=True, gamma=GAMMA_MX)
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k,
                                            mode=moe.MODE_PREFILL_MXFP8)
    torch.cuda.synchronize()
    what = f"MXFP8 T={T} H={H} I={I} E={E} k={k}"
    check_route(route, ref["idx"], ref["gates"], orc.permute(ref["idx"], E), what)
    hb = host_bits(h)
    check_h(hb, ref["h"], ref["hpre"], ref["hbound"], what)
    _check_y_mx(y.cpu().numpy(), ref["y"],
                _y_from_h(orc, experts, ref["idx"], ref["gates"], hb, range(T)), what)
    return x, lg, w, y


MX_CASES = [  # (T, H, I, E, k): H and I multiples of 128
    (8, 256, 128, 16, 2),
    (1, 128, 128, 1, 1),       # minimum
    (37, 384, 256, 9, 3),      # ragged token tiles
    (70, 256, 128, 4, 4),      # k = E, more than 64 tokens per expert (two passes)
    (16, 512, 256, 24, 6),
    # K % 256 == 0, K >= 512: weight scales four blocks to a load, the last group short
    (20, 1536, 1024, 6, 3),    # 6 blocks on w1/w3 (last group of 2), 4 on w2 (one group)
    (12, 2560, 512, 4, 2),     # 10 blocks on w1/w3, 2 on w2
    (24, 768, 2304, 6, 2),     # 3 and 9 blocks: a one-block last pair
    (40, 5248, 384, 8, 2),     # K % 512 != 0 at large K: block-pair scale loads, half tail block
    (700, 512, 256, 20, 2),    # 1400 pairs: many-workgroup permutation, experts with two passes
]


@pytest.mark.parametrize("T,H,I,E,k", MX_CASES)
def test_forward_mxfp8_small(moe, orc, T, H, I, E, k):
    say(f"MXFP8 forward T={T} H={H} I={I} E={E} k={k}")
    _forward_mx(moe, orc, T, H, I, E, k, seed=T * 13 + H + I)


def test_mxfp8_differs_from_bf16_by_quantisation(moe, orc):
    """The mode's results are a different (coarser) computation from PREFILL's:
    the relative difference is that of FP8 activations, about 5e-2."""
    import torch
    x, lg, w, y8 = _forward_mx(moe, orc, 24, 256, 128, 8, 2, seed=5)
    yb = moe.moe_fp4_forward(dev_bits(x), torch.from_numpy(lg).cuda(), w, 2, mode=moe.MODE_PREFILL)
    torch.cuda.synchronize()
    a, b = y8.cpu().numpy().astype(np.float64), yb.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    say(f"  MXFP8 vs bf16 activations: rel_l2 = {rel:.3e}")
    assert 1e-3 < rel < 0.2


def test_prefill_chunk_mxfp8(moe, orc):
    """T=2048 at the full shape in the MXFP8 mode: routing bit-exact, x quantised
    bit-exact, y and h on 16 sampled tokens."""
    import torch
    wl = PREFILL
    say("MXFP8 prefill T=2048: generating the 384-expert layer")
    w = moe.ExpertWeights.from_dict(synth.layer_device(wl, layer=0))
    x = synth.gen_x(wl, 0)
    lg = synth.gen_logits(wl, 0)
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, wl.k,
                                            mode=moe.MODE_PREFILL_MXFP8)
    codes, scales = moe.moe_fp4_quant_mxfp8(dev_bits(x))
    torch.cuda.synchronize()
    idx, g = orc.route(lg, wl.k)
    check_route(route, idx, g, orc.permute(idx, wl.E), "MXFP8 prefill route")
    rng = np.random.default_rng(2049)
    toks = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 14, replace=False)]))
    rc, rs = orc.mx8_quant(pins.bf16_to_f64(x[toks]))
    assert np.array_equal(codes.cpu().numpy()[toks], rc) and np.array_equal(scales.cpu().numpy()[toks], rs)
    experts = {int(e): synth.expert_host(wl, 0, int(e)) for e in np.unique(idx[toks])}
    ref = orc.forward(wl.H, wl.I, wl.E, wl.k, x, lg, experts, tokens=toks, want_h=True, mx8=True,
                      gamma=GAMMA_MX)
    y = y.cpu().numpy()
    h = host_bits(h)
    pairs = (toks[:, None] * wl.k + np.arange(wl.k)[None, :]).ravel()
    check_h(h[pairs], ref["h"][pairs], ref["hpre"][pairs], ref["hbound"][pairs], "MXFP8 prefill sampled h")
    _check_y_mx(y[toks], ref["y"], _y_from_h(orc, experts, idx, g, h, toks), "MXFP8 prefill sampled y")
    assert np.all(np.isfinite(y))
    del w
    torch.cuda.empty_cache()
