"""GPU parity of the shared expert (FP8 E4M3 weights, 32 x 32 UE8M0 block
scales) and of the layer with it added.

h is held to the same interval rule as the routed path's h (the oracle's
exact value and fp32 evaluation bound); y to the layer's tolerances (rel-L2
<= 2e-3, max-abs <= 2e-2 RMS)."""
import numpy as np
import pytest

import accum
import pins
import synth
from synth.configs import DECODE
from gpu_common import check_h, check_y, dev_bits, dev_weights, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


def _dev_shared(moe, sw):
    import torch
    return moe.SharedWeights.from_dict({n: torch.from_numpy(np.ascontiguousarray(a)).cuda()
                                        for n, a in sw.items()})


SHARED_CASES = [  # (T, H, I): T = 1 on the one-token decode kernels where they fit,
    # T <= 4 one wave per row, T > 4 MFMA tiles
    (1, 256, 128),
    (1, 5120, 2304),     # one token at the real shape
    (1, 256, 4128),      # one token, a w2 row of 258 chunks: the one-wave-per-row kernels
    (1, 8224, 64),       # one token, H past the one-token kernels: the one-wave-per-row kernels
    (3, 224, 96),        # 7 and 3 chunks of 32 columns: ragged lanes
    (4, 5120, 2304),     # the real shape
    (5, 256, 128),
    (70, 352, 160),      # K = 352 and 160: a half block at the end; ragged tiles
    (130, 512, 256),
]


@pytest.mark.parametrize("T,H,I", SHARED_CASES)
def test_shared_expert(moe, orc, T, H, I):
    import torch
    say(f"shared expert T={T} H={H} I={I}")
    rng = np.random.default_rng(T * 17 + H + I)
    sw = pins.random_shared(rng, H, I)
    x = pins.rand_bf16(rng, (T, H))
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    dsw, xd = _dev_shared(moe, sw), dev_bits(x)
    y, h = moe.moe_fp4_shared_expert(xd, dsw)
    y2, _ = moe.moe_fp4_shared_expert(xd, dsw)
    ya, _ = moe.moe_fp4_shared_expert(xd, dsw, y=torch.from_numpy(y0).cuda(), accumulate=True)
    torch.cuda.synchronize()
    ref = orc.shared(x, sw, want_h=True, acc=accum.shared_model(T, H))
    what = f"shared T={T} H={H} I={I}"
    check_h(host_bits(h), ref["h"], ref["hpre"], ref["hbound"], what)
    y = y.cpu().numpy()
    check_y(y, ref["y"], what)
    assert np.array_equal(y.view(np.uint32), y2.cpu().numpy().view(np.uint32))
    check_y(ya.cpu().numpy(), y0.astype(np.float64) + ref["y"], what + " accumulate")


@pytest.mark.parametrize("mode,T", [(1, 1), (1, 2), (2, 40), (3, 40)],
                         ids=["decode1", "decode2", "prefill", "mxfp8"])
def test_forward_shared(moe, orc, mode, T):
    """forward_shared is forward followed by the shared expert added to y (bit
    for bit), and matches the oracle's routed layer plus its shared expert.
    One token carries the shared rows in the routed launches."""
    import torch
    H, I, E, k = (256, 128, 16, 2) if mode == 1 else (256, 128, 24, 6)
    say(f"forward_shared T={T} mode={mode}")
    rng = np.random.default_rng(5 + mode)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    sw = pins.random_shared(rng, H, I)
    dsw = _dev_shared(moe, sw)
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xd, lgd = dev_bits(x), torch.from_numpy(lg).cuda()
    y = moe.moe_fp4_forward_shared(xd, lgd, w, dsw, k, mode=mode)
    y1 = moe.moe_fp4_forward(xd, lgd, w, k, mode=mode)
    y1, _ = moe.moe_fp4_shared_expert(xd, dsw, y=y1, accumulate=True)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y1.cpu().numpy().view(np.uint32))
    if mode != 3:
        ref = orc.forward(H, I, E, k, x, lg, experts)["y"].astype(np.float64) + orc.shared(x, sw)["y"]
        check_y(y, ref, f"forward_shared mode={mode}")


def test_forward_shared_one_token_accumulate(moe, orc):
    """One token with MOE_FP4_ACCUMULATE (the shared rows carried in the
    routed launches): y0 + layer + shared expert, bit for bit the separate
    calls', and the oracle's sum to the layer tolerance."""
    import torch
    T, H, I, E, k = 1, 512, 256, 12, 3
    say("forward_shared T=1 accumulate")
    rng = np.random.default_rng(31)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    sw = pins.random_shared(rng, H, I)
    dsw = _dev_shared(moe, sw)
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    xd, lgd = dev_bits(x), torch.from_numpy(lg).cuda()
    ya = torch.from_numpy(y0).cuda()
    moe.moe_fp4_forward_shared(xd, lgd, w, dsw, k, y=ya, mode=1, accumulate=True)
    yb = torch.from_numpy(y0).cuda()
    moe.moe_fp4_forward(xd, lgd, w, k, y=yb, mode=1, accumulate=True)
    moe.moe_fp4_shared_expert(xd, dsw, y=yb, accumulate=True)
    torch.cuda.synchronize()
    ya, yb = ya.cpu().numpy(), yb.cpu().numpy()
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    ref = (y0.astype(np.float64) + orc.forward(H, I, E, k, x, lg, experts)["y"].astype(np.float64)
           + orc.shared(x, sw)["y"])
    check_y(ya, ref, "forward_shared T=1 accumulate")


@pytest.mark.parametrize("H", [1024, 1568, 2048, 3072, 4096, 5120, 8192])
def test_forward_shared_one_token_row_parts(moe, orc, H):
    """One token: a shared expert's w1 row and w3 row are carried as two units
    of the routed w1/w3 kernel, each 1 to 8 16-byte chunks a lane over these H
    (at H = 1568 the second chunk of a lane covers only 34 of 64 lanes).  Bit
    for bit the separate calls, and the oracle's sum."""
    import torch
    T, I, E, k = 1, 256, 8, 2
    say(f"forward_shared T=1 H={H}")
    rng = np.random.default_rng(H)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    sw = pins.random_shared(rng, H, 384)
    dsw = _dev_shared(moe, sw)
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xd, lgd = dev_bits(x), torch.from_numpy(lg).cuda()
    y = moe.moe_fp4_forward_shared(xd, lgd, w, dsw, k, mode=1)
    y1 = moe.moe_fp4_forward(xd, lgd, w, k, mode=1)
    y1, _ = moe.moe_fp4_shared_expert(xd, dsw, y=y1, accumulate=True)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y1.cpu().numpy().view(np.uint32))
    ref = orc.forward(H, I, E, k, x, lg, experts)["y"].astype(np.float64) + orc.shared(x, sw)["y"]
    check_y(y, ref, f"forward_shared T=1 H={H}")


def test_forward_shared_decode_real_shape(moe, orc):
    """One token at the real shape: 6 of 384 routed experts plus the shared expert."""
    import torch
    wl = DECODE
    say("forward_shared, one token, real shape")
    w = moe.ExpertWeights.from_dict(synth.layer_device(wl, layer=0))
    sw = synth.gen_shared(wl)
    x = synth.gen_x(wl, 5)
    lg = synth.gen_logits(wl, 5)
    dsw, xd, lgd = _dev_shared(moe, sw), dev_bits(x), torch.from_numpy(lg).cuda()
    y = moe.moe_fp4_forward_shared(xd, lgd, w, dsw, wl.k)
    y1 = moe.moe_fp4_forward(xd, lgd, w, wl.k)
    y1, _ = moe.moe_fp4_shared_expert(xd, dsw, y=y1, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32))
    idx, _ = orc.route(lg, wl.k)
    experts = {int(e): synth.expert_host(wl, 0, int(e)) for e in idx[0]}
    ref = orc.forward(wl.H, wl.I, wl.E, wl.k, x, lg, experts)["y"].astype(np.float64)
    ref += orc.shared(x, sw)["y"]
    check_y(y.cpu().numpy(), ref, "forward_shared, real shape")
    del w
    torch.cuda.empty_cache()
