"""GPU parity of the router-logits step (x . Wr^T, Wr bf16 [E, H]) and of the
forward that starts from it.

The logits are a floating-point sum, so they are compared with the oracle's
exact (double) value within the bound on an fp32 evaluation that the oracle
returns with it (gamma_H sum |x w|).  The routing taken from them is an integer
decision: it is compared bit for bit with the oracle's routing of the GPU's own
logits, and with the oracle's routing of the exact logits wherever the k-th
and (k+1)-th logits are further apart than the bound allows a flip."""
import numpy as np
import pytest

import pins
import synth
from synth.configs import DECODE, PREFILL
from gpu_common import check_route, check_y, dev_bits, dev_weights, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


def _check_logits(got, exact, bound, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - exact)
    lim = bound + np.abs(exact) * 2.0 ** -24
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (what, [(tuple(b), got[tuple(b)], exact[tuple(b)], lim[tuple(b)])
                                  for b in bad[:5]])


def _flip_safe(exact, bound, k):
    """Tokens whose top-k set and order cannot change within the bound: every
    adjacent gap among the first k + 1 sorted logits exceeds twice the bound."""
    order = np.argsort(-exact, axis=1, kind="stable")[:, :k + 1]
    v = np.take_along_axis(exact, order, 1)
    b = 2 * np.take_along_axis(bound, order, 1).max(axis=1, keepdims=True)
    return np.all(np.diff(-v, axis=1) > b, axis=1)


ROUTER_CASES = [  # (T, H, E): T <= 4 takes the one-wave-per-expert kernel, T > 4 the MFMA tiles
    (1, 5120, 384),
    (3, 256, 19),
    (4, 96, 7),
    (5, 224, 19),
    (70, 352, 138),      # ragged token and expert tiles
    (130, 512, 64),
]


@pytest.mark.parametrize("T,H,E", ROUTER_CASES)
def test_router_logits(moe, orc, T, H, E):
    import torch
    say(f"router logits T={T} H={H} E={E}")
    rng = np.random.default_rng(T * 31 + H + E)
    x = pins.rand_bf16(rng, (T, H))
    w = pins.rand_bf16(rng, (E, H), scale=1.0 / np.sqrt(H))
    xd, wd = dev_bits(x), dev_bits(w)
    a = moe.moe_fp4_router_logits(xd, wd)
    b = moe.moe_fp4_router_logits(xd, wd)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "logits differ between runs"
    exact, bound = orc.router_logits(x, w)
    _check_logits(a, exact, bound, f"T={T} H={H} E={E}")


def test_router_logits_extremes(moe, orc):
    """Large, tiny and cancelling products, a zero row of x."""
    import torch
    rng = np.random.default_rng(77)
    T, H, E = 6, 512, 40
    xf = rng.standard_normal((T, H)) * np.ldexp(1.0, rng.integers(-20, 20, (T, H)))
    xf[2] = 0.0
    x = np.array([[orc.to_bf16(v) for v in row] for row in xf], np.uint16)
    w = pins.rand_bf16(rng, (E, H))
    w[5] = w[4] ^ 0x8000  # row 5 = -row 4: logits cancelling against row 4's
    got = moe.moe_fp4_router_logits(dev_bits(x), dev_bits(w))
    torch.cuda.synchronize()
    exact, bound = orc.router_logits(x, w)
    got = got.cpu().numpy()
    _check_logits(got, exact, bound, "extremes")
    assert np.all(got[2] == 0.0)
    # the matrix cores' internal accumulation is not sign-symmetric bit for bit,
    # so -row 4 is held to the bound, as every logit is (above)
    assert np.all(np.abs(got[:, 5] + got[:, 4]) <= bound[:, 4] + bound[:, 5])


def test_router_logits_prefill_shape(moe, orc):
    """T = 2048, H = 5120, E = 384 (the prefill chunk), sampled tokens."""
    import torch
    wl = PREFILL
    say("router logits at the prefill chunk's shape")
    x = synth.gen_x(wl, 0)
    w = synth.gen_router(wl)
    got = moe.moe_fp4_router_logits(dev_bits(x), dev_bits(w))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 63, 64, wl.T - 1],
                                     np.random.default_rng(5).choice(wl.T, 12, replace=False)]))
    exact, bound = orc.router_logits(x[toks], w)
    _check_logits(got.cpu().numpy()[toks], exact, bound, "prefill shape")


ROUTED_CASES = [  # (T, H, I, E, k, mode)
    (1, 256, 128, 16, 2, 1),     # one-token decode: routing inside the w1/w3 kernel
    (2, 256, 128, 16, 2, 1),     # decode MFMA path
    (40, 256, 128, 24, 6, 2),    # prefill
    (40, 256, 128, 24, 6, 3),    # prefill, MXFP8 activations
]


@pytest.mark.parametrize("T,H,I,E,k,mode", ROUTED_CASES)
def test_forward_routed(moe, orc, T, H, I, E, k, mode):
    """forward_routed(x, Wr) is forward(x, router_logits(x, Wr)) bit for bit,
    its routing is the oracle's routing of those logits, and y meets the
    layer's tolerance against the oracle on them (bf16 modes)."""
    import torch
    say(f"forward_routed T={T} H={H} I={I} E={E} k={k} mode={mode}")
    rng = np.random.default_rng(T + 100 * mode)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    wts = dev_weights(dense)
    x = pins.rand_bf16(rng, (T, H))
    wr = pins.rand_bf16(rng, (E, H), scale=1.0 / np.sqrt(H))
    xd, wrd = dev_bits(x), dev_bits(wr)
    y1 = moe.moe_fp4_forward_routed(xd, wrd, wts, k, mode=mode)
    lg = moe.moe_fp4_router_logits(xd, wrd)
    y2, _, route = moe.moe_fp4_forward_debug(xd, lg, wts, k, mode=mode)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    lg = lg.cpu().numpy()
    idx, g = orc.route(lg, k)
    check_route(route, idx, g, orc.permute(idx, E), f"routed T={T} mode={mode}")
    exact, bound = orc.router_logits(x, wr)
    safe = _flip_safe(exact, bound, k)
    idx_exact, _ = orc.route(exact.astype(np.float32), k)
    assert safe.mean() > 0.5
    assert np.array_equal(idx[safe], idx_exact[safe])
    if mode != 3:
        ref = orc.forward(H, I, E, k, x, lg, experts)
        check_y(y1.cpu().numpy(), ref["y"], f"routed T={T} mode={mode}")


def test_forward_routed_decode_shape(moe, orc):
    """One token at the real shape (384 experts): the routed decode picks the
    experts the oracle picks from the GPU's logits; y on them within tolerance."""
    import torch
    wl = DECODE
    say("forward_routed, one token, 384 experts")
    w = moe.ExpertWeights.from_dict(synth.layer_device(wl, layer=0))
    wr = synth.gen_router(wl)
    x = synth.gen_x(wl, 3)
    xd, wrd = dev_bits(x), dev_bits(wr)
    y = moe.moe_fp4_forward_routed(xd, wrd, w, wl.k)
    lg = moe.moe_fp4_router_logits(xd, wrd)
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    idx, _ = orc.route(lg, wl.k)
    experts = {int(e): synth.expert_host(wl, 0, int(e)) for e in idx[0]}
    ref = orc.forward(wl.H, wl.I, wl.E, wl.k, x, lg, experts)
    check_y(y.cpu().numpy(), ref["y"], "routed decode, real shape")
    del w
    torch.cuda.empty_cache()
