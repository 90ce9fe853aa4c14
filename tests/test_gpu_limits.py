"""GPU parity at the top of the C-ABI's token range (T = 65535): the routing
and permutation of a quarter and of one million pairs bit for bit, and the
prefill modes on a layer whose experts hold thousands of tokens each (the
grouped GEMMs then make up to 1024 passes over an expert's weights), every
token's h and y against the oracle.  Small H and I keep the oracle's share to
seconds."""
import numpy as np
import pytest

import accum
import pins
from gpu_common import check_h, check_route, check_y, dev_bits, dev_weights, host_bits, say
from test_gpu_mx8 import MX_H_REL_L2, check_mx_y

pytestmark = pytest.mark.gpu

T_MAX = 65535


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


@pytest.mark.parametrize("E,k", [(384, 6), (1024, 16)])
def test_route_at_token_limit(moe, orc, E, k):
    """moe_fp4_route at T = 65535: 393,210 and 1,048,560 pairs through the
    many-workgroup permutation (256 workgroups at the larger)."""
    import torch
    say(f"route T={T_MAX} E={E} k={k}")
    rng = np.random.default_rng(E + k)
    lg = rng.standard_normal((T_MAX, E)).astype(np.float32)
    lg[:, :8] = np.round(lg[:, :8], 1)  # exact ties among the first experts
    r = moe.moe_fp4_route(torch.from_numpy(lg).cuda(), k)
    torch.cuda.synchronize()
    idx, g = orc.route(lg, k)
    check_route(r, idx, g, orc.permute(idx, E), f"T={T_MAX} E={E} k={k}")


@pytest.mark.parametrize("H,I,E,k,mode", [
    (256, 128, 32, 2, 2),     # bf16: w1/w3 on the LDS-fed GEMMs, w2 (K = 128) on the register-fed ones
    (256, 256, 16, 2, 2),     # bf16: both GEMMs LDS-fed, about 8,200 tokens an expert
    (256, 128, 1, 1, 2),      # one expert takes every token: 1024 passes
    (256, 128, 32, 2, 3),     # MXFP8
], ids=["bf16", "bf16_lds", "one_expert", "mxfp8"])
def test_forward_at_token_limit(moe, orc, H, I, E, k, mode):
    import torch
    say(f"forward T={T_MAX} H={H} I={I} E={E} k={k} mode={mode}")
    rng = np.random.default_rng(H + I + E + k + mode)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    x = pins.rand_bf16(rng, (T_MAX, H))
    lg = rng.standard_normal((T_MAX, E)).astype(np.float32)
    mx = mode == moe.MODE_PREFILL_MXFP8
    acc = accum.model("mx8", H) if mx else accum.forward_model(T_MAX, H, I, E, k, mode)
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True, mx8=mx, acc=acc)
    w = dev_weights({n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]})
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k, mode=mode)
    torch.cuda.synchronize()
    what = f"T={T_MAX} H={H} I={I} E={E} k={k} mode={mode}"
    check_route(route, ref["idx"], ref["gates"], orc.permute(ref["idx"], E), what)
    hb = host_bits(h)
    check_h(hb, ref["h"], ref["hpre"], ref["hbound"], what, MX_H_REL_L2 if mx else None)
    if mx:
        check_mx_y(orc, experts, route, hb, y.cpu().numpy(), ref["y"], H, I, what)
    else:
        check_y(y.cpu().numpy(), ref["y"], what)
