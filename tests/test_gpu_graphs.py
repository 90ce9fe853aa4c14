"""Every entry point's kernel paths captured in a HIP graph and replayed: each
replay, with new inputs copied into the captured buffers by eager work between
replays, equals an eager call on the same inputs bit for bit.  No path may
record a memset node or any allocation, and nothing a call leaves behind may
change the next one's result."""
import zlib

import numpy as np
import pytest

import pins
from gpu_common import dev_bits, dev_weights, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


CASES = [  # (name, T, H, I, E, k, mode, entry point)
    ("one_token", 1, 1024, 512, 32, 6, 0, "forward"),
    ("few_token", 6, 1024, 512, 32, 6, 0, "forward"),
    ("decode_mfma", 1, 16384, 64, 4, 2, 1, "forward"),
    ("prefill_many_workgroup_permutation", 300, 512, 256, 24, 4, 2, "forward"),
    ("mxfp8", 100, 512, 256, 16, 4, 3, "forward"),
    ("routed_one_token", 1, 1024, 512, 32, 6, 0, "routed"),
    ("routed_prefill", 40, 512, 256, 24, 6, 2, "routed"),
    ("shared_one_token", 1, 1024, 512, 12, 3, 1, "shared"),
    ("shared_prefill", 40, 256, 128, 16, 2, 2, "shared"),
    ("residual_one_token", 1, 1024, 512, 32, 6, 0, "residual"),
    ("residual_prefill", 40, 256, 128, 24, 6, 2, "residual"),
    ("noalloc_one_token", 1, 1024, 512, 32, 6, 0, "noalloc"),
    ("saliency", 64, 512, 256, 16, 4, 2, "saliency"),
]


@pytest.mark.parametrize("name,T,H,I,E,k,mode,entry", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager(moe, name, T, H, I, E, k, mode, entry):
    import torch
    say(f"graph {name}: T={T} H={H} I={I} E={E} k={k} mode={mode} path "
        f"{moe.moe_fp4_plan(T, H, I, E, k, mode)}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    experts = [pins.random_expert(rng, H, I) for _ in range(E)]
    w = dev_weights({n: np.stack([e[n] for e in experts]) for n in experts[0]})
    sw = None
    if entry == "shared":
        sw = moe.SharedWeights.from_dict({n: torch.from_numpy(np.ascontiguousarray(a)).cuda()
                                          for n, a in pins.random_shared(rng, H, I).items()})
    wr = dev_bits(pins.rand_bf16(rng, (E, H), 1.0 / np.sqrt(H))) if entry == "routed" else None
    ws = torch.empty(moe.moe_fp4_workspace_size(T, H, I, E, k, mode), dtype=torch.uint8, device="cuda")
    xb = dev_bits(pins.rand_bf16(rng, (T, H)))
    xf = torch.empty((T, H), dtype=torch.float32, device="cuda")
    lb = torch.empty((T, E), dtype=torch.float32, device="cuda")
    yb = torch.empty((T, H), dtype=torch.float32, device="cuda")
    sal = torch.zeros(E, dtype=torch.float32, device="cuda")

    def call(y, s):
        if entry == "forward":
            moe.moe_fp4_forward(xb, lb, w, k, y=y, mode=mode, workspace=ws)
        elif entry == "routed":
            moe.moe_fp4_forward_routed(xb, wr, w, k, y=y, mode=mode, workspace=ws)
        elif entry == "shared":
            moe.moe_fp4_forward_shared(xb, lb, w, sw, k, y=y, mode=mode, workspace=ws)
        elif entry == "residual":
            moe.moe_fp4_forward_residual(xf, lb, w, k, mode=mode, workspace=ws)
        elif entry == "noalloc":
            moe.moe_fp4_forward_noalloc(xb, lb, w, k, y=y, mode=mode)
        else:
            moe.moe_fp4_forward_saliency(xb, lb, w, k, saliency=s, y=y, mode=mode, workspace=ws)

    def new_inputs():
        xb.copy_(dev_bits(pins.rand_bf16(rng, (T, H))))
        lb.copy_(torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)))
        x0 = torch.from_numpy((rng.standard_normal((T, H)) * 3.0).astype(np.float32)).cuda()
        xf.copy_(x0)
        sal.zero_()
        return x0

    stream = torch.cuda.Stream()
    new_inputs()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        call(yb, sal)  # eager on the capture stream first (the no-alloc array's address is looked up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(yb, sal)
    torch.cuda.synchronize()
    for rep in range(4):
        x0 = new_inputs()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (xf if entry == "residual" else yb).clone()
        got_sal = sal.clone()
        # the same inputs eagerly
        xf.copy_(x0)
        sal.zero_()
        y2 = torch.empty_like(yb)
        call(y2, sal)
        torch.cuda.synchronize()
        want = xf if entry == "residual" else y2
        assert torch.isfinite(got).all(), (name, rep)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), (name, rep)
        if entry == "saliency":
            assert torch.equal(got_sal.view(torch.int32), sal.view(torch.int32)), (name, rep)
    say(f"  {name}: 4 replays equal the eager calls")
