"""moe_fp4_forward_noalloc, the entry point that allocates nothing (its
workspace is the library's static per-GPU array), against moe_fp4_forward with
a workspace of its own: the same kernels run, so y must match bit for bit.
Calls come in pairs, the second smaller than the first, so the second runs on
whatever the first left in the shared array."""
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


PAIRS = [  # two calls in a row, (T, H, I, E, k, mode), the second smaller
    ((1, 2048, 1024, 32, 6, 1), (1, 512, 256, 16, 2, 1)),         # one-token decode path
    ((12, 1024, 512, 16, 4, 0), (3, 512, 256, 16, 4, 0)),         # few-token decode path
    ((96, 1024, 512, 24, 4, 2), (9, 512, 256, 8, 2, 2)),          # prefill GEMMs
    ((64, 1024, 512, 16, 2, 3), (16, 512, 256, 8, 2, 3)),         # MXFP8 prefill
]


def _case(moe, T, H, I, E, k, mode, seed, accumulate):
    import torch
    rng = np.random.default_rng(seed)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    w = dev_weights({n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]})
    x = dev_bits(pins.rand_bf16(rng, (T, H)))
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    y0 = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).cuda()
    y_ref = y0.clone() if accumulate else None
    y_ref = moe.moe_fp4_forward(x, lg, w, k, y=y_ref, mode=mode, accumulate=accumulate)
    y_na = y0.clone() if accumulate else None
    y_na = moe.moe_fp4_forward_noalloc(x, lg, w, k, y=y_na, mode=mode, accumulate=accumulate)
    torch.cuda.synchronize()
    a, b = y_ref.cpu().numpy(), y_na.cpu().numpy()
    assert np.all(np.isfinite(b))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
        (T, H, I, E, k, mode, float(np.abs(a - b).max()))


@pytest.mark.parametrize("first,second", PAIRS, ids=["one_token", "few_tokens", "prefill", "mxfp8"])
def test_noalloc_equals_forward(moe, first, second):
    for n, (shape, acc) in enumerate(((first, False), (second, True))):
        say(f"no-alloc forward, call {n + 1}: T,H,I,E,k,mode = {shape}, accumulate={acc}")
        _case(moe, *shape, seed=sum(shape) + n, accumulate=acc)


def test_noalloc_refuses_a_chunk(moe):
    import torch
    T, H, I, E, k = 2048, 512, 256, 8, 2
    need = moe.moe_fp4_workspace_size(T, H, I, E, k, moe.MODE_PREFILL)
    assert need > (8 << 20)
    w = moe.ExpertWeights.from_dict({n: torch.zeros((E,) + s, dtype=torch.uint8, device="cuda")
                                     for n, s in {"w1": (I, H // 2), "s1": (I, H // 32),
                                                  "w3": (I, H // 2), "s3": (I, H // 32),
                                                  "w2": (H, I // 2), "s2": (H, I // 32)}.items()})
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeFp4Error) as ei:
        moe.moe_fp4_forward_noalloc(x, lg, w, k, mode=moe.MODE_PREFILL)
    from mxfp4_routed_expert_router_amd import _lib
    assert ei.value.status == _lib.EWORKSPACE
