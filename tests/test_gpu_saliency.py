"""GPU parity of the saliency side output of the prefill w2 GEMMs:
saliency[e] += sum over the pairs routed to e of gate * ||expert output||_2.

The expert outputs are fp32 sums (and, in the MXFP8 mode, follow discrete
quantisation decisions), so each expert's saliency is compared with the
oracle's within a relative tolerance: 1e-3 with bf16 activations, 5e-3 with
MXFP8 ones (the FP8 codes of h follow the GPU's own h, see the MXFP8 tests).
The sums run in a fixed order, so repeated calls are compared bit for bit."""
import numpy as np
import pytest

import pins
import synth
from synth.configs import PREFILL
from gpu_common import dev_bits, dev_weights, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


def _check_sal(got, ref, rtol, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    bad = np.argwhere(err > rtol * np.abs(ref) + 1e-30)
    assert bad.size == 0, (what, [(int(b[0]), got[b[0]], ref[b[0]]) for b in bad[:5]])


SAL_CASES = [  # (T, H, I, E, k, mode, scale shift): shift 1 takes the register-fed kernels
    (40, 256, 128, 24, 6, 2, 0),
    (40, 512, 256, 24, 6, 2, 0),
    (40, 512, 256, 24, 6, 2, 1),
    (70, 256, 128, 4, 4, 2, 0),     # more than 64 tokens per expert: several passes
    (40, 512, 256, 24, 6, 3, 0),    # MXFP8
    (9, 384, 256, 7, 2, 3, 0),      # MXFP8, K = 384 (a half block)
]


def _weights_shifted(moe, experts, E, shift):
    """The experts' tensors as one blob each, scale tensors `shift` bytes off a
    16-byte boundary (shift 1 makes the bf16 prefill use its register kernels)."""
    import torch
    if shift == 0:
        dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
        return dev_weights(dense)
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    sizes = [experts[0][n].size for n in names]
    offs, o = [], 0
    for n, sz in zip(names, sizes):
        o = (o + 15) // 16 * 16 + (shift if n.startswith("s") else 0)
        offs.append(o)
        o += sz
    buf = np.zeros((E, (o + 255) // 256 * 256), np.uint8)
    for e in range(E):
        for n, off, sz in zip(names, offs, sizes):
            buf[e, off:off + sz] = experts[e][n].ravel()
    dbuf = torch.from_numpy(buf).cuda()
    views = {n: dbuf.view(-1)[off:] for n, off in zip(names, offs)}
    I = experts[0]["w1"].shape[0]
    return moe.ExpertWeights(strides=(buf.shape[1],) * 6, I=I, **views), dbuf


@pytest.mark.parametrize("T,H,I,E,k,mode,shift", SAL_CASES)
def test_saliency_small(moe, orc, T, H, I, E, k, mode, shift):
    import torch
    say(f"saliency T={T} H={H} I={I} E={E} k={k} mode={mode} shift={shift}")
    rng = np.random.default_rng(T * 7 + H + E + mode + shift)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    wts = _weights_shifted(moe, experts, E, shift)
    keep = None
    if isinstance(wts, tuple):
        wts, keep = wts
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    xd, lgd = dev_bits(x), torch.from_numpy(lg).cuda()
    y1, s1 = moe.moe_fp4_forward_saliency(xd, lgd, wts, k, mode=mode)
    y2, s2 = moe.moe_fp4_forward_saliency(xd, lgd, wts, k, saliency=s1.clone(), mode=mode)
    y0 = moe.moe_fp4_forward(xd, lgd, wts, k, mode=mode)
    torch.cuda.synchronize()
    s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.array_equal(y1.cpu().numpy().view(np.uint32), y0.cpu().numpy().view(np.uint32))
    assert np.array_equal(s2, 2 * s1)  # the second call adds the same bits again
    ref = orc.saliency(H, I, E, k, x, lg, experts, mx8=(mode == 3))
    _check_sal(s1, ref, 5e-3 if mode == 3 else 1e-3, f"saliency mode={mode}")
    idx, _ = orc.route(lg, k)
    assert np.all(s1[np.setdiff1d(np.arange(E), idx)] == 0.0)
    del keep


@pytest.mark.parametrize("mode", [2, 3], ids=["bf16", "mxfp8"])
def test_saliency_prefill_chunk(moe, orc, mode):
    """The 2048-token chunk: the saliency of all 384 experts against the oracle
    (each summed over all of the expert's tokens, the pages' signal summed over
    the tokens), and exactly zero for experts without tokens."""
    import torch
    wl = PREFILL
    say(f"saliency on the 2048-token chunk, mode={mode}")
    w = moe.ExpertWeights.from_dict(synth.layer_device(wl, layer=0))
    x = synth.gen_x(wl, 0)
    lg = synth.gen_logits(wl, 0)
    y, sal = moe.moe_fp4_forward_saliency(dev_bits(x), torch.from_numpy(lg).cuda(), w, wl.k,
                                          mode=mode)
    torch.cuda.synchronize()
    sal = sal.cpu().numpy()
    del w
    torch.cuda.empty_cache()
    idx, _ = orc.route(lg, wl.k)
    counts = np.bincount(idx.ravel(), minlength=wl.E)
    assert np.all(np.isfinite(sal)) and np.all((sal > 0) == (counts > 0))
    used = [int(e) for e in np.nonzero(counts)[0]]
    say(f"  oracle saliency of the {len(used)} experts with tokens")
    experts = {e: synth.expert_host(wl, 0, e) for e in used}
    ref = orc.saliency(wl.H, wl.I, wl.E, wl.k, x, lg, experts, expert_list=used, mx8=(mode == 3))
    _check_sal(sal[used], ref, 5e-3 if mode == 3 else 1e-3, f"chunk saliency mode={mode}")
