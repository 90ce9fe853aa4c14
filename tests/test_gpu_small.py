"""GPU parity at small shapes: the HIP path against the CPU oracle, element by
element, through the C-ABI.  Shapes span several tiles and ragged tails."""
import numpy as np
import pytest

import accum
import pins
from gpu_common import bf16_value, check_h, check_route, check_y, dev_bits, dev_weights, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_routed_expert_router_amd as m
    return m


def _route_ref(orc, lg, k, E):
    idx, g = orc.route(lg, k)
    return idx, g, orc.permute(idx, E)


def _gpu_route(moe, lg, k):
    import torch
    r = moe.moe_fp4_route(torch.from_numpy(np.ascontiguousarray(lg)).cuda(), k)
    torch.cuda.synchronize()
    return r


# --------------------------------------------------------------------------- router
ROUTE_CASES = [  # (T, E, k, seed)
    (1, 1, 1, 0), (1, 384, 6, 1), (8, 16, 2, 2), (6, 384, 6, 3), (32, 384, 6, 4), (64, 384, 6, 5),
    (65, 384, 6, 6), (2048, 384, 6, 7), (3, 1024, 16, 8), (100, 1024, 16, 9), (5, 16, 16, 10),
    (3000, 7, 7, 11), (200, 138, 6, 12), (171, 64, 1, 13),
    # the one-launch routing at its limits: 1024 pairs over 1024 experts, and
    # 1024 pairs over 64 experts (each expert's 64-token mask full or nearly)
    (64, 1024, 16, 14), (64, 64, 16, 15), (64, 17, 16, 16),
]


@pytest.mark.parametrize("T,E,k,seed", ROUTE_CASES)
def test_route_random(moe, orc, T, E, k, seed):
    say(f"route T={T} E={E} k={k}")
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, g, perm = _route_ref(orc, lg, k, E)
    check_route(_gpu_route(moe, lg, k), idx, g, perm, f"T={T} E={E} k={k}")


def test_route_ties_zero_nan(moe, orc):
    say("route ties / -0 / NaN / inf")
    rng = np.random.default_rng(42)
    T, E, k = 40, 100, 8
    lg = np.round(rng.standard_normal((T, E)), 1).astype(np.float32)  # many exact ties
    lg[0, :] = 0.5
    lg[1, ::2] = -0.0
    lg[1, 1::2] = 0.0
    lg[2, 5] = np.nan
    lg[2, 7] = np.inf
    lg[2, 9] = -np.inf
    lg[3, :] = np.nan
    lg[4, :50] = -np.inf
    idx, g, perm = _route_ref(orc, lg, k, E)
    r = _gpu_route(moe, lg, k)
    assert np.array_equal(r.topk_idx.cpu().numpy(), idx)
    for name, ref in zip(("counts", "offsets", "sorted_pairs", "pair_slot"), perm):
        assert np.array_equal(getattr(r, name).cpu().numpy(), ref), name
    ok = np.isfinite(lg).all(axis=1) | (np.arange(T) > 4)
    gg = r.gates.cpu().numpy()
    assert np.max(np.abs(gg[ok] - g[ok])) <= 1e-6


def _one_token_rows(rng, E):
    """Logit rows for the one-token kernel's in-kernel ranking: exact ties,
    neighbouring floats at the top (keys equal but for their lowest bits),
    signed zeros, NaN and infinities, and plain rows."""
    rows = [rng.standard_normal(E).astype(np.float32) for _ in range(3)]
    r = np.round(rng.standard_normal(E), 1).astype(np.float32)  # many exact ties
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32)
    top = np.float32(3.0)
    for j, e in enumerate((17, 250, 3, 99, 300, 64, 128)):  # 3.0 and its neighbours
        v = top
        for _ in range(j % 4):
            v = np.nextafter(v, np.float32(np.inf) if j % 2 else np.float32(-np.inf))
        r[e] = v
    rows.append(r)
    r = np.zeros(E, np.float32)
    r[::2] = -0.0
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32)
    r[5], r[7], r[9], r[200] = np.nan, np.inf, -np.inf, np.inf
    rows.append(r)
    return rows


def test_one_token_routing_ties(moe, orc):
    """The one-token kernel ranks the logits itself: bit-exact against the
    oracle on ties, near-ties, signed zeros, NaN and infinities."""
    import torch
    say("one-token in-kernel routing: ties and near-ties")
    rng = np.random.default_rng(77)
    H, I, E, k = 256, 128, 384, 6
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    x = pins.rand_bf16(rng, (1, H))
    for i, row in enumerate(_one_token_rows(rng, E)):
        lg = row[None, :]
        idx, g, perm = _route_ref(orc, lg, k, E)
        _, _, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k,
                                                mode=moe.MODE_DECODE)
        torch.cuda.synchronize()
        assert np.array_equal(route.topk_idx.cpu().numpy(), idx), f"row {i}"
        for name, ref in zip(("counts", "offsets", "sorted_pairs", "pair_slot"), perm):
            assert np.array_equal(getattr(route, name).cpu().numpy(), ref), f"row {i} {name}"
        if np.isfinite(row).all():
            assert np.max(np.abs(route.gates.cpu().numpy() - g)) <= 1e-6, f"row {i}"


def test_route_repeatable(moe):
    say("route twice, bitwise")
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((2048, 384)).astype(np.float32)
    a, b = _gpu_route(moe, lg, 6), _gpu_route(moe, lg, 6)
    for n in ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot"):
        assert np.array_equal(getattr(a, n).cpu().numpy(), getattr(b, n).cpu().numpy()), n


# --------------------------------------------------------------------------- forward
def decode_supported(moe, T, H, I, E, k):
    try:
        moe.moe_fp4_workspace_size(T, H, I, E, k, moe.MODE_DECODE)
        return True
    except moe.MoeFp4Error:
        return False


def _forward_case(moe, orc, T, H, I, E, k, seed, mode, scale_lo=120, scale_hi=124, accumulate=False):
    import torch
    rng = np.random.default_rng(seed)
    experts = {e: pins.random_expert(rng, H, I, scale_lo, scale_hi) for e in range(E)}
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True,
                      acc=accum.forward_model(T, H, I, E, k, mode))
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    y0 = None
    if accumulate:
        y0 = rng.standard_normal((T, H)).astype(np.float32)
        y_in = torch.from_numpy(y0).cuda()
    else:
        y_in = None
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k, y=y_in,
                                            mode=mode, accumulate=accumulate)
    torch.cuda.synchronize()
    what = f"T={T} H={H} I={I} E={E} k={k} mode={mode}"
    check_route(route, ref["idx"], ref["gates"], orc.permute(ref["idx"], E), what)
    check_h(host_bits(h), ref["h"], ref["hpre"], ref["hbound"], what)
    want = ref["y"] if y0 is None else (y0.astype(np.float64) + ref["y"]).astype(np.float32)
    check_y(y.cpu().numpy(), want, what)


FORWARD_CASES = [  # (T, H, I, E, k)
    (8, 256, 128, 16, 2),     # the tiny workload's shape
    (5, 352, 96, 7, 3),       # ragged: 11 input groups, 3 intermediate groups
    (1, 32, 32, 1, 1),        # minimum
    (3, 64, 32, 4, 4),        # k = E
    (16, 512, 256, 24, 6),
    (17, 224, 160, 9, 4),     # two decode token tiles
    (32, 256, 192, 6, 6),     # every expert takes all 32 tokens
    (16, 256, 128, 20, 2),    # a full 16-token decode tile
    (1, 352, 96, 7, 3),       # one token, ragged groups
    (1, 256, 2080, 10, 5),    # one token, 65 groups per w2 row
    (1, 256, 1024, 16, 16),   # one token, k = 16: k * I / 32 at the one-token path's limit
    (1, 1568, 96, 7, 3),      # one token, two slots a lane, the second one ragged (49 groups a row)
    (1, 3104, 160, 9, 4),     # one token, four slots, one group in the last
    (1, 8192, 128, 8, 4),     # one token, eight slots a lane (H = 8192)
    (1, 256, 128, 1024, 16),  # one token, E = 1024: the routing kernel feeds the one-token kernels
    (1, 512, 256, 600, 6),    # one token, E = 600 (above the 512 the w1/w3 kernel ranks itself)
    (64, 256, 128, 1024, 16), # 1024 pairs over 1024 experts: the one-launch routing's limit
    (100, 64, 32, 1024, 16),  # E = 1024, k = 16: the largest router tables, 1600 pairs
    (2, 8192, 256, 8, 4),     # few-token GEMV path, 4 groups a lane (H = 8192)
    (6, 1024, 2304, 12, 8),   # few-token path at T = 6, two (pair, group)s a lane in w2
    (4, 2080, 160, 5, 5),     # few-token path, k = E (every token on every expert), 65 groups a row
    (6, 256, 128, 2, 2),      # few-token path, two experts shared by all six tokens
    (8, 5120, 256, 16, 4),    # few-token path with 16-wave workgroups (x rows take 82 KB of LDS)
    (15, 4096, 128, 32, 6),   # few-token path at its token limit (124 KB of LDS)
    (15, 256, 512, 32, 16),   # few-token path with k = 16: 240 pairs
    (1, 16384, 64, 4, 2),     # H at its limit: T = 1 on the MFMA decode kernels
    (2, 64, 16384, 3, 2),     # I at its limit (prefill only)
]


@pytest.mark.parametrize("mode", [1, 2], ids=["decode", "prefill"])
@pytest.mark.parametrize("T,H,I,E,k", FORWARD_CASES)
def test_forward_small(moe, orc, T, H, I, E, k, mode):
    if mode == 1 and not decode_supported(moe, T, H, I, E, k):
        pytest.skip("shape outside the decode path's range")
    say(f"forward T={T} H={H} I={I} E={E} k={k} mode={mode}")
    _forward_case(moe, orc, T, H, I, E, k, seed=T * 7 + H + I, mode=mode)


@pytest.mark.parametrize("T", [40, 130, 300, 700, 3000])
def test_forward_prefill_many_tokens(moe, orc, T):
    """Experts with more than 64 tokens (several passes); above 1024 pairs
    (T = 700, 3000) the permutation runs on many workgroups."""
    say(f"forward prefill T={T}: experts with more than 64 tokens (several passes)")
    _forward_case(moe, orc, T, 128, 96, 3, 2, seed=T, mode=2)


def test_forward_prefill_many_pairs_lds(moe, orc):
    """1400 pairs (the many-workgroup permutation) over E = 20 experts, about
    half of them with more than 64 tokens (two passes), K a multiple of 256
    (the LDS-fed GEMMs)."""
    say("forward prefill T=700 E=20: many-workgroup permutation, LDS-fed GEMMs")
    _forward_case(moe, orc, 700, 256, 256, 20, 2, seed=7, mode=2)


@pytest.mark.parametrize("T,H,I,E,k", [
    (700, 512, 512, 20, 2),     # both GEMMs: K = 512, two blocks (the quad's second half past the end); two passes
    (300, 1536, 1024, 12, 3),   # K = 1536: six blocks, the last quad half full; w2 four blocks
    (20, 1536, 512, 10, 3),     # the small-batch shape
])
def test_forward_prefill_quad_scales(moe, orc, T, H, I, E, k):
    """K a multiple of 512: the LDS-fed GEMMs load the scale bytes of four
    blocks of both tiles in one 16-byte load per wave."""
    say(f"forward prefill quad scales T={T} H={H} I={I} E={E} k={k}")
    _forward_case(moe, orc, T, H, I, E, k, seed=T + H + I, mode=2)


@pytest.mark.parametrize("mode", [1, 2])
def test_forward_accumulate(moe, orc, mode):
    say(f"forward accumulate mode={mode}")
    _forward_case(moe, orc, 4, 256, 128, 8, 2, seed=5, mode=mode, accumulate=True)


@pytest.mark.parametrize("mode", [1, 2])
def test_forward_scale_extremes(moe, orc, mode):
    say(f"forward with scale bytes over the supported range, mode={mode}")
    _forward_case(moe, orc, 3, 128, 64, 4, 2, seed=9, mode=mode, scale_lo=100, scale_hi=140)


@pytest.mark.parametrize("mode", [1, 2])
def test_probes(moe, orc, mode):
    """One-hot weights: pins nibble order, orientation and scale indexing on the GPU."""
    import torch
    H, I = 256, 128
    for n0, c0, code, sc in [(0, 1, 7, 124), (I - 1, H - 1, 13, 120), (37, 64 + 33, 5, 130)]:
        say(f"probe w1 n0={n0} c0={c0} mode={mode}")
        ex = pins.const_expert(H, I, 0, 2, 2)
        pins.set_nibble(ex["w1"], n0, c0, code)
        ex["s1"][n0, c0 // 32] = sc
        x = np.zeros((1, H), np.uint16)
        x[0, c0] = pins.bf16_bits(1.5)
        x[0, c0 ^ 1] = pins.bf16_bits(-0.625)
        lg = np.zeros((1, 1), np.float32)
        ref = orc.forward(H, I, 1, 1, x, lg, {0: ex}, want_h=True,
                          acc=accum.forward_model(1, H, I, 1, 1, mode))
        w = dev_weights({n: a[None] for n, a in ex.items()})
        y, h, _ = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, 1, mode=mode)
        torch.cuda.synchronize()
        check_h(host_bits(h), ref["h"], ref["hpre"], ref["hbound"], "probe w1")
        check_y(y.cpu().numpy(), ref["y"], "probe w1")
    for m0, n0, code, sc in [(0, 0, 7, 124), (H - 1, I - 1, 13, 125), (3, 33, 5, 127)]:
        say(f"probe w2 m0={m0} n0={n0} mode={mode}")
        ex = pins.const_expert(H, I, 2, 2, 0)
        pins.set_nibble(ex["w2"], m0, n0, code)
        ex["s2"][m0, n0 // 32] = sc
        x = np.zeros((1, H), np.uint16)
        x[0, 0] = pins.bf16_bits(1.25)
        lg = np.zeros((1, 1), np.float32)
        ref = orc.forward(H, I, 1, 1, x, lg, {0: ex}, want_h=True)
        w = dev_weights({n: a[None] for n, a in ex.items()})
        y, h, _ = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, 1, mode=mode)
        torch.cuda.synchronize()
        yy = y.cpu().numpy()
        assert np.array_equal(host_bits(h), ref["h"])
        assert np.array_equal(yy, ref["y"]), (np.nonzero(yy)[1], np.nonzero(ref["y"])[1])


def test_decode_and_prefill_agree(moe):
    """Both paths on one input: routing identical, outputs within fp32 reordering."""
    import torch
    rng = np.random.default_rng(77)
    T, H, I, E, k = 12, 512, 256, 20, 4
    dense = {n: np.stack([pins.random_expert(rng, H, I)[n] for _ in range(E)])
             for n in ("w1", "s1", "w3", "s3", "w2", "s2")}
    w = dev_weights(dense)
    x = dev_bits(pins.rand_bf16(rng, (T, H)))
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    y1 = moe.moe_fp4_forward(x, lg, w, k, mode=1)
    y2 = moe.moe_fp4_forward(x, lg, w, k, mode=2)
    torch.cuda.synchronize()
    check_y(y1.cpu().numpy(), y2.cpu().numpy(), "decode vs prefill")


@pytest.mark.parametrize("mode", [1, 2])
def test_forward_repeatable(moe, mode):
    """Same call twice gives bitwise the same y (no atomics-order dependence)."""
    import torch
    rng = np.random.default_rng(8)
    T, H, I, E, k = 8, 256, 128, 16, 2
    dense = {n: np.stack([pins.random_expert(rng, H, I)[n] for _ in range(E)])
             for n in ("w1", "s1", "w3", "s3", "w2", "s2")}
    w = dev_weights(dense)
    x = dev_bits(pins.rand_bf16(rng, (T, H)))
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    a = moe.moe_fp4_forward(x, lg, w, k, mode=mode).cpu().numpy()
    b = moe.moe_fp4_forward(x, lg, w, k, mode=mode).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_expert_blob_layout(moe, orc):
    """Experts stored as one blob each (the six tensors back to back) via strides."""
    import torch
    rng = np.random.default_rng(19)
    T, H, I, E, k = 4, 256, 128, 5, 2
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    sizes = [experts[0][n].size for n in names]
    blob = sum(sizes) + 16 * 6
    offs = []
    o = 0
    for s in sizes:
        offs.append(o)
        o += (s + 15) // 16 * 16
    buf = np.zeros((E, (blob + 255) // 256 * 256), np.uint8)
    for e in range(E):
        for n, off, s in zip(names, offs, sizes):
            buf[e, off:off + s] = experts[e][n].ravel()
    dbuf = torch.from_numpy(buf).cuda()
    stride = buf.shape[1]
    views = {n: dbuf.view(-1)[off:] for n, off in zip(names, offs)}
    w = moe.ExpertWeights(strides=(stride,) * 6, I=I, **views)
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ref = orc.forward(H, I, E, k, x, lg, experts)
    y = moe.moe_fp4_forward(dev_bits(x), torch.from_numpy(lg).cuda(), w, k)
    torch.cuda.synchronize()
    check_y(y.cpu().numpy(), ref["y"], "blob layout")


@pytest.mark.parametrize("shift", [0, 1, 2])
def test_prefill_scale_alignment(moe, orc, shift):
    """H and I multiples of 256: 4-byte aligned scale tensors take the LDS-fed
    GEMMs, scale tensors at an odd or 2 mod 4 offset the register-fed ones.
    Both are checked against the oracle, h included."""
    import torch
    say(f"prefill with scale tensors shifted by {shift} bytes")
    rng = np.random.default_rng(23 + shift)
    T, H, I, E, k = 40, 512, 256, 6, 3
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
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
    w = moe.ExpertWeights(strides=(buf.shape[1],) * 6, I=I, **views)
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True, acc=accum.model("mfma", H))
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k,
                                            mode=moe.MODE_PREFILL)
    torch.cuda.synchronize()
    what = f"prefill scale shift {shift}"
    check_h(host_bits(h), ref["h"], ref["hpre"], ref["hbound"], what)
    check_y(y.cpu().numpy(), ref["y"], what)


def test_prenorm(moe, orc):
    import torch
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((6, 5120)) * 300).astype(np.float32)
    u = moe.moe_fp4_prenorm_bf16(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    got = host_bits(u)
    ref = orc.prenorm(x)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 1e-3 * diff.size


def test_device_generator_matches_host(moe):
    """The device weight generator writes the same bytes as the host generator."""
    import torch
    import synth
    from synth.configs import TINY, DECODE
    dev = synth.layer_device(TINY, layer=2)
    host = synth.layer_host(TINY, layer=2)
    for n in host:
        assert np.array_equal(dev[n].cpu().numpy(), host[n]), n
    dev = synth.layer_device(DECODE, layer=0, n_experts=3)
    torch.cuda.synchronize()
    for e in range(3):
        h = synth.expert_host(DECODE, 0, e)
        for n in h:
            assert np.array_equal(dev[n][e].cpu().numpy(), h[n]), (e, n)


RESIDUAL_CASES = [  # (T, H, I, E, k, mode): one-token path (pre-norm fused), decode MFMA, prefill, MXFP8
    (1, 256, 128, 16, 2, 0),
    (1, 5120, 2304, 8, 6, 0),
    (2, 256, 128, 16, 2, 1),
    (40, 256, 128, 24, 6, 2),
    (40, 256, 128, 24, 6, 3),
]


@pytest.mark.parametrize("T,H,I,E,k,mode", RESIDUAL_CASES)
def test_forward_residual(moe, orc, T, H, I, E, k, mode):
    """x += layer(prenorm(x)) in one call: the same bits as the pre-norm entry
    point followed by an accumulating forward, and the oracle's stack layer."""
    import torch
    say(f"forward_residual T={T} H={H} I={I} E={E} k={k} mode={mode}")
    rng = np.random.default_rng(T * 3 + H + mode)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    dense = {n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]}
    w = dev_weights(dense)
    x0 = (rng.standard_normal((T, H)) * 3.0).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lgd = torch.from_numpy(lg).cuda()
    x1 = torch.from_numpy(x0).cuda()
    moe.moe_fp4_forward_residual(x1, lgd, w, k, mode=mode)
    x2 = torch.from_numpy(x0).cuda()
    u = moe.moe_fp4_prenorm_bf16(x2)
    moe.moe_fp4_forward(u, lgd, w, k, y=x2, mode=mode, accumulate=True)
    torch.cuda.synchronize()
    x1, x2 = x1.cpu().numpy(), x2.cpu().numpy()
    assert np.array_equal(x1.view(np.uint32), x2.view(np.uint32))
    if mode != 3:
        xr = orc.stack_layer(I, E, k, x0, lg, experts)
        check_y(x1.astype(np.float64) - x0, xr.astype(np.float64) - x0, f"residual mode={mode}")


@pytest.mark.parametrize("T,mode", [(1, 1), (2, 1), (2, 2), (40, 2)],
                         ids=["one_token", "few_tokens", "prefill_T2", "prefill_T40"])
def test_scale_bytes_0_and_255(moe, orc, T, mode):
    """UE8M0 byte 0 is 2^-127 and 255 is NaN (OCP MX).  Expert 0 carries bytes 0
    in some w1, w3 and w2 groups (products that small leave the output as with
    zero weights there); expert 1 carries a 255 in one w1 group, so every
    token routed to it has NaN in h and in all of y, on both sides."""
    import torch
    H, I, E, k = 256, 128, 2, 1
    rng = np.random.default_rng(255 + T + mode)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    experts[0]["s1"][5, 2] = 0
    experts[0]["s3"][9, 7] = 0
    experts[0]["s2"][7, 1] = 0
    experts[1]["s1"][3, 0] = 255
    x = pins.rand_bf16(rng, (T, H))
    lg = np.zeros((T, E), np.float32)
    lg[np.arange(T), np.arange(T) % 2] = 1.0       # odd tokens take expert 1
    if T == 1:
        lg[0] = [0.0, 1.0]
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True,
                      acc=accum.forward_model(T, H, I, E, k, mode))
    w = dev_weights({n: np.stack([experts[e][n] for e in range(E)]) for n in experts[0]})
    y, h, route = moe.moe_fp4_forward_debug(dev_bits(x), torch.from_numpy(lg).cuda(), w, k, mode=mode)
    torch.cuda.synchronize()
    y, h = y.cpu().numpy(), host_bits(h)
    nan_tok = ref["idx"][:, 0] == 1
    assert np.array_equal(np.isnan(y), np.isnan(ref["y"])), "NaN positions of y"
    assert np.all(np.isnan(y[nan_tok])) and not np.isnan(y[~nan_tok]).any()
    hn = bf16_value(h)
    assert np.array_equal(np.isnan(hn), np.isnan(bf16_value(ref["h"]))), "NaN positions of h"
    ok = ~nan_tok
    if ok.any():
        pairs = np.nonzero(ok)[0]
        check_h(h[pairs], ref["h"][pairs], ref["hpre"][pairs], ref["hbound"][pairs], "scale byte 0")
        check_y(y[ok], ref["y"][ok], "scale byte 0")
