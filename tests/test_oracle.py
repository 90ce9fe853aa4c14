"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_layout_closed_forms():
    """Byte shapes and totals printed on the pages, recomputed from the layout rule
    (two E2M1 codes per byte, one UE8M0 byte per 32 inputs)."""
    import synth
    g = pins.read_golden("expert_layout.txt")
    H, I = int(g["hidden"][0]), int(g["w1_weight"][0])
    shapes = synth.tensor_shapes(H, I)
    for name, key in (("w1", "w1_weight"), ("s1", "w1_scale"), ("w3", "w3_weight"),
                      ("s3", "w3_scale"), ("w2", "w2_weight"), ("s2", "w2_scale")):
        assert list(shapes[name]) == [int(v) for v in g[key]], name
    per = sum(r * c for r, c in shapes.values())
    assert per == int(g["bytes_per_expert"][0]) == 18_800_640
    n = int(g["layers"][0]) * int(g["experts_per_layer"][0])
    assert n == int(g["total_experts"][0])
    assert round(per * n / 1e9, 1) == g["total_GB"][0]
    scales = sum(r * c for k, (r, c) in shapes.items() if k.startswith("s"))
    assert round(scales / 1e6, 1) == g["scale_MB"][0]
    assert round((per - scales) / 1e6, 1) == g["weight_MB"][0]
    layer = per * int(g["experts_per_layer"][0])
    assert layer == 7_219_445_760 and abs(layer / 2**30 - g["layer_GB"][0]) < 0.1
    kept = int(g["pruned_keep_min"][0] * int(g["experts_per_layer"][0]))
    assert kept == 138 and kept * per * int(g["layers"][0]) == 103_779_532_800


@pytest.mark.slow
def test_probes_real_shape(orc):
    """One-hot probes at H=5120, I=2304, including the last row and column."""
    H, I = 5120, 2304
    pins.pin_probe_w1(orc, H, I, cases=[(I - 1, H - 1, 7, 124), (1000, 4097, 11, 122)])
    pins.pin_probe_w2(orc, H, I, cases=[(H - 1, I - 1, 6, 123), (2500, 1311, 9, 127)])


def test_gate_invariants_large(orc):
    """sum_j g = 1 and gates non-increasing along rank on a 2048 x 384 logit block."""
    import synth
    from synth.configs import PREFILL
    lg = synth.gen_logits(PREFILL)
    idx, g = orc.route(lg, 6)
    assert np.max(np.abs(g.astype(np.float64).sum(1) - 1)) < 1e-6
    assert np.all(np.diff(g, axis=1) <= 0)
    counts, offsets, sp, slot = orc.permute(idx, 384)
    assert counts.sum() == 2048 * 6


@pytest.mark.parametrize("T,H,I,E,k", [(50, 256, 128, 8, 2), (9, 384, 256, 7, 3)])
def test_mx8_w2_reference_matches_oracle(orc, T, H, I, E, k):
    """The GPU tests' reference for the MXFP8 w2 stage (numpy: the oracle's
    quantiser on a given h, exact FP4 and E4M3 values, float64 products) gives
    the oracle's own MXFP8 y when handed the oracle's h: two implementations of
    the same stage agree to the rounding of y to float32."""
    from gpu_common import mx8_w2_on_h
    rng = np.random.default_rng(T + H + I)
    experts = {e: pins.random_expert(rng, H, I) for e in range(E)}
    x = pins.rand_bf16(rng, (T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ref = orc.forward(H, I, E, k, x, lg, experts, want_h=True, mx8=True)
    y = mx8_w2_on_h(orc, experts, ref["idx"], ref["gates"], ref["h"], H, I)
    yo = ref["y"].astype(np.float64)
    assert np.max(np.abs(y - yo)) <= 1e-6 * np.sqrt(np.mean(yo ** 2))
    # and it is not the bf16 path's w2 stage: quantising h moves y
    yb = orc.forward(H, I, E, k, x, lg, experts)["y"].astype(np.float64)
    assert np.linalg.norm(y - yb) > 1e-3 * np.linalg.norm(yb)
