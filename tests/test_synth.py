"""Seeded input generators (no GPU)."""
import numpy as np

import synth
from synth.configs import DECODE, PREFILL, TINY, STACK1

M64 = 2**64 - 1


def _py_sm64(state, i):
    z = (state + (i + 1) * 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix64_published_outputs():
    # first outputs of SplitMix64 seeded with 0 (Vigna's reference splitmix64.c)
    assert synth.sm64_at(0, 0) == 0xE220A8397B1DCDAF
    assert synth.sm64_at(0, 1) == 0x6E789E6AA1B965F4
    for s, i in ((1, 0), (0xDEADBEEF, 12345), (M64, 7)):
        assert synth.sm64_at(s, i) == _py_sm64(s, i)


def test_expert_bytes_match_python_stream():
    ex = synth.expert_host(TINY, layer=3, expert=5)
    st = synth.stream(TINY.weight_seed, 3, 5, synth.W1)
    flat = ex["w1"].ravel()
    for o in (0, 1, 7, 8, 1000, flat.size - 1):
        assert flat[o] == (_py_sm64(st, o >> 3) >> (8 * (o & 7))) & 0xFF
    st = synth.stream(TINY.weight_seed, 3, 5, synth.S2)
    flat = ex["s2"].ravel()
    for o in (0, 3, flat.size - 1):
        assert flat[o] == 120 + (((_py_sm64(st, o) >> 32) * 5) >> 32)


def test_weight_distributions():
    ex = synth.expert_host(DECODE, 0, 17)
    for n in ("w1", "w3", "w2"):
        nib = np.concatenate([ex[n].ravel() & 15, ex[n].ravel() >> 4])
        c = np.bincount(nib, minlength=16) / nib.size
        assert np.all(np.abs(c - 1 / 16) < 2e-3), n
    for n in ("s1", "s3", "s2"):
        v = ex[n].ravel()
        assert v.min() == 120 and v.max() == 124
        assert np.all(np.abs(np.bincount(v - 120) / v.size - 0.2) < 1e-2)
    assert synth.expert_host(DECODE, 0, 17)["w2"].tobytes() == ex["w2"].tobytes()
    assert synth.expert_host(DECODE, 0, 18)["w2"].tobytes() != ex["w2"].tobytes()


def test_x_is_bf16_normal():
    x = synth.bf16_bits_to_f32(synth.gen_x(PREFILL))
    assert x.shape == (2048, 5120)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert np.array_equal(synth.gen_x(PREFILL, step=1), synth.gen_x(PREFILL, step=1))
    assert not np.array_equal(synth.gen_x(PREFILL, step=1), synth.gen_x(PREFILL, step=2))


def _top6(lg):
    return np.argsort(-lg, axis=1, kind="stable")[:, :6]


def test_decode_skew_statistic():
    """Zipf(1.1) bias: about a quarter of the experts take 80 % of the selections."""
    lg = np.concatenate([synth.gen_logits(DECODE, step=s) for s in range(4000)])
    c = np.sort(np.bincount(_top6(lg).ravel(), minlength=384))[::-1]
    n80 = int(np.searchsorted(np.cumsum(c) / c.sum(), 0.8)) + 1
    assert 0.20 * 384 <= n80 <= 0.30 * 384, n80


def test_prefill_touches_nearly_all_experts():
    idx = _top6(synth.gen_logits(PREFILL))
    assert len(np.unique(idx)) >= 370


def test_stack_layers_have_own_bias():
    assert not np.array_equal(synth.logit_bias(STACK1, 0), synth.logit_bias(STACK1, 1))
    assert synth.gen_logits(STACK1, 0, 5).shape == (1, 138)
