"""Synthetic workloads of one routed-expert FP4 MoE layer.

Each workload fixes shapes, routing skew and seeds.  Shapes follow the
DeepSeek-V4.1-Flash expert layout on the 10100.com page (section on the
expert-capacity bottleneck): w1/w3 are [I, H/2] nibble bytes plus [I, H/32]
scale bytes, w2 is [H, I/2] plus [H, I/32], with H = 5120, I = 2304, 384
routed experts per layer and 6 active per token.  The pruned stack keeps 36 %
of the experts per layer (same page, section on approach two), 138 of 384.
"""
from __future__ import annotations

from dataclasses import dataclass

# Logit bias strength: bias_e = -ZIPF_ALPHA * s * ln(rank_e).  With alpha = 1
# a Zipf(1.1) bias concentrates 80 % of the top-6 selections on ~3 % of the
# experts; alpha = 0.43 puts 80 % of the selections on ~25 % of them, which is
# the skew the decode workload asks for (checked in tests/test_synth.py).
ZIPF_ALPHA = 0.43

WEIGHT_SEED = 0x5EED_F4E2_0001
INPUT_SEED = 0x5EED_0000_1000


@dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens per step
    H: int              # hidden size (w1/w3 input width, w2 output rows)
    I: int              # intermediate size
    E: int              # routed experts per layer
    k: int              # experts per token
    zipf_s: float = 0.0  # 0 = unbiased N(0,1) logits
    layers: int = 1
    steps: int = 1
    scale_lo: int = 120
    scale_hi: int = 124
    weight_seed: int = WEIGHT_SEED
    input_seed: int = INPUT_SEED

    @property
    def pairs(self) -> int:
        return self.T * self.k


TINY = Workload("tiny", T=8, H=256, I=128, E=16, k=2, input_seed=INPUT_SEED + 1)
DECODE = Workload("decode", T=1, H=5120, I=2304, E=384, k=6, zipf_s=1.1, steps=256,
                  input_seed=INPUT_SEED + 2)
VERIFY6 = Workload("verify6", T=6, H=5120, I=2304, E=384, k=6, zipf_s=1.1, steps=256,
                   input_seed=INPUT_SEED + 3)
VERIFY32 = Workload("verify32", T=32, H=5120, I=2304, E=384, k=6, zipf_s=1.1, steps=256,
                    input_seed=INPUT_SEED + 4)
PREFILL = Workload("prefill", T=2048, H=5120, I=2304, E=384, k=6, zipf_s=0.3,
                   input_seed=INPUT_SEED + 5)
STACK1 = Workload("stack1", T=1, H=5120, I=2304, E=138, k=6, zipf_s=1.1, layers=40, steps=64,
                  weight_seed=WEIGHT_SEED + 7, input_seed=INPUT_SEED + 6)
STACK6 = Workload("stack6", T=6, H=5120, I=2304, E=138, k=6, zipf_s=1.1, layers=40, steps=64,
                  weight_seed=WEIGHT_SEED + 7, input_seed=INPUT_SEED + 7)

# One GPU's share of the layer when eight GPUs hold it.  Decode in tensor
# parallel: the routing is replicated and each GPU holds 288 of the 2304
# intermediate rows of every expert (w1/w3 [288, 2560 B] + [288, 160], w2
# [5120, 144 B] + [5120, 9]); its y is a partial sum that an all-reduce
# completes.  The inputs are the decode workload's.  Prefill in expert
# parallel: each GPU holds 48 of the 384 experts and receives the pairs routed
# to them, about 1,536 of the chunk's 12,288 (32 an expert); here 256 tokens
# routed top-6 over 48 experts give the same pairs per expert.
DECODE_TP8 = Workload("decode_tp8", T=1, H=5120, I=288, E=384, k=6, zipf_s=1.1, steps=256,
                      weight_seed=WEIGHT_SEED + 9, input_seed=INPUT_SEED + 2)
PREFILL_EP8 = Workload("prefill_ep8", T=256, H=5120, I=2304, E=48, k=6, zipf_s=0.3,
                       input_seed=INPUT_SEED + 8)

ALL = {w.name: w for w in (TINY, DECODE, VERIFY6, VERIFY32, PREFILL, STACK1, STACK6)}
