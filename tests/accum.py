"""How far a kernel's fp32 evaluation of G and U may stray from the exact sums,
for the h checks of the GPU parity tests.

A kernel sums the exact products x_c * w_c (bf16 times a decoded FP4 or FP8
weight: exact in fp32) through a fixed structure of instructions: v_dot2c
chains per lane and a DPP tree, or chains of matrix-core instructions.  Each
instruction returns the sum of its terms (the accumulator input included)
within EPS times the sum of their absolute values; tests/test_gpu_accum.py
measures that on the GPU for each instruction.

From those per-instruction bounds each kernel family gets an accumulation
model, the (sum, prefix, block) triple the oracle takes (oracle_acc in
oracle/oracle.c): the evaluation of a row's sum S is within
    sum * A + prefix * P
of S, A = sum |p_c|, P = the magnitudes of the exact partial sums at every
`block` inputs (natural order).

  gemv        one-token and few-token decode: lane l chains the v_dot2c of its
              32-input groups l, l + 64, ... (16 per group: four per 8-input
              chunk, four chunks), then a 6-add DPP tree.  Worst case of that
              depth, D = 16 ceil(K / 2048) EPS_DOT2 + 6:  sum = D u / (1 - D u).
  gemv_mfma   small-shape decode (gemv13_kernel): wave w chains 4 MFMAs per
              128-input block over its ceil(ceil(K / 128) / 8) blocks, then the
              8 wave partials are added in order: worst case of that depth.
  mfma        prefill with bf16 activations (LDS-fed and register-fed): one
              accumulator takes K in ascending 128-input blocks, each through
              4 MFMAs.  Before an instruction of block j the accumulator is
              within the block's absolute sum of the exact prefix P_j, so with
              e = EPS / (1 - N EPS u), N = K / 32 instructions:
              error <= e u (4 sum_j |P_j| + 5 A).
  mx8         MXFP8 prefill: as mfma with one scaled MFMA per 128-input block:
              error <= e u (sum_j |P_j| + 2 A).
  shared_gemv shared expert, T <= 4: lane chains of 8 v_dot2c per 16-code
              chunk over ceil(K / 1024) chunks, then the DPP tree.
  shared_mfma shared expert, T > 4: 64-input blocks, 2 MFMAs each.
"""
from __future__ import annotations

import math

U = 2.0 ** -24

# Per-instruction bounds, in units of u, relative to the sum of the absolute
# values of the instruction's terms: twice the largest error the probes of
# tests/test_gpu_accum.py measured on MI355X (2.19 u, 3.81 u, 4533 u).
EPS_ADD = 1.0                  # one fp32 add, round to nearest
EPS_DOT2 = 4.5                 # v_dot2c_f32_bf16
EPS_MFMA_BF16 = 8.0            # v_mfma_f32_16x16x32_bf16
EPS_MFMA_SCALE = 9100.0        # v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 x E4M3

FAMILIES = ("gemv", "gemv_mfma", "mfma", "mx8", "shared_gemv", "shared_mfma")


def _worst(D: float):
    d = D * U
    return (d / (1.0 - d), 0.0, 0)


def _blocked(eps: float, n_inst: int, m: int, block: int):
    e = eps * U / (1.0 - n_inst * eps * U)
    return ((m + 1) * e, m * e, block)


def model(family: str, K: int):
    """The oracle's accumulation model (sum, prefix, block) of a family for rows
    of K inputs."""
    if family == "gemv":
        return _worst(16 * math.ceil(K / 2048) * EPS_DOT2 + 6 * EPS_ADD)
    if family == "gemv_mfma":
        return _worst(4 * math.ceil(math.ceil(K / 128) / 8) * EPS_MFMA_BF16 + 8 * EPS_ADD)
    if family == "mfma":
        return _blocked(EPS_MFMA_BF16, math.ceil(K / 32), 4, 128)
    if family == "mx8":
        return _blocked(EPS_MFMA_SCALE, math.ceil(K / 128), 1, 128)
    if family == "shared_gemv":
        return _worst(8 * math.ceil(K / 1024) * EPS_DOT2 + 6 * EPS_ADD)
    if family == "shared_mfma":
        return _blocked(EPS_MFMA_BF16, math.ceil(K / 32), 2, 64)
    raise ValueError(family)


def family_of_path(path: int) -> str:
    """Family of a forward call's kernel path (moe_fp4_plan)."""
    import mxfp4_routed_expert_router_amd as moe
    return {moe.PATH_DECODE_ONE: "gemv", moe.PATH_DECODE_FEW: "gemv",
            moe.PATH_DECODE_MFMA: "gemv_mfma", moe.PATH_PREFILL: "mfma",
            moe.PATH_PREFILL_MXFP8: "mx8"}[path]


def forward_model(T: int, H: int, I: int, E: int, k: int, mode: int):
    """Accumulation model of G and U for the kernels a forward call takes."""
    import mxfp4_routed_expert_router_amd as moe
    return model(family_of_path(moe.moe_fp4_plan(T, H, I, E, k, mode)), H)


def shared_model(T: int, H: int):
    """Accumulation model of the shared expert's G and U (T <= 4: one wave per
    row; more tokens: MFMA tiles)."""
    return model("shared_gemv" if T <= 4 else "shared_mfma", H)
