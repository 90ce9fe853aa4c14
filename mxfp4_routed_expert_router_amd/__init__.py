"""MI355X-native routed-expert FP4 MoE layer (DeepSeek-V4.1-Flash style).

The layer -- top-k router, by-expert token permutation, SwiGLU experts whose
w1/w3/w2 are FP4 E2M1 codes with UE8M0 scales per 32 inputs, gate-weighted
combine -- runs entirely in the HIP kernels of libmoe_fp4.so (gfx950).  This
package is its thin Python binding; see include/moe_fp4.h for the C-ABI.
"""
from ._lib import (ACCUMULATE, MODE_AUTO, MODE_DECODE, MODE_PREFILL,  # noqa: F401
                   MODE_PREFILL_MXFP8, ExpertWeights, MoeFp4Error, Route, StageEvents,
                   moe_fp4_forward, moe_fp4_forward_debug, moe_fp4_forward_profiled,
                   moe_fp4_prenorm_bf16, moe_fp4_quant_mxfp8, moe_fp4_route,
                   moe_fp4_router_logits, moe_fp4_forward_routed, moe_fp4_forward_saliency,
                   SharedWeights, moe_fp4_shared_expert, moe_fp4_forward_shared,
                   moe_fp4_forward_residual, moe_fp4_forward_noalloc, moe_fp4_plan, moe_fp4_route_workspace_size,
                   PATH_DECODE_ONE, PATH_DECODE_FEW, PATH_DECODE_MFMA, PATH_PREFILL,
                   PATH_PREFILL_MXFP8, moe_fp4_workspace_size, status_string)
