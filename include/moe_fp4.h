/*
 * moe_fp4 -- one routed-expert FP4 mixture-of-experts layer on MI355X (gfx950).
 *
 * The layer is the DeepSeek-V4.1-Flash routed-expert block as the 10100.com
 * page describes it (section on the MoE expert-capacity bottleneck): each token
 * picks k of E routed experts (6 of 384 in the model), and each picked expert is
 * an FFN with three matrices w1, w3 (I x H) and w2 (H x I) stored as FP4 E2M1
 * codes, two per byte, with one UE8M0 scale byte per 32 consecutive inputs of a
 * row: w1/w3 [2304, 2560 B] + [2304, 160], w2 [5120, 1152 B] + [5120, 72],
 * 18,800,640 bytes per expert.  The ai-shiz.ru page (section on the model) gives
 * hidden 5120 and the 6-of-384 routing.
 *
 * Computation (readings of what the pages leave open):
 *   route    idx[t][0..k) = the k largest logits of token t, larger first, ties to
 *            the lower expert index, -0 equal to +0, NaN below every number;
 *            gates[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k chosen.
 *   expert   G = W1 x, U = W3 x, h = bf16_rne(silu(G) * U), Y = W2 h, with
 *            W[r][c] = E2M1(nibble) * 2^(scale - 127), the low nibble of a byte
 *            holding the even input.
 *   combine  y[t] = sum_j gates[t][j] * Y_(t, idx[t][j]), j ascending, fp32.
 * Products of bf16 activations and decoded weights are exact in fp32 and are
 * summed in fp32 (MFMA or v_dot2c_f32_bf16); h is rounded to bf16 once, after
 * silu(G)*U.
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no state between calls.
 *   - A call validates its arguments on the host before any HIP call, enqueues
 *     its kernels on `stream` and returns without synchronising.  Faults in the
 *     kernels surface at the caller's next synchronisation.
 *   - Inputs are read-only.  Calls that share a workspace must not overlap.
 *   - Return value: MOE_FP4_OK or one of the error codes below; nothing is
 *     enqueued when a call returns an error found during validation.
 *   - No C++ exception crosses this boundary.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes */
#define MOE_FP4_OK            0
#define MOE_FP4_EINVAL        1  /* null pointer, non-positive or inconsistent size */
#define MOE_FP4_EUNSUPPORTED  2  /* sizes outside the supported range (see below)  */
#define MOE_FP4_EALIGN        3  /* a pointer or stride breaks its alignment rule   */
#define MOE_FP4_EWORKSPACE    4  /* workspace missing or smaller than required      */
#define MOE_FP4_EHIP          5  /* a kernel launch failed (hipGetLastError)        */

/* ---- forward modes */
#define MOE_FP4_MODE_AUTO     0  /* DECODE up to 8 tokens where it supports the    */
                                 /* dims, else PREFILL                            */
#define MOE_FP4_MODE_DECODE   1  /* GEMV path for a few tokens (see below)           */
#define MOE_FP4_MODE_PREFILL  2  /* grouped-GEMM path; any T                         */
#define MOE_FP4_MODE_PREFILL_MXFP8 3  /* grouped GEMM on FP4 x FP8 scaled MFMA (below)  */
/* MOE_FP4_MODE_PREFILL_MXFP8 computes the layer with the activations in the OCP
 * MX FP8 format: x is quantised to MXFP8 along H before w1/w3 and the bf16 h
 * along I before w2 (see moe_fp4_quant_mxfp8); the matrix cores then take the
 * FP4 weights and their UE8M0 scales as stored.  Routing, the SwiGLU epilogue
 * (h rounded to bf16 first) and the combine are as in PREFILL.  Requires H and
 * I to be multiples of 128, and the scale tensors s1, s3, s2 to have 4-byte
 * aligned bases and expert strides (MOE_FP4_EALIGN otherwise).  Its results
 * differ from PREFILL by the FP8 quantisation of the activations (about 5e-2
 * relative), not by rounding. */
/* DECODE takes one token on a dedicated path (H <= 8192 and k * I / 32 <=
 * 1024); 2 <= T <= 15 on the same GEMV design with the T activation rows staged
 * in LDS, as far as they fit 160 KiB (T * (H / 32 + 1) * 64 bytes, plus
 * 8 * T * k; at H = 5120 that is T <= 15); and other shapes with T <= 16 on
 * MFMA kernels as far as the T activation rows and the T*k h rows they stage
 * in LDS fit 64 KiB each and I <= 3072.
 * moe_fp4_workspace_size(dims, MOE_FP4_MODE_DECODE, ...) returns
 * MOE_FP4_EUNSUPPORTED outside that range. */

/* ---- forward flags */
#define MOE_FP4_ACCUMULATE    1  /* y += layer output (default: y = layer output)    */

/* Supported range: 1 <= T <= 65535, 1 <= E <= 1024, 1 <= k <= min(E, 16),
 * H and I multiples of 32 with 32 <= H, I <= 16384. */
typedef struct {
  int32_t T;  /* tokens in the call                  */
  int32_t H;  /* hidden size (input of w1/w3)        */
  int32_t I;  /* intermediate size (input of w2)     */
  int32_t E;  /* routed experts in the weight tensors */
  int32_t k;  /* experts per token                   */
} moe_fp4_dims;

/* Expert weights in the checkpoint layout, all uint8:
 *   w1, w3  per expert [I][H/2] E2M1 code pairs (low nibble = even input column)
 *   s1, s3  per expert [I][H/32] UE8M0 scales (scale g covers inputs 32g..32g+31)
 *   w2      per expert [H][I/2]
 *   s2      per expert [H][I/32]
 * expert_stride[i] is the byte distance between consecutive experts of tensor
 * i (order w1, s1, w3, s3, w2, s2); 0 means dense stacking (the per-expert size).
 * Nibble tensors (w1, w3, w2) need 16-byte aligned bases and strides; scale
 * tensors have no alignment rule except in MOE_FP4_MODE_PREFILL_MXFP8 (4
 * bytes).  Supported scale bytes are 2..252. */
typedef struct {
  const uint8_t *w1, *s1, *w3, *s3, *w2, *s2;
  int64_t expert_stride[6];
} moe_fp4_weights;

/* Routing result, all device arrays written by moe_fp4_route:
 *   topk_idx      [T][k] expert ids in rank order
 *   gates         [T][k] fp32 gates in rank order
 *   counts        [E]    pairs routed to each expert
 *   offsets       [E+1]  exclusive prefix sum of counts (offsets[E] = T*k)
 *   sorted_pairs  [T*k]  pair ids p = t*k + j grouped by expert (ascending expert),
 *                        ascending p within an expert
 *   pair_slot     [T*k]  inverse permutation: sorted_pairs[pair_slot[p]] == p */
typedef struct {
  int32_t *topk_idx;
  float *gates;
  int32_t *counts;
  int32_t *offsets;
  int32_t *sorted_pairs;
  int32_t *pair_slot;
} moe_fp4_route_out;

/* Bytes of workspace moe_fp4_forward needs for these dims and mode.
 * Errors: EINVAL (null), EUNSUPPORTED (dims out of range or mode unknown). */
int moe_fp4_workspace_size(const moe_fp4_dims *dims, int mode, size_t *bytes);

/* ---- kernel paths (moe_fp4_plan) */
#define MOE_FP4_PATH_DECODE_ONE     1  /* one token: GEMV kernels, routing in the first  */
#define MOE_FP4_PATH_DECODE_FEW     2  /* 2..15 tokens: the same GEMV design, x in LDS   */
#define MOE_FP4_PATH_DECODE_MFMA    3  /* other small shapes: MFMA GEMV kernels          */
#define MOE_FP4_PATH_PREFILL        4  /* grouped GEMMs, bf16 activations                */
#define MOE_FP4_PATH_PREFILL_MXFP8  5  /* grouped GEMMs, MXFP8 activations               */

/* Which kernels moe_fp4_forward takes for these dims and mode (for profiling
 * and for checks that depend on the kernels' accumulation order): *path is one
 * of MOE_FP4_PATH_*.  Host only, enqueues nothing.
 * Errors: EINVAL (null), EUNSUPPORTED (as moe_fp4_workspace_size). */
int moe_fp4_plan(const moe_fp4_dims *dims, int mode, int *path);

/* Bytes of workspace moe_fp4_route needs: 0 up to 64 tokens and 1024 pairs
 * (one workgroup ranks and permutes them), else the per-workgroup expert
 * counts and per-slot records of the permutation spread over many workgroups.
 * dims->H and dims->I are not used.
 * Errors: EINVAL (null or a non-positive size), EUNSUPPORTED (T > 65535,
 * E > 1024, k > 16). */
int moe_fp4_route_workspace_size(const moe_fp4_dims *dims, size_t *bytes);

/* Router and token permutation (top-k + softmax over the chosen logits, then a
 * histogram, scan and stable scatter of the T*k pairs grouped by expert).
 *   logits  [T][E] fp32, row-major, 4-byte aligned.
 *   ws      device workspace of at least moe_fp4_route_workspace_size bytes,
 *           256-byte aligned (may be NULL when that size is 0); its contents
 *           need no initialisation.
 * Results are bit-exact functions of the logits (no atomics-order dependence).
 * Errors: EINVAL (a null pointer), EUNSUPPORTED (dims), EALIGN, EWORKSPACE,
 * EHIP. */
int moe_fp4_route(const moe_fp4_dims *dims, const float *logits, moe_fp4_route_out *out,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer: route, experts, combine.
 *   x       [T][H] bf16 bit patterns, 16-byte aligned
 *   logits  [T][E] fp32
 *   w       expert weights (see moe_fp4_weights)
 *   y       [T][H] fp32, 16-byte aligned; overwritten, or added to with
 *           MOE_FP4_ACCUMULATE
 *   ws      device workspace of at least moe_fp4_workspace_size(dims, mode)
 *           bytes, 256-byte aligned; its contents need no initialisation
 * Errors: EINVAL, EUNSUPPORTED (dims, unknown mode or flag, DECODE outside its range),
 * EALIGN, EWORKSPACE, EHIP. */
int moe_fp4_forward(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                    const moe_fp4_weights *w, float *y, int mode, int flags, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* As moe_fp4_forward, with no workspace argument and no allocation: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc).  The workspace is a static
 * device array of MOE_FP4_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends; its address is looked up on the first
 * call on each device (hipGetSymbolAddress), and no call allocates or frees
 * anything.  Every call on a GPU uses that GPU's array: calls that overlap on
 * one GPU (other streams, other host threads) race and must not be made.
 * Nothing in it needs clearing between calls.
 * Errors: as moe_fp4_forward; EWORKSPACE when the call needs more workspace
 * than the array holds (moe_fp4_workspace_size(dims, mode) >
 * MOE_FP4_NOALLOC_SCRATCH_BYTES: one decode token needs about 30 KB, a
 * 2048-token prefill chunk about 311 MB), found before any HIP call. */
#define MOE_FP4_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_fp4_forward_noalloc(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                            const moe_fp4_weights *w, float *y, int mode, int flags,
                            hipStream_t stream);

/* As moe_fp4_forward, and also writes the intermediates:
 *   h_out      [T*k][I] bf16 bits in pair order (row p = t*k + j), or NULL
 *   route_out  routing result as moe_fp4_route writes it, or NULL */
int moe_fp4_forward_debug(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                          const moe_fp4_weights *w, float *y, int mode, int flags, void *ws,
                          size_t ws_bytes, hipStream_t stream, uint16_t *h_out,
                          moe_fp4_route_out *route_out);

/* As moe_fp4_forward, and times the kernels of each stage on `stream`.
 * Stage s is 0 routing, 1 w1/w3, 2 w2, 3 combine; the dispatch of the stage's
 * first kernel records events[2s] when it starts and the dispatch of its last
 * kernel records events[2s+1] when it ends (hipExtLaunchKernel), so
 * hipEventElapsedTime(events[2s], events[2s+1]) is kernel time without launch
 * gaps.  A stage that has no kernel of its own has both events recorded
 * together: routing for one token in DECODE (it runs inside the w1/w3 kernel)
 * and the combine in DECODE (inside the w2 kernel).
 * `events` holds n_events >= 8 events created by the caller.
 * Errors: as moe_fp4_forward, and EINVAL for null events or n_events < 8. */
int moe_fp4_forward_profiled(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                             const moe_fp4_weights *w, float *y, int mode, int flags, void *ws,
                             size_t ws_bytes, hipStream_t stream, hipEvent_t *events,
                             int n_events);

/* Router logits, the step before routing (the router is one of the layer's
 * resident weights: 10100.com page, section on the expert-capacity
 * bottleneck; its format is not given and is taken as bf16):
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c]
 *   x         [T][H] bf16 bits, 16-byte aligned (dims->T, dims->H)
 *   w_router  [E][H] bf16 bits, row-major, 16-byte aligned (dims->E)
 *   logits    [T][E] fp32, 4-byte aligned
 * dims->I and dims->k are not used.  bf16 products are exact in fp32 and are
 * summed in fp32 in a fixed order: the same inputs give the same bits.
 * Errors: EINVAL (null, sizes < 1), EUNSUPPORTED (T > 65535, E > 1024, H not a
 * multiple of 32 in [32, 16384]), EALIGN, EHIP. */
int moe_fp4_router_logits(const moe_fp4_dims *dims, const uint16_t *x, const uint16_t *w_router,
                          float *logits, hipStream_t stream);

/* As moe_fp4_forward, with the logits computed from x and w_router (as
 * moe_fp4_router_logits does) into the workspace first, in place of a logits
 * argument.  Same workspace size.  w_router [E][H] bf16, 16-byte aligned.
 * Errors: as moe_fp4_forward (EINVAL for a null w_router, EALIGN if misaligned). */
int moe_fp4_forward_routed(const moe_fp4_dims *dims, const uint16_t *x, const uint16_t *w_router,
                           const moe_fp4_weights *w, float *y, int mode, int flags, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* As moe_fp4_forward, and adds each expert's saliency for this call to
 * saliency[e] (fp32 [E], 4-byte aligned; the caller zeroes it once and sums a
 * corpus over calls).  Saliency is the pruning signal of the 10100.com page
 * (section on choosing experts, frequency against saliency): router weight
 * times the L2 norm of the expert's output, summed over tokens; here
 *   saliency[e] += sum over pairs (t, j) routed to e of gates[t][j] * ||Y_(t,j)||_2
 * with Y the expert's w2 output before the gate.  Prefill modes only: AUTO
 * runs PREFILL, DECODE is EUNSUPPORTED; the workspace is that of the mode run.
 * The sums are in a fixed order: the same inputs give the same bits.
 * Errors: as moe_fp4_forward, and EINVAL for a null saliency. */
int moe_fp4_forward_saliency(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                             const moe_fp4_weights *w, float *y, float *saliency, int mode,
                             int flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* The shared expert (one per layer beside the routed experts: ai-shiz.ru
 * page, section "what the model is"; FP8 per the 10100.com page, plan two;
 * 32 x 32 blocks for the main weights per the ai-shiz.ru page).  Taken as a
 * SwiGLU expert of the routed experts' form, E4M3 weights, one UE8M0 scale per
 * 32 x 32 block:
 *   w1, w3  [I][H] E4M3 codes (row n = output n), 16-byte aligned
 *   s1, s3  [I/32][H/32] UE8M0: W1[n][c] = E4M3(w1[n][c]) * 2^(s1[n/32][c/32] - 127)
 *   w2      [H][I] E4M3 codes, 16-byte aligned
 *   s2      [H/32][I/32] UE8M0
 *   I       intermediate size, a multiple of 32 in [32, 16384]
 * Scale tensors have no alignment rule. */
typedef struct {
  const uint8_t *w1, *s1, *w3, *s3, *w2, *s2;
  int32_t I;
} moe_fp4_shared_weights;

/* The shared expert alone:
 *   h[t] = bf16(silu(W1 x[t]) * (W3 x[t]))   (rounded once, as the routed h)
 *   y[t] = W2 h[t], or y[t] += W2 h[t] with MOE_FP4_ACCUMULATE
 *   dims  T and H used (I, E, k ignored)
 *   x     [T][H] bf16 bits, 16-byte aligned;  y [T][H] fp32, 16-byte aligned
 *   h     [T][sw->I] bf16 bits, 16-byte aligned: written (scratch and output)
 * fp32 sums in a fixed order: the same inputs give the same bits.
 * Errors: EINVAL (null), EUNSUPPORTED (sizes, flags), EALIGN, EHIP. */
int moe_fp4_shared_expert(const moe_fp4_dims *dims, const uint16_t *x,
                          const moe_fp4_shared_weights *sw, float *y, int flags, uint16_t *h,
                          hipStream_t stream);

/* As moe_fp4_forward, then adds the shared expert's output:
 *   y[t] (+)= sum_j gates[t][j] * Y_(t,j) + W2s h_s[t]
 * The shared expert's h uses the routed path's workspace, so sw->I <=
 * dims->k * dims->I is required (EUNSUPPORTED otherwise); same workspace size
 * as moe_fp4_forward.  For one token in MOE_FP4_MODE_DECODE (the one-token
 * kernels) with sw->I <= dims->H, the shared w1/w3 rows run in the routed
 * w1/w3 launch and the shared w2 rows in the routed w2 launch (the shared
 * expert's own kernels after the layer where its rows do not fit them), and
 * the shared h sits in the workspace's pre-norm section.  y is in every case
 * the same, bit for bit, as moe_fp4_forward followed by moe_fp4_shared_expert.
 * Errors: as moe_fp4_forward and moe_fp4_shared_expert. */
int moe_fp4_forward_shared(const moe_fp4_dims *dims, const uint16_t *x, const float *logits,
                           const moe_fp4_weights *w, const moe_fp4_shared_weights *sw, float *y,
                           int mode, int flags, void *ws, size_t ws_bytes, hipStream_t stream);

/* One layer of a residual stack, in place (the pre-norm of moe_fp4_prenorm_bf16
 * with eps = 1e-6, then the layer, its output added to the residual stream):
 *   x[t] += layer( bf16(x[t] / sqrt(mean_m x[t][m]^2 + 1e-6)) )
 *   x       [T][H] fp32, 16-byte aligned, read and updated
 *   logits, w, mode, ws, ws_bytes: as moe_fp4_forward (same workspace size)
 * Same bits as moe_fp4_prenorm_bf16 into a bf16 buffer followed by
 * moe_fp4_forward(..., y = x, MOE_FP4_ACCUMULATE).  On the one-token decode
 * path the pre-norm runs inside the first expert kernel (no launch of its own).
 * Errors: as moe_fp4_forward. */
int moe_fp4_forward_residual(const moe_fp4_dims *dims, float *x, const float *logits,
                             const moe_fp4_weights *w, int mode, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* Pre-normalisation for a residual stack of layers:
 *   u[t][m] = bf16_rne(x[t][m] / sqrt(mean_m x[t][m]^2 + eps))
 *   x [T][H] fp32, u [T][H] bf16 bits, both 16-byte aligned.
 * The sum of squares runs in one fixed order (reproducible bit for bit), the
 * order the fused pre-norm of moe_fp4_forward_residual uses.
 * Errors: EINVAL, EUNSUPPORTED (H not a multiple of 32 or above 16384), EALIGN,
 * EHIP. */
int moe_fp4_prenorm_bf16(const float *x, uint16_t *u, int32_t T, int32_t H, float eps,
                         hipStream_t stream);

/* MXFP8 quantisation (OCP MX, blocks of 32 consecutive values of a row):
 *   src     [rows][K] bf16 bits, 16-byte aligned, K a multiple of 32
 *   codes   [rows][K] E4M3 codes, 8-byte aligned
 *   scales  [rows][K/32] UE8M0 bytes
 * Per block: byte = floor(log2(max |v|)) - 8 + 127, clamped to [0, 254] (0 for a
 * block of zeros); code = E4M3(v / 2^(byte - 127)) rounded to nearest, ties to
 * even, saturated to +-448, sign kept for zero.  This is the quantiser of
 * MOE_FP4_MODE_PREFILL_MXFP8.
 * Errors: EINVAL (null, sizes < 1), EUNSUPPORTED (K % 32), EALIGN, EHIP. */
int moe_fp4_quant_mxfp8(const uint16_t *src, int32_t rows, int32_t K, uint8_t *codes,
                        uint8_t *scales, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *moe_fp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
