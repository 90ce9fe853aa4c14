// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

constexpr int kMaxExperts = 1024;      // router / permutation LDS tables
constexpr int kMaxK = 16;
constexpr int kFewRouteTokens = 64;    // one-launch route (route_few_kernel) up to these
constexpr int kFewRoutePairs = 1024;
constexpr int kDecodeMaxTokens = 16;   // decode GEMV: one 16-token MFMA tile per expert
constexpr size_t kDecodeLds = 65536;   // LDS budget of each decode kernel (x / h rows staged whole)

// Optional kernel timing.  `ev` holds 2 events per stage (0 route, 1 w1/w3,
// 2 w2, 3 combine): the dispatch of the stage's first kernel records ev[2s]
// when it starts and that of its last kernel ev[2s+1] when it ends, so the
// elapsed time is kernel time only.  A stage without a kernel of its own has
// both events recorded together.
constexpr int kStages = 4;
inline hipEvent_t ev_start(const hipEvent_t* ev, int stage) { return ev ? ev[2 * stage] : nullptr; }
inline hipEvent_t ev_stop(const hipEvent_t* ev, int stage) { return ev ? ev[2 * stage + 1] : nullptr; }
inline void ev_empty(const hipEvent_t* ev, int stage, hipStream_t s) {
  if (ev) {
    (void)hipEventRecord(ev[2 * stage], s);
    (void)hipEventRecord(ev[2 * stage + 1], s);
  }
}
template <typename K, typename... Args>
inline void launch_k(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t start,
                     hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

struct RouteArgs {
  const float* logits;
  int T, E, k;
  int32_t *idx, *counts, *offsets, *sorted_pairs, *pair_slot, *dinfo, *meta;  // dinfo: per distinct expert {id, first sorted slot, pairs, 0}
  float* gates;
  // optional (forward path): per sorted slot, the pair's gate and token
  float* slot_gate;
  int32_t* slot_tok;
  const hipEvent_t* ev;  // optional stage timing (see ev_start)
  // optional [kPermBlocksMax][E] scratch: with it (and dinfo, slot_gate) large
  // batches are permuted by many workgroups instead of one
  int32_t* perm_scratch;
};

constexpr int kPermBlocksMax = 256;  // workgroups of the multi-block permutation
int perm_pairs_per_block(int P);     // pairs each of them owns (a multiple of 256)

// One matrix product of the shared expert (FP8 E4M3 codes, one UE8M0 scale per
// 32 x 32 block): M = 2 takes w[0], w[1] (w1, w3) into h with the SwiGLU
// epilogue, M = 1 takes w[0] (w2) into y.
struct SharedArgs {
  const uint16_t* act;   // M = 2: x [T][K]; M = 1: h [T][K] (bf16 bits)
  const uint8_t *w[2], *s[2];
  int N, K, T;           // output rows, inputs per row, tokens
  uint16_t* h;           // M = 2 output [T][N]
  float* y;              // M = 1 output [T][N]
  int accumulate;
};

// Weights and routing state shared by the expert kernels.
struct LayerArgs {
  int T, H, I, E, k;
  const uint16_t* x;
  const uint8_t *w1, *s1, *w3, *s3, *w2, *s2;
  int64_t stride[6];  // resolved byte strides between experts
  const int32_t *counts, *offsets, *sorted_pairs, *pair_slot, *dinfo, *meta;  // dinfo: per distinct expert {id, first sorted slot, pairs, 0}
  const float* gates;
  const float* slot_gate;   // [T*k] gate of the pair in each sorted slot
  const int32_t* slot_tok;  // [T*k] token of the pair in each sorted slot
  uint16_t* h;   // [T*k][I] bf16, rows in sorted (by-expert) order
  float* ypair;  // [T*k][H] fp32 gate-scaled expert outputs, sorted order (prefill only)
  // optional saliency side output (prefill only): per sorted slot and 256-row
  // tile of w2, the sum of squares of the expert's output rows, [T*k][sal_tiles]
  float* sal_part;
  int sal_tiles;
  // MXFP8 prefill: E4M3 codes and UE8M0 scales (one per 32 along the row) of x
  // [T][H] and of h [T*k][I] (sorted order)
  uint8_t *xq, *xqs, *hq, *hqs;
  float* y;      // [T][H]
  int accumulate;
  const hipEvent_t* ev;  // optional stage timing (see ev_start)
  // one-token decode: the first expert kernel ranks the logits itself and
  // publishes the routing result (no separate routing launch)
  int fused_route;
  RouteArgs route;
  const float* logits;
  // one-token decode with the pre-norm inside the w1/w3 kernel: x is then
  // unused and the layer's input is bf16(xf / sqrt(mean(xf^2) + eps))
  const float* xf;
  float eps;
  // one-token decode with the shared expert: its w1/w3 rows (M = 2, T = 1) run
  // in the routed w1/w3 launch and its w2 rows (M = 1, T = 1, accumulating
  // into y) in the routed w2 launch; host memory, read when launching (null:
  // none; both or neither)
  const SharedArgs* shared13;
  const SharedArgs* shared2;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t stream);
bool decode_fits(int T, int H, int I, int k);  // shapes the decode kernels take
bool decode_fuses_route(int T, int H, int I, int E, int k);  // decode routes in its first kernel
bool decode_one_token(int T, int H, int I, int k);           // the one-token decode kernels run
int decode_family(int T, int H, int I, int k);  // 1 one-token, 2 few-token GEMV, 3 MFMA GEMV
hipError_t launch_decode(const LayerArgs& a, hipStream_t stream);
hipError_t launch_prefill(const LayerArgs& a, hipStream_t stream);
hipError_t launch_prefill_mx8(const LayerArgs& a, hipStream_t stream);
// LDS-fed bf16 prefill GEMMs: taken when K is a multiple of 256 and the n
// scale tensors have 4-byte aligned bases and strides.
bool prefill_lds_takes(int K, const uint8_t* const* scales, const int64_t* strides, int n);
hipError_t launch_gemm13_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_gemm2_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_combine(const LayerArgs& a, hipStream_t stream);
hipError_t launch_quant_mx8(const uint16_t* src, int rows, int K, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);
// Row length in codes of the MXFP8 prefill's quantised activations: K rounded
// up to its K block (the padding holds zeros).
size_t mx8_padded(int K);
hipError_t launch_unsort_h(const LayerArgs& a, uint16_t* h_out, hipStream_t stream);
// saliency[e] += sum over e's sorted slots s of slot_gate[s] * sqrt(sum_tiles sal_part[s][.])
hipError_t launch_saliency(const LayerArgs& a, float* saliency, hipStream_t stream);
constexpr int kSalRows = 256;  // w2 rows per workgroup tile in every prefill w2 kernel

// The shared expert: h = bf16(silu(W1 x) * (W3 x)) [T][I], y (+)= W2 h.
// w = {w1, s1, w3, s3, w2, s2}: E4M3 codes with 32 x 32 UE8M0 block scales.
// the shared expert's w2 alone: y (+)= W2 h
hipError_t launch_shared_w2(const uint16_t* h, const uint8_t* w2, const uint8_t* s2, int T, int H,
                            int I, float* y, int accumulate, hipStream_t stream);
hipError_t launch_shared(const uint16_t* x, const uint8_t* const w[6], int T, int H, int I,
                         float* y, int accumulate, uint16_t* h, hipStream_t stream);
// One token through the one-token decode kernels with no routed expert (sets
// done; leaves it false, launching nothing, where the shapes do not fit them).
hipError_t launch_shared_one(const uint16_t* x, const uint8_t* const w[6], int H, int I, float* y,
                             int accumulate, uint16_t* h, hipStream_t stream, bool& done);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w, float* logits, int T, int H,
                                int E, hipStream_t stream);
hipError_t launch_prenorm(const float* x, uint16_t* u, int T, int H, float eps, hipStream_t stream);

}  // namespace moe_fp4
