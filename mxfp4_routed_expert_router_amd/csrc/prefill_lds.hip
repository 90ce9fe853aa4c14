// Prefill grouped GEMMs with bf16 activations, every operand staged in LDS by
// direct global->LDS loads (lds_dma.h).  Same work, tiles and epilogues as the
// register-fed kernels of prefill.hip, which remain for shapes these do not
// take (a K that is not a multiple of 256, scale tensors not 4-byte aligned).
//
// The weights advance in blocks of 256 inputs -- one 128-byte line of each
// weight row, read by 8 lanes of one load, which the register-fed kernels
// cannot do (the MFMA wants each row's chunks on lanes 16 apart).  Three
// weight blocks are resident per wave (two in flight while one is used).  A
// bf16 activation tile of 256 inputs for 64 tokens would take 32 KB a stage,
// so the activations advance in half blocks of 128 inputs, also three stages
// deep, and the loop steps by half blocks: a weight block is issued every
// other step.  The FP4 codes are decoded from LDS into bf16 MFMA operands in
// registers (v_cvt_scalef32_pk_bf16_fp4, exact).
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "saliency.h"

namespace moe_fp4 {
namespace {

constexpr int kKB = 256;                // inputs per weight block
constexpr int kHB = 128;                // inputs per activation half block
constexpr int kTiles = 2;               // weight tiles per wave (w1 and w3, or two w2 tiles)
// Loads a wave issues per weight block.  The scale bytes of two blocks come in
// one load, issued with the even block (one scale load gathers 8 bytes from
// each of 16 rows, so a load per block costs as much request traffic as the
// weight halves).
constexpr int kWLoads = 3 * kTiles;     // even weight block: two 1 KB halves and the scales per tile
constexpr int kWLoadsOdd = 2 * kTiles;  // odd weight block: the halves only
constexpr int kXLoads = 2;              // per half block, waves whose tokens are read: two 1 KB quarters

// Two shapes of the same kernels: 8 waves and 64 tokens per pass (one
// workgroup per CU, 150 KB of LDS) for prefill chunks; 4 waves and 32 tokens
// (two workgroups per CU, 75 KB) for small batches, where each expert has a
// few tokens and a second resident workgroup hides the first one's pipeline
// fill.  Wave w stages tokens 8 w .. 8 w + 7 of a pass in both.
template <int W, int TOK>
struct LdsCfg {
  static constexpr int kWaves = W, kThreads = W * kWave, kTok = TOK, kMaxNT = TOK / 16;
  static constexpr int kRows13 = 16 * W;  // w1/w3 rows per workgroup (one 16-row tile per wave)
  static constexpr int kRows2 = 32 * W;   // w2 rows per workgroup (two 16-row tiles per wave)
  static_assert(TOK == 8 * W, "each wave stages 8 tokens of a pass");
};
using CfgBig = LdsCfg<8, 64>;
using CfgSmall = LdsCfg<4, 32>;

template <class C>
struct SmemL {
  uint8_t w[3][C::kWaves][kTiles][2048];   // 16 rows x 128 bytes (see woff)
  uint8_t x[3][C::kTok * kHB * 2];         // kTok tokens x 128 bf16 (see xoff_h)
  uint32_t ws[2][C::kWaves][kTiles][64];   // blocks 2p, 2p+1 in slot p % 2: dword d of row r at 16 d + r
  int row[C::kTok];                        // source row of each staged token
  float sal[C::kWaves * 64];               // saliency reduction (saliency.h, 8 waves only)
};

// Byte offset in a half-block activation tile of token t's 16-byte chunk c (of
// 16, 8 inputs each): 256 bytes a token, slot c ^ xsw(t), where xsw swaps the
// two 2-bit halves of t % 16.  A B read takes chunk 4 kb + i of token c16 for
// lane (c16, kb); with this slot order the 64 lanes' 16-byte reads hit the
// LDS banks without conflicts (the plain c ^ (t % 16) order costs four extra
// cycles per read, measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int xsw(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int xoff_h(int t, int c) { return t * 256 + ((c ^ xsw(t)) << 4); }

template <int N>
__device__ __forceinline__ void wait_n() { wait_then_barrier<N>(); }

// Wait for this wave's loads of the operands of step hb (the activation half
// block, and for hb even the weight block), allowing in flight what was issued
// after them: one weight block and one half block (see the issue order in
// gemm_pass_lds).  xw: whether this wave loads activations.
__device__ __forceinline__ void wait_step(int hb, int NHB, int NB, bool xw) {
  const int wb = (hb + 1) / 2 + 1;  // the weight block issued after step hb's operands
  const bool w_after = wb < NB, w_even = (wb & 1) == 0;
  const bool x_after = xw && hb + 1 < NHB;
  if (w_after && x_after)
    w_even ? wait_n<kWLoads + kXLoads>() : wait_n<kWLoadsOdd + kXLoads>();
  else if (w_after)
    w_even ? wait_n<kWLoads>() : wait_n<kWLoadsOdd>();
  else if (x_after)
    wait_n<kXLoads>();
  else
    wait_n<0>();
}

// One pass over all K (a multiple of 256) for up to NT*16 staged token rows of
// src (row length ld = K): acc[m][rt][nt] = W_m[rows of tile rt] . X^T[tokens of nt].
// wrow0[m][rt] points at row 0 of the wave's 16-row tile (inside the weights
// even for a tile past the end, whose results are not stored), srow0 at that
// row's scales.  Tokens past nc read token 0's row.
template <class C, int M, int kRT, int NT>
__device__ __forceinline__ void gemm_pass_lds(SmemL<C>& sm, const uint8_t* const (&wrow0)[M][kRT],
                                              const uint8_t* const (&srow0)[M][kRT], size_t wrow,
                                              size_t srow, const uint16_t* __restrict__ src, int nc,
                                              int K, f32x4 (&acc)[M][kRT][NT]) {
  static_assert(M * kRT == kTiles, "tile count");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15, kb = lane >> 4;
  const int NB = K / kKB, NHB = 2 * NB;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[m][rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wr_r = lane >> 3, wr_c0 = wtile_chunk(lane, 0), wr_c1 = wtile_chunk(lane, 1);
  // activation lanes: quarter q covers tokens 8 w + 4 q + lane / 16, slot lane % 16
  const bool xw = 8 * w < 16 * NT;  // this wave stages tokens that are read
  const uint8_t* xsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 8 * w + 4 * q + (lane >> 4);
    xsrc[q] = reinterpret_cast<const uint8_t*>(src + (size_t)sm.row[t < nc ? t : 0] * K) +
              ((c16 ^ xsw(t)) << 4);
  }

  // scale lanes: tile row lane % 16, dword lane / 16 of a block pair's 16
  // bytes (dwords 2, 3 belong to the odd block; past the last block a lane
  // re-reads the even block's)
  auto issue_w = [&](int b) {
    const int s = b % 3;
    const bool even = (b & 1) == 0;
    const int so = b * 8 + 4 * (b + 1 < NB ? kb : kb & 1);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        uint8_t* const dst = &sm.w[s][w][m * kRT + rt][0];
        const uint8_t* const g = wrow0[m][rt] + (size_t)b * 128;
        lds_load16(lds_addr(dst), g + wr_r * wrow + 16 * wr_c0);
        lds_load16(lds_addr(dst + 1024), g + (8 + wr_r) * wrow + 16 * wr_c1);
        if (even)
          lds_load4(lds_addr(&sm.ws[(b >> 1) & 1][w][m * kRT + rt][0]), srow0[m][rt] + c16 * srow + so);
      }
  };
  auto issue_x = [&](int hb) {
    if (!xw) return;
    uint8_t* const dst = &sm.x[hb % 3][0];
    lds_load16(lds_addr(dst + (8 * w) * 256), xsrc[0] + (size_t)hb * (kHB * 2));
    lds_load16(lds_addr(dst + (8 * w + 4) * 256), xsrc[1] + (size_t)hb * (kHB * 2));
  };
  auto compute = [&](int hb) {
    const int b = hb >> 1, s = b % 3, hh = hb & 1, ps = (b >> 1) & 1, d = 2 * (b & 1) + hh;
    const uint8_t* const xt = &sm.x[hb % 3][0];
    u32x4 A4[M][kRT];
    float sc[M][kRT];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        A4[m][rt] = ld16(&sm.w[s][w][m * kRT + rt][woff(c16, 4 * hh + kb)]);
        sc[m][rt] = ue8m0_to_f32((sm.ws[ps][w][m * kRT + rt][16 * d + c16] >> (8 * kb)) & 0xFFu);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 A[M][kRT];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) A[m][rt] = fp4x8_to_bf16x8(A4[m][rt][i], sc[m][rt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // MFMA i takes inputs 32 (l / 16) + 8 i .. +7 of the half block from
        // lane group l / 16, in A and B alike
        const bf16x8 B = as_bf16x8(ld16(xt + xoff_h(16 * nt + c16, 4 * kb + i)));
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) acc[m][rt][nt] = mfma16x16x32(A[m][rt], B, acc[m][rt][nt]);
      }
    }
  };

  // Issue order: W0 X0 W1 X1, then per step hb: X(hb + 2), and for hb even
  // W(hb/2 + 2).  At step hb, X(hb) (and W(hb/2), which precedes it) were
  // issued before W((hb + 1)/2 + 1) and X(hb + 1), the loads wait_step leaves
  // in flight: two weight blocks are in flight during each step.
  issue_w(0);
  issue_x(0);
  if (NB > 1) issue_w(1);
  issue_x(1);
  for (int hb = 0; hb < NHB; ++hb) {
    wait_step(hb, NHB, NB, xw);
    // every wave is past step hb - 1: its slots (x (hb - 1) % 3, and for hb
    // even the weight slot of block hb/2 - 1, and the scale pair slot of
    // blocks hb/2 - 2 and hb/2 - 1) may be loaded again
    if (hb + 2 < NHB) issue_x(hb + 2);
    if (!(hb & 1) && hb / 2 + 2 < NB) issue_w(hb / 2 + 2);
    compute(hb);
  }
  __syncthreads();  // the LDS is free for the caller (and its row table may change)
}

template <class C>
__global__ void __launch_bounds__(C::kThreads) gemm13_lds_kernel(LayerArgs a) {
  constexpr int kRows13 = C::kRows13, kTok = C::kTok;
  const int tpe = (a.I + kRows13 - 1) / kRows13;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  const int ne = a.counts[e];
  if (ne == 0) return;
  const int off = a.offsets[e];
  __shared__ SmemL<C> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15, kb = lane >> 4;
  const int rw = rtile * kRows13 + w * 16;
  const size_t wrow = (size_t)a.H / 2, srow = (size_t)a.H / 32;
  const bool act = rw < a.I;
  const size_t ro = (size_t)(act ? rw : 0);  // a tile past the end reads rows 0..15
  const uint8_t* const wr[2][1] = {{a.w1 + (size_t)e * a.stride[0] + ro * wrow},
                                   {a.w3 + (size_t)e * a.stride[2] + ro * wrow}};
  const uint8_t* const sr[2][1] = {{a.s1 + (size_t)e * a.stride[1] + ro * srow},
                                   {a.s3 + (size_t)e * a.stride[3] + ro * srow}};
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (tid < nc) sm.row[tid] = a.slot_tok[off + c0 + tid];
    lds_barrier();
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[2][1][NT];
      gemm_pass_lds<C, 2, 1, NT>(sm, wr, sr, wrow, srow, a.x, nc, a.H, acc);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = 16 * nt + c16;
        if (act && tok < nc) {
          uint16_t hv[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) hv[qq] = swiglu_bf16(acc[0][0][nt][qq], acc[1][0][nt][qq]);
          const uint2 pk = {(uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                            (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
          *reinterpret_cast<uint2*>(a.h + (size_t)(off + c0 + tok) * a.I + rw + 4 * kb) = pk;
        }
      }
    };
    if constexpr (C::kMaxNT == 4) {
      switch ((nc + 15) / 16) {
        case 1: pass(IntC<1>{}); break;
        case 2: pass(IntC<2>{}); break;
        case 3: pass(IntC<3>{}); break;
        default: pass(IntC<4>{}); break;
      }
    } else {
      if (nc <= 16) pass(IntC<1>{}); else pass(IntC<2>{});
    }
  }
}

template <class C>
__global__ void __launch_bounds__(C::kThreads) gemm2_lds_kernel(LayerArgs a) {
  constexpr int kRows2 = C::kRows2, kTok = C::kTok;
  const int tpe = (a.H + kRows2 - 1) / kRows2;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  const int ne = a.counts[e];
  if (ne == 0) return;
  const int off = a.offsets[e];
  __shared__ SmemL<C> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15, kb = lane >> 4;
  const int rw = rtile * kRows2 + w * 32;
  const size_t wrow = (size_t)a.I / 2, srow = (size_t)a.I / 32;
  bool act[2];
  const uint8_t* wr[1][2];
  const uint8_t* sr[1][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rw + 16 * rt;
    act[rt] = r < a.H;
    const size_t ro = (size_t)(act[rt] ? r : 0);
    wr[0][rt] = a.w2 + (size_t)e * a.stride[4] + ro * wrow;
    sr[0][rt] = a.s2 + (size_t)e * a.stride[5] + ro * srow;
  }
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (tid < nc) sm.row[tid] = off + c0 + tid;
    lds_barrier();
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[1][2][NT];
      gemm_pass_lds<C, 1, 2, NT>(sm, wr, sr, wrow, srow, a.h, nc, a.I, acc);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int tok = 16 * nt + c16;
          if (act[rt] && tok < nc) {
            const int s = off + c0 + tok;
            const float gate = a.slot_gate[s];
            const f32x4 v = acc[0][rt][nt];
            const float4 o = {gate * v[0], gate * v[1], gate * v[2], gate * v[3]};
            *reinterpret_cast<float4*>(a.ypair + (size_t)s * a.H + rw + 16 * rt + 4 * kb) = o;
          }
        }
      if constexpr (C::kWaves == 8)
        if (a.sal_part) saliency_tile<2, NT>(a, acc, act, sm.sal, off + c0, nc, rtile);
    };
    if constexpr (C::kMaxNT == 4) {
      switch ((nc + 15) / 16) {
        case 1: pass(IntC<1>{}); break;
        case 2: pass(IntC<2>{}); break;
        case 3: pass(IntC<3>{}); break;
        default: pass(IntC<4>{}); break;
      }
    } else {
      if (nc <= 16) pass(IntC<1>{}); else pass(IntC<2>{});
    }
  }
}

static_assert(CfgBig::kRows2 == kSalRows, "saliency tiles are the w2 workgroup tiles");

}  // namespace

bool prefill_lds_takes(int K, const uint8_t* const* scales, const int64_t* strides, int n) {
  if (K % kKB) return false;
  for (int i = 0; i < n; ++i)
    if ((uintptr_t)scales[i] % 4 || strides[i] % 4) return false;
  return true;
}

namespace {
// Small batches (at most 32 tokens, so at most 32 per expert: one pass) take
// the 4-wave shape; saliency needs the 8-wave one's 256-row w2 tiles.
bool small_batch(const LayerArgs& a) { return a.T <= CfgSmall::kTok && !a.sal_part; }

template <class C>
void launch13(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int t13 = a.E * ((a.I + C::kRows13 - 1) / C::kRows13);
  launch_k(gemm13_lds_kernel<C>, dim3(xcd_grid(t13)), dim3(C::kThreads), 0, stream, start, stop, a);
}
template <class C>
void launch2(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int t2 = a.E * ((a.H + C::kRows2 - 1) / C::kRows2);
  launch_k(gemm2_lds_kernel<C>, dim3(xcd_grid(t2)), dim3(C::kThreads), 0, stream, start, stop, a);
}
}  // namespace

hipError_t launch_gemm13_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (small_batch(a))
    launch13<CfgSmall>(a, stream, start, stop);
  else
    launch13<CfgBig>(a, stream, start, stop);
  return hipGetLastError();
}

hipError_t launch_gemm2_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (small_batch(a))
    launch2<CfgSmall>(a, stream, start, stop);
  else
    launch2<CfgBig>(a, stream, start, stop);
  return hipGetLastError();
}

}  // namespace moe_fp4
