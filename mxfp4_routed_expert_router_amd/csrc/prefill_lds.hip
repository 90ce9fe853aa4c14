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
constexpr int kXLoads = 2;              // per half block, waves whose tokens are read: two 1 KB quarters

// Two shapes of the same kernels: 8 waves and 64 tokens per pass (one
// workgroup per CU, 150 KB of LDS) for prefill chunks; 4 waves and 32 tokens
// (two workgroups per CU, 75 KB) for small batches, where each expert has a
// few tokens and a second resident workgroup hides the first one's pipeline
// fill.  Wave w stages tokens 8 w .. 8 w + 7 of a pass in both.
//
// The scale bytes of the weight tiles come in one of two ways.  Pair loads
// (any K): one 4-byte load per tile with every even block, the 8 bytes of two
// blocks from each of the tile's 16 rows.  Such a load touches 16 cache lines
// for 256 bytes, as many line requests as the tile's two weight halves.  Quad
// loads (QS: rows of scales a multiple of 16 bytes, i.e. K a multiple of 512,
// and 16-byte aligned scale tensors): one 16-byte load per wave with every
// fourth block, lanes 0-31 the 32 bytes of four blocks of each row of tile 0,
// lanes 32-63 those of tile 1: a quarter of the instructions and half the line
// requests.  They need twice the LDS, found by keeping the row table and the
// saliency buffer in the activation stages, which are free when those are used.
template <int W, int TOK, bool QS>
struct LdsCfg {
  static constexpr int kWaves = W, kThreads = W * kWave, kTok = TOK, kMaxNT = TOK / 16;
  static constexpr int kRows13 = 16 * W;  // w1/w3 rows per workgroup (one 16-row tile per wave)
  static constexpr int kRows2 = 32 * W;   // w2 rows per workgroup (two 16-row tiles per wave)
  static constexpr bool kQuad = QS;
  // small batches: the grid runs over the routing's distinct-expert records
  // (expert_slots), not over all E experts
  static constexpr bool kDistinct = W == 4;
  // loads a wave issues with weight block b: the two 1 KB halves of each tile,
  // and the scale loads that come with it (kWLoadsBig when b is a multiple of
  // kScaleEvery)
  static constexpr int kScaleEvery = QS ? 4 : 2;
  static constexpr int kWLoadsBig = QS ? 2 * kTiles + 1 : 3 * kTiles;
  static constexpr int kWLoadsSmall = 2 * kTiles;
  static_assert(TOK == 8 * W, "each wave stages 8 tokens of a pass");
};
template <bool QS>
using CfgBig = LdsCfg<8, 64, QS>;
template <bool QS>
using CfgSmall = LdsCfg<4, 32, QS>;

template <class C>
struct SmemL {
  static constexpr int kXStage = C::kTok * kHB * 2;  // kTok tokens x 128 bf16 (see xoff_h)
  uint8_t w[3][C::kWaves][kTiles][2048];             // 16 rows x 128 bytes (see woff)
  union {
    uint8_t x[3][kXStage];
    // between passes: the row table of a later pass in stage 2 (written after
    // the previous pass's last barrier; stage 2 is loaded again only after the
    // first barrier of the pass, when every wave has read the table)
    struct {
      uint8_t before[2 * kXStage];
      int row[C::kTok];  // source row of each staged token
    } t;
    float sal[C::kWaves * 64];  // saliency reduction after a pass (saliency.h, 8 waves only)
  } u;
  // pair loads: blocks 2p, 2p + 1 in slot p % 2, dword d of row r of tile t at
  // [t][16 d + r]; quad loads: blocks 4p .. 4p + 3 in slot p % 2, byte g of
  // block b of row r of tile t at 512 t + 32 r + 8 (b % 4) + g
  uint32_t ws[2][C::kWaves][kTiles][C::kQuad ? 128 : 64];
};
static_assert(sizeof(SmemL<CfgBig<true>>) <= 160 * 1024, "LDS of the quad-scale shape");

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
template <class C>
__device__ __forceinline__ void wait_step(int hb, int NHB, int NB, bool xw) {
  const int wb = (hb + 1) / 2 + 1;  // the weight block issued after step hb's operands
  const bool w_after = wb < NB, w_big = wb % C::kScaleEvery == 0;
  const bool x_after = xw && hb + 1 < NHB;
  if (w_after && x_after)
    w_big ? wait_n<C::kWLoadsBig + kXLoads>() : wait_n<C::kWLoadsSmall + kXLoads>();
  else if (w_after)
    w_big ? wait_n<C::kWLoadsBig>() : wait_n<C::kWLoadsSmall>();
  else if (x_after)
    wait_n<kXLoads>();
  else
    wait_n<0>();
}

// Weight block b (256 inputs) of the wave's tiles into stage b % 3, and the
// scale bytes that come with it (pair loads: for b even, those of blocks b and
// b + 1 into slot (b / 2) % 2; quad loads: for b a multiple of 4, those of
// blocks b .. b + 3 into slot (b / 4) % 2).  The
// weight halves carry the non-temporal hint: each is read once a pass, and
// the L2 then keeps the gathered activation rows that every row tile of the
// expert reads again (w1/w3 reads 5.50 -> 5.07 GB, 1.375 -> 1.368 ms; the
// same hint made the MXFP8 kernels 3% slower, so they go without it).
// Pair-load lanes: tile row lane % 16, dword lane / 16 of a block pair's 16
// bytes (dwords 2, 3 belong to the odd block; past the last block a lane
// re-reads the even block's).  Quad-load lanes: tile lane / 32, row
// (lane % 32) / 2, bytes 16 (lane % 2) .. +15 of the quad (blocks 4p + 2
// (lane % 2) and the next); with K a multiple of 512 the blocks come in pairs,
// and a lane whose pair lies past the last block re-reads the quad's first.
template <class C, int M, int kRT>
__device__ __forceinline__ void issue_wblock(SmemL<C>& sm, const uint8_t* const (&wrow0)[M][kRT],
                                             const uint8_t* const (&srow0)[M][kRT], size_t wrow,
                                             size_t srow, int b, int NB) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c16 = lane & 15, kb = lane >> 4;
  const int wr_r = lane >> 3, wr_c0 = wtile_chunk(lane, 0), wr_c1 = wtile_chunk(lane, 1);
  const int s = b % 3;
  const bool even = (b & 1) == 0;
  const int so = b * 8 + 4 * (b + 1 < NB ? kb : kb & 1);
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      uint8_t* const dst = &sm.w[s][w][m * kRT + rt][0];
      const uint8_t* const g = wrow0[m][rt] + (size_t)b * 128;
      lds_load16_nt(lds_addr(dst), g + wr_r * wrow + 16 * wr_c0);
      lds_load16_nt(lds_addr(dst + 1024), g + (8 + wr_r) * wrow + 16 * wr_c1);
      if constexpr (!C::kQuad)
        if (even)
          lds_load4(lds_addr(&sm.ws[(b >> 1) & 1][w][m * kRT + rt][0]), srow0[m][rt] + c16 * srow + so);
    }
  if constexpr (C::kQuad)
    if ((b & 3) == 0) {
      static_assert(M * kRT == 2, "quad loads: two tiles a wave");
      const int t = lane >> 5, r = (lane & 31) >> 1, hp = lane & 1;
      // tile 1's row 0 as an offset from tile 0's (a select of the two array
      // elements by lane would become an indexed load from scratch)
      const uint8_t* const sp = srow0[0][0] + (ptrdiff_t)t * (srow0[M - 1][kRT - 1] - srow0[0][0]);
      const int qo = b * 8 + (b + 2 * hp < NB ? 16 * hp : 0);
      lds_load16(lds_addr(&sm.ws[(b >> 2) & 1][w][0][0]), sp + r * srow + qo);
    }
}

// Weight blocks 0 and 1 of a pass: they need only the expert and the rows, so
// the kernels issue them before the token rows of the pass are known.
template <class C, int M, int kRT>
__device__ __forceinline__ void issue_first_wblocks(SmemL<C>& sm, const uint8_t* const (&wrow0)[M][kRT],
                                                    const uint8_t* const (&srow0)[M][kRT],
                                                    size_t wrow, size_t srow, int K) {
  const int NB = K / kKB;
  issue_wblock<C, M, kRT>(sm, wrow0, srow0, wrow, srow, 0, NB);
  if (NB > 1) issue_wblock<C, M, kRT>(sm, wrow0, srow0, wrow, srow, 1, NB);
}

// One pass over all K (a multiple of 256) for up to NT*16 staged token rows of
// src (row length ld = K): acc[m][rt][nt] = W_m[rows of tile rt] . X^T[tokens of nt].
// wrow0[m][rt] points at row 0 of the wave's 16-row tile (inside the weights
// even for a tile past the end, whose results are not stored), srow0 at that
// row's scales.  trow[i]: the source row of the wave's staged token 8 w + i
// (any valid row past the pass's tokens: their results are not stored).  The
// caller has issued weight blocks 0 and 1 (issue_first_wblocks).
template <class C, int M, int kRT, int NT>
__device__ __forceinline__ void gemm_pass_lds(SmemL<C>& sm, const uint8_t* const (&wrow0)[M][kRT],
                                              const uint8_t* const (&srow0)[M][kRT], size_t wrow,
                                              size_t srow, const uint16_t* __restrict__ src,
                                              const int (&trow)[8], int K,
                                              f32x4 (&acc)[M][kRT][NT]) {
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

  // activation lanes: quarter q covers tokens 8 w + 4 q + lane / 16, slot lane % 16
  const bool xw = 8 * w < 16 * NT;  // this wave stages tokens that are read
  const uint8_t* xsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 8 * w + 4 * q + (lane >> 4), li = 4 * q + (lane >> 4);
    int row = trow[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) row = li == i ? trow[i] : row;  // a select: trow stays uniform
    xsrc[q] = reinterpret_cast<const uint8_t*>(src + (size_t)row * K) + ((c16 ^ xsw(t)) << 4);
  }

  auto issue_w = [&](int b) { issue_wblock<C, M, kRT>(sm, wrow0, srow0, wrow, srow, b, NB); };
  auto issue_x = [&](int hb) {
    if (!xw) return;
    uint8_t* const dst = &sm.u.x[hb % 3][0];
    lds_load16(lds_addr(dst + (8 * w) * 256), xsrc[0] + (size_t)hb * (kHB * 2));
    lds_load16(lds_addr(dst + (8 * w + 4) * 256), xsrc[1] + (size_t)hb * (kHB * 2));
  };
  auto compute = [&](int hb) {
    const int b = hb >> 1, s = b % 3, hh = hb & 1, ps = (b >> 1) & 1, d = 2 * (b & 1) + hh;
    const uint8_t* const xt = &sm.u.x[hb % 3][0];
    u32x4 A4[M][kRT];
    float sc[M][kRT];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        A4[m][rt] = ld16(&sm.w[s][w][m * kRT + rt][woff(c16, 4 * hh + kb)]);
        if constexpr (C::kQuad) {
          const uint8_t* const q = reinterpret_cast<const uint8_t*>(&sm.ws[(b >> 2) & 1][w][0][0]);
          sc[m][rt] = ue8m0_to_f32(q[512 * (m * kRT + rt) + 32 * c16 + 8 * (b & 3) + 4 * hh + kb]);
        } else {
          sc[m][rt] = ue8m0_to_f32((sm.ws[ps][w][m * kRT + rt][16 * d + c16] >> (8 * kb)) & 0xFFu);
        }
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

  // Issue order: W0 W1 (by the caller) X0 X1, then per step hb: X(hb + 2), and
  // for hb even W(hb/2 + 2).  At step hb > 0, X(hb) (and W(hb/2), which
  // precedes it) were issued before W((hb + 1)/2 + 1) and X(hb + 1), the loads
  // wait_step leaves in flight: two weight blocks are in flight during each
  // step.  At step 0 only X1 follows X0 (W1 came first).
  issue_x(0);
  issue_x(1);
  for (int hb = 0; hb < NHB; ++hb) {
    if (hb == 0) {
      if (xw && NHB > 1)
        wait_n<kXLoads>();
      else if (!xw && NB > 1)
        wait_n<C::kWLoadsSmall>();  // block 1 is never one that brings scales
      else
        wait_n<0>();
    } else {
      wait_step<C>(hb, NHB, NB, xw);
    }
    // every wave is past step hb - 1: its slots (x (hb - 1) % 3, and for hb
    // even the weight slot of block hb/2 - 1, and the scale pair slot of
    // blocks hb/2 - 2 and hb/2 - 1) may be loaded again
    if (hb + 2 < NHB) issue_x(hb + 2);
    if (!(hb & 1) && hb / 2 + 2 < NB) issue_w(hb / 2 + 2);
    compute(hb);
  }
  __syncthreads();  // the LDS is free for the caller (and its row table may change)
}

// An expert's token count and offset by scalar loads issued and waited for in
// one asm block: they follow the weight DMA loads of the kernel's entry,
// behind which the compiler would otherwise place vector loads and a wait for
// every load (it cannot see what the DMA loads write).  Scalar loads count
// apart from them (lgkmcnt), so the weights stay in flight.
__device__ __forceinline__ void scalar_count_offset(const int32_t* cnt, const int32_t* offp, int& ne,
                                                    int& off) {
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(ne), "=&s"(off)
      : "s"(cnt), "s"(offp)
      : "memory");
}
// The wave's 8 token rows of the first pass the same way: trow[i] =
// slot_tok[first + min(8 w + i, nc - 1)].
__device__ __forceinline__ void scalar_token_rows(const int32_t* slot_tok, int first, int nc,
                                                  int (&trow)[8]) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int32_t* p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = slot_tok + first + min(8 * w + i, nc - 1);
  asm volatile(
      "s_load_dword %0, %8, 0x0\n\t"
      "s_load_dword %1, %9, 0x0\n\t"
      "s_load_dword %2, %10, 0x0\n\t"
      "s_load_dword %3, %11, 0x0\n\t"
      "s_load_dword %4, %12, 0x0\n\t"
      "s_load_dword %5, %13, 0x0\n\t"
      "s_load_dword %6, %14, 0x0\n\t"
      "s_load_dword %7, %15, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(trow[0]), "=&s"(trow[1]), "=&s"(trow[2]), "=&s"(trow[3]), "=&s"(trow[4]),
        "=&s"(trow[5]), "=&s"(trow[6]), "=&s"(trow[7])
      : "s"(p[0]), "s"(p[1]), "s"(p[2]), "s"(p[3]), "s"(p[4]), "s"(p[5]), "s"(p[6]), "s"(p[7])
      : "memory");
}

// The expert slots of a grid: all E experts (each workgroup then reads its
// expert's token count and offset, and leaves at once if there are none), or
// for the small-batch shape the distinct-expert records of the routing, at
// most min(E, T k), those past the last distinct expert marked -1.  At 32
// tokens, top-6 of 384, that is 192 slots for about 95 distinct experts
// instead of 384, so about 3,500 instead of 10,400 w1/w3 workgroups find
// nothing to do.
template <class C>
__host__ __device__ inline int expert_slots(const LayerArgs& a) {
  return C::kDistinct ? (a.E < a.T * a.k ? a.E : a.T * a.k) : a.E;
}

// A workgroup's expert slot and row tile.  Over all E experts: xcd_tile's
// ranges, an expert's tiles on one XCD.  Over the distinct-expert records,
// which are dense at the front: XCD x (blockIdx % 8) takes records x, x + 8,
// x + 16, ..., so the records that have an expert spread over every XCD
// (contiguous ranges would give them all to the first few).
template <class C>
__device__ __forceinline__ bool expert_tile(const LayerArgs& a, int tpe, int& es, int& rtile) {
  if constexpr (C::kDistinct) {
    const int j = blockIdx.x >> 3, r = j / tpe;
    es = (blockIdx.x & 7) + 8 * r;
    rtile = j - r * tpe;
    return es < expert_slots<C>(a);
  } else {
    int logical;
    if (!xcd_tile(a.E * tpe, logical)) return false;
    es = logical / tpe;
    rtile = logical - es * tpe;
    return true;
  }
}
template <class C>
unsigned expert_grid(const LayerArgs& a, int tpe) {
  return C::kDistinct ? (unsigned)(8 * ((expert_slots<C>(a) + 7) / 8) * tpe) : xcd_grid(a.E * tpe);
}

// A distinct-expert record (expert, first sorted slot, pairs) by scalar loads.
__device__ __forceinline__ void scalar_record(const int32_t* rec, int& e, int& off, int& ne) {
  asm volatile(
      "s_load_dword %0, %3, 0x0\n\t"
      "s_load_dword %1, %3, 0x4\n\t"
      "s_load_dword %2, %3, 0x8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(e), "=&s"(off), "=&s"(ne)
      : "s"(rec)
      : "memory");
}

// Whether a workgroup issues its first two weight blocks before it has read
// its expert's token count: worth it where nearly every expert has tokens (two
// or more slots per expert on average).  In small batches most experts have
// none, and the early loads of their workgroups would only add traffic (at 32
// tokens, top-6 of 384, about a third more w1/w3 bytes).
__device__ __forceinline__ bool early_wblocks(const LayerArgs& a) { return a.T * a.k >= 2 * a.E; }

template <class C>
__global__ void __launch_bounds__(C::kThreads) gemm13_lds_kernel(LayerArgs a) {
  constexpr int kRows13 = C::kRows13, kTok = C::kTok;
  const int tpe = (a.I + kRows13 - 1) / kRows13;
  int es, rtile;
  if (!expert_tile<C>(a, tpe, es, rtile)) return;
  int e = es, ne = 0, off = 0;
  if constexpr (C::kDistinct) {
    scalar_record(a.dinfo + 4 * es, e, off, ne);
    if (e < 0) return;
  }
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
  const int NB = a.H / kKB;
  // Weight blocks 0 and 1 of the first pass need only the expert and the rows:
  // where most experts have tokens they go out at entry, before the expert's
  // token count, offset and token rows are known (early_wblocks).
  const bool early = !C::kDistinct && early_wblocks(a);
  if (early) issue_first_wblocks<C, 2, 1>(sm, wr, sr, wrow, srow, a.H);
  if constexpr (!C::kDistinct) {
    scalar_count_offset(a.counts + e, a.offsets + e, ne, off);
    if (ne == 0) {
      if (early) wait_n<0>();  // the DMA lands before the workgroup's LDS is released
      return;
    }
  }
  if (!early) issue_first_wblocks<C, 2, 1>(sm, wr, sr, wrow, srow, a.H);
  int trow[8];
  scalar_token_rows(a.slot_tok, off, min(kTok, ne), trow);
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (c0 > 0) {
      // A later pass: its token rows go to LDS by a DMA load of wave 0 issued
      // before weight blocks 0 and 1, so the wait for the rows leaves the
      // weights in flight.
      static_assert(kTok <= kWave, "one row-table load per pass");
      if (w == 0) lds_load4(lds_addr(&sm.u.t.row[0]), a.slot_tok + off + c0 + min(lane, nc - 1));
      issue_first_wblocks<C, 2, 1>(sm, wr, sr, wrow, srow, a.H);
      if (NB > 1)
        wait_n<C::kWLoadsBig + C::kWLoadsSmall>();
      else
        wait_n<C::kWLoadsBig>();
#pragma unroll
      for (int i = 0; i < 8; ++i) trow[i] = sm.u.t.row[min(8 * w + i, nc - 1)];
    }
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[2][1][NT];
      gemm_pass_lds<C, 2, 1, NT>(sm, wr, sr, wrow, srow, a.x, trow, a.H, acc);
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
  int es, rtile;
  if (!expert_tile<C>(a, tpe, es, rtile)) return;
  int e = es, ne = 0, off = 0;
  if constexpr (C::kDistinct) {
    scalar_record(a.dinfo + 4 * es, e, off, ne);
    if (e < 0) return;
  }
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
  // weight blocks 0 and 1 of the first pass as in gemm13_lds_kernel
  const bool early = !C::kDistinct && early_wblocks(a);
  if (early) issue_first_wblocks<C, 1, 2>(sm, wr, sr, wrow, srow, a.I);
  if constexpr (!C::kDistinct) {
    scalar_count_offset(a.counts + e, a.offsets + e, ne, off);
    if (ne == 0) {
      if (early) wait_n<0>();
      return;
    }
  }
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (c0 > 0 || !early) issue_first_wblocks<C, 1, 2>(sm, wr, sr, wrow, srow, a.I);
    int trow[8];  // the h rows are the sorted slots
#pragma unroll
    for (int i = 0; i < 8; ++i) trow[i] = off + c0 + min(8 * w + i, nc - 1);
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[1][2][NT];
      gemm_pass_lds<C, 1, 2, NT>(sm, wr, sr, wrow, srow, a.h, trow, a.I, acc);
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
        if (a.sal_part) saliency_tile<2, NT>(a, acc, act, sm.u.sal, off + c0, nc, rtile);
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

static_assert(CfgBig<false>::kRows2 == kSalRows, "saliency tiles are the w2 workgroup tiles");

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
bool small_batch(const LayerArgs& a) { return a.T <= CfgSmall<false>::kTok && !a.sal_part; }

// Quad scale loads (see LdsCfg): K a multiple of 512, so that each row's
// K / 32 scale bytes are whole 16-byte chunks, and 16-byte aligned tensors and
// expert strides.
bool quad_scales(int K, const uint8_t* const* scales, const int64_t* strides, int n) {
  if (K % (2 * kKB)) return false;
  for (int i = 0; i < n; ++i)
    if ((uintptr_t)scales[i] % 16 || strides[i] % 16) return false;
  return true;
}

template <class C>
void launch13(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int tpe = (a.I + C::kRows13 - 1) / C::kRows13;
  launch_k(gemm13_lds_kernel<C>, dim3(expert_grid<C>(a, tpe)), dim3(C::kThreads), 0, stream, start, stop, a);
}
template <class C>
void launch2(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int tpe = (a.H + C::kRows2 - 1) / C::kRows2;
  launch_k(gemm2_lds_kernel<C>, dim3(expert_grid<C>(a, tpe)), dim3(C::kThreads), 0, stream, start, stop, a);
}
}  // namespace

hipError_t launch_gemm13_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const uint8_t* const sc[2] = {a.s1, a.s3};
  const int64_t st[2] = {a.stride[1], a.stride[3]};
  const bool q = quad_scales(a.H, sc, st, 2), small = small_batch(a);
  if (small && q)
    launch13<CfgSmall<true>>(a, stream, start, stop);
  else if (small)
    launch13<CfgSmall<false>>(a, stream, start, stop);
  else if (q)
    launch13<CfgBig<true>>(a, stream, start, stop);
  else
    launch13<CfgBig<false>>(a, stream, start, stop);
  return hipGetLastError();
}

hipError_t launch_gemm2_lds(const LayerArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const uint8_t* const sc[1] = {a.s2};
  const int64_t st[1] = {a.stride[5]};
  const bool q = quad_scales(a.I, sc, st, 1), small = small_batch(a);
  if (small && q)
    launch2<CfgSmall<true>>(a, stream, start, stop);
  else if (small)
    launch2<CfgSmall<false>>(a, stream, start, stop);
  else if (q)
    launch2<CfgBig<true>>(a, stream, start, stop);
  else
    launch2<CfgBig<false>>(a, stream, start, stop);
  return hipGetLastError();
}

}  // namespace moe_fp4
