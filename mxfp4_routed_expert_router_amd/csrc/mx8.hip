// MXFP8 mode of the prefill path.  The activations are quantised to the OCP MX
// FP8 format (E4M3 codes, one UE8M0 scale per 32 consecutive inputs) so that
// the matrix cores take the FP4 weights exactly as the checkpoint stores them:
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies A = 16 rows x 128 inputs of
// E2M1 codes by B = 128 inputs x 16 tokens of E4M3 codes, each operand with one
// UE8M0 scale per 32 inputs.  Lane l supplies A row l % 16, inputs 32 (l/16) ..
// +31 -- one 16-byte scale group of a weight row, low nibble first, with that
// group's scale byte -- and B column l % 16, inputs 16 (l/16) .. +15 and
// 64 + 16 (l/16) .. +15, with the scale byte of column l % 16's group l / 16;
// it receives D rows 4 (l/16) .. +3 of column l % 16.  One instruction covers
// four scale groups, with no FP4 decode on the vector units.
//
// What the mode computes is the plain layer with x quantised before w1/w3 and
// the bf16 h quantised before w2 (DeepSeek-V4.1-Flash pages: the expert weights
// are FP4 E2M1 with UE8M0 scales, 10100.com page, section on the expert-capacity
// bottleneck; the FP8 activations are this mode's reading).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "saliency.h"

namespace moe_fp4 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ quantiser
// One thread per 8 values; the 4 threads of a quad hold one block of 32 and
// take its maximum with quad_perm exchanges.  Shared exponent: the UE8M0 byte
// floor(log2(amax)) - 8 + 127 (8 = largest E4M3 exponent), clamped to
// [0, 254]; 0 for a zero block.  Element: v * 2^(127 - byte) (exact: a power
// of two), clamped to +-448 and converted by v_cvt_scalef32_pk_fp8_f32 (round
// to nearest even, sign kept for zero).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v))));
  return v;
}

__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (amax == 0.0f) return 0u;
  const int ef = (int)((b >> 23) & 0xFF);
  // floor(log2(amax)): from the exponent field, or the mantissa's top bit when subnormal
  const int e = ef ? ef - 127 : (31 - __builtin_clz(b & 0x7FFFFF)) - 149;
  const int se = e - 8 + 127;
  return (uint32_t)(se < 0 ? 0 : se > 254 ? 254 : se);
}

// 2^(127 - se) for se in [0, 254] (a subnormal fp32 for se = 254).
__device__ __forceinline__ float mx8_inv_scale(uint32_t se) {
  const int e = 127 - (int)se;
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(1u << (e + 149));
}

__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  s16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Rows of K values in, rows of Kp >= K codes out (Kp / 32 scale bytes); the
// codes and scales of columns K .. Kp-1 are written as zeros.
__global__ void __launch_bounds__(256) quant_mx8_kernel(const uint16_t* __restrict__ src, int rows,
                                                        int K, int Kp, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  // K and Kp are multiples of 32 and the grid stride is a multiple of 4: the
  // four threads of a quad always hold one block, and take the same branch
  const int c8 = Kp / 8;
  const size_t n8 = (size_t)rows * c8;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / c8;
    const int c = (int)(i - r * c8) * 8;
    uint2 out = {0u, 0u};
    uint32_t se = 0;
    if (c < K) {
      const u32x4 raw = ld16(src + r * K + c);
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(raw[j] << 16);
        v[2 * j + 1] = __uint_as_float(raw[j] & 0xFFFF0000u);
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = quad_max(amax);
      se = mx8_scale_byte(amax);
      const float f = mx8_inv_scale(se);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = fminf(fmaxf(v[j] * f, -448.0f), 448.0f);
      out = uint2{fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
    }
    *reinterpret_cast<uint2*>(codes + i * 8) = out;
    if ((i & 3) == 0) scales[i / 4] = (uint8_t)se;
  }
}

// ------------------------------------------------------------------ grouped GEMM
// Every operand of the main loop reaches LDS by direct global->LDS loads
// (lds_dma.h), kStages K blocks deep, so the blocks in flight cost no
// registers.  Each wave's weight chunks go to a slot that only that wave
// reads; the activation tile is shared, so one barrier per K block orders its
// loads before the reads and the reads before the slot is loaded again.
//
// A K block is 256 inputs: 128 bytes of each weight row, one whole cache line,
// read by 8 lanes together.  (Half-line blocks leave each line to be fetched
// in two pieces a block apart, which costs a sixth of the bandwidth.)  The
// quantised activations have rows padded with zeros to a multiple of 256
// inputs; in a last block of 128 inputs the weight lanes of the upper half
// re-read the lower half, whose products with those zeros vanish.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kTok = 64;                 // tokens per pass
constexpr int kKB = 256;                 // inputs per K block (two MFMAs)
constexpr int kRows13 = 16 * kWaves;     // w1/w3 rows per workgroup
constexpr int kRows2 = 32 * kWaves;      // w2 rows per workgroup (two 16-row tiles per wave)
constexpr int kStages = 3;               // K blocks resident in LDS (kStages - 1 in flight)
constexpr int kTiles = 2;                // weight tiles per wave and block (M x row tiles)
// Loads a wave issues for one block.  The scale bytes of two blocks come in
// one load, issued with the even block: a scale load gathers 8 bytes from
// each of 16 rows (16 cache lines), so fetching them a block at a time made
// the scales cost as much request traffic as the weights themselves.
constexpr int kWLoads = 3 * kTiles;      // even block, per tile: two 1 KB halves and the scales
constexpr int kXLoads = 3;               // even block, per wave holding tokens: two 1 KB quarters and scales
constexpr int kWLoadsOdd = 2 * kTiles;   // odd block: the halves only
constexpr int kXLoadsOdd = 2;
// Where K is a whole number of blocks (K % 256 == 0, K >= 512) the weight
// scales come four blocks at a time instead (QS below): one 16-byte load a
// lane, 32 lanes (16 rows x two block pairs), so half the cache lines of the
// block-pair loads, into one slot a tile.  A row's last pair may hold one
// block (K % 512 == 256): its load starts 8 bytes earlier, inside the row.  The loads of group g
// (blocks 4 g .. 4 g + 3) go out right after block 4 g - 1 has read its
// scale bytes, ahead of that iteration's block loads, so the wait for block
// 4 g (at most the next block's loads in flight) covers them.

struct SmemMx {
  uint8_t w[kStages][kWaves][kTiles][2048];   // 16 rows x 128 bytes, swizzled: see woff
  uint8_t x[kStages][kTok * kKB];             // E4M3 codes of 64 tokens, swizzled: see xoff
  // blocks 2p, 2p+1 in slot p % 2: dword d of row r at 16 d + r; or (QS) blocks
  // 4g .. 4g+3 in both slots: dword d of row r, block pair q at 4 (16 q + r) + d
  uint32_t ws[2][kWaves][kTiles][64];
  uint32_t xs[2][kWaves][32];           // token 8 w + i: scale dword d (blocks 2p, 2p+1) at 8 d + i
  int row[kTok];                              // source row of each staged token
  float sal[kWaves * 64];                     // saliency reduction (saliency.h)
};

// Byte offset in the activation tile of token t's 16-byte chunk c (of 16):
// 256 bytes a token, chunk slot c ^ (t & 15), so the B reads of 16 lanes
// (16 tokens, one chunk) spread over the banks.
__device__ __forceinline__ int xoff(int t, int c) { return t * 256 + ((c ^ (t & 15)) << 4); }

static_assert(kStages == 3, "the loop below waits for all but at most one block");

// One pass over all K (Kp = K rounded up to 256) for up to NT*16 staged token
// rows: acc[m][rt][nt] = W_m[rows of tile rt] . X^T[tokens of nt].
// M * kRT == kTiles.  wrow0[m][rt] points at row 0 of the wave's 16-row tile
// (inside the weights even for rows past the end, whose results are not
// stored); srow0 at that row's scales.  Tokens past nc load token 0's row.
// QS: weight scales four blocks to a load (K % 256 == 0, K >= 512), else two.
template <bool QS, int M, int kRT, int NT>
__device__ __forceinline__ void gemm_pass_mx(SmemMx& sm, const uint8_t* const (&wrow0)[M][kRT],
                                             const uint8_t* const (&srow0)[M][kRT], size_t wrow,
                                             size_t srow, const uint8_t* __restrict__ q,
                                             const uint8_t* __restrict__ qs, int nc, int K,
                                             f32x4 (&acc)[M][kRT][NT]) {
  static_assert(M * kRT == kTiles, "tile count");
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int c16 = lane & 15, kb = lane >> 4;
  const int Kp = (K + kKB - 1) / kKB * kKB, NB = Kp / kKB, KSp = Kp / 32;
  const bool half_tail = K != Kp;          // the last block holds 128 inputs
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[m][rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight lanes: half h covers rows 8 h + lane / 8 (see woff)
  const int wr_r = lane >> 3, wr_c0 = wtile_chunk(lane, 0), wr_c1 = wtile_chunk(lane, 1);
  // scale lanes: tile row lane % 16, dword lane / 16 of a block pair
  // activation lanes: quarter h covers tokens 8 w + 4 h + lane / 16, LDS slot
  // lane % 16 holding chunk (lane % 16) ^ (t & 15)
  const bool xw = 8 * w < 16 * NT;         // this wave stages tokens that are read
  const uint8_t* xsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * w + 4 * h + (lane >> 4);
    xsrc[h] = q + (size_t)sm.row[t < nc ? t : 0] * Kp + ((c16 ^ (t & 15)) << 4);
  }
  const int st = 8 * w + (lane & 7);
  const uint8_t* const ssrc = qs + (size_t)sm.row[st < nc ? st : 0] * KSp;

  // Byte offset, from the row's scales, of scale dword dd (0..3) of the block
  // pair starting at b: dwords 0, 1 belong to block b and 2, 3 to block b + 1.
  // Past the last block the lane re-reads block b; in a half block only dword
  // 0 exists, and dword 1 re-reads it (the inputs it scales are zeros).
  auto pair_off = [&](int b, int dd) {
    int blk = b + (dd >> 1), sub = dd & 1;
    if (blk >= NB) blk = b;
    if (half_tail && blk == NB - 1) sub = 0;
    return blk * 8 + 4 * sub;
  };
  const int wdd = lane >> 4, xdd = (lane >> 3) & 3;

  // QS scale loads of group g: lane l < 32 reads row l % 16, block pair
  // 2 g + l / 16 -- its 16 bytes, moved back to end at the row's end where
  // they pass it (a one-block last pair; pairs past the end are never used)
  uint32_t* const qslot = &sm.ws[0][0][0][0] + (size_t)w * kTiles * 128;
  auto issue_scales = [&](int g) {
    if (lane < 32) {
      const int off = min(32 * g + 16 * (lane >> 4), (int)srow - 16);
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          lds_load16(lds_addr(qslot + (m * kRT + rt) * 128), srow0[m][rt] + c16 * srow + off);
    }
  };

  auto issue = [&](int b, int s) {
    const bool tail = half_tail && b == NB - 1;
    const bool even = (b & 1) == 0;
    // in a half block, chunks 4..7 re-read chunks 0..3
    const int c0 = tail ? wr_c0 & 3 : wr_c0, c1 = tail ? wr_c1 & 3 : wr_c1;
    const int ps = (b >> 1) & 1;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        uint8_t* const dst = &sm.w[s][w][m * kRT + rt][0];
        const uint8_t* const src = wrow0[m][rt] + (size_t)b * 128;
        lds_load16(lds_addr(dst), src + wr_r * wrow + 16 * c0);
        lds_load16(lds_addr(dst + 1024), src + (8 + wr_r) * wrow + 16 * c1);
        if (!QS && even)
          lds_load4(lds_addr(&sm.ws[ps][w][m * kRT + rt][0]), srow0[m][rt] + c16 * srow + pair_off(b, wdd));
      }
    if (xw) {
      lds_load16(lds_addr(&sm.x[s][(8 * w) * kKB]), xsrc[0] + (size_t)b * kKB);
      lds_load16(lds_addr(&sm.x[s][(8 * w + 4) * kKB]), xsrc[1] + (size_t)b * kKB);
      if (even && lane < 32) lds_load4(lds_addr(&sm.xs[ps][w][0]), ssrc + pair_off(b, xdd));
    }
  };
  // this lane's weight scale bytes of block b, both halves
  auto read_scales = [&](int b, int (&sa)[2][M][kRT]) {
    const int ps = (b >> 1) & 1, d0 = 2 * (b & 1);
    // QS: dword of the block's first half in its 16 bytes, after the shift
    // of a load moved back (a one-block last pair: by 8 bytes)
    const int qd = d0 + max(0, 16 * (b >> 1) + 16 - (int)srow) / 4;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const uint32_t v = QS ? qslot[(m * kRT + rt) * 128 + 4 * (16 * ps + c16) + qd + j]
                                : sm.ws[ps][w][m * kRT + rt][16 * (d0 + j) + c16];
          sa[j][m][rt] = (int)((v >> (8 * kb)) & 0xFFu);
        }
  };
  auto compute = [&](int b, const int (&sa)[2][M][kRT]) {
    const int s = b % kStages, ps = (b >> 1) & 1, d0 = 2 * (b & 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 A[M][kRT];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) A[m][rt] = ld16(&sm.w[s][w][m * kRT + rt][woff(c16, 4 * j + kb)]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int t = 16 * nt + c16;
        const u32x4 lo = ld16(&sm.x[s][xoff(t, 8 * j + kb)]);
        const u32x4 hi = ld16(&sm.x[s][xoff(t, 8 * j + 4 + kb)]);
        const i32x8 B = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const int sb = (int)((sm.xs[ps][t / 8][8 * (d0 + j) + (t & 7)] >> (8 * kb)) & 0xFFu);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) {
            const u32x4 a4 = A[m][rt];
            const i32x8 Av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
            acc[m][rt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                Av, B, acc[m][rt][nt], 4 /* A: E2M1 */, 0 /* B: E4M3 */, 0, sa[j][m][rt], 0, sb);
          }
      }
    }
  };

  constexpr int kWEven = QS ? kWLoadsOdd : kWLoads;
  if constexpr (QS) issue_scales(0);
  for (int b = 0; b < kStages - 1 && b < NB; ++b) issue(b, b);
  for (int b = 0; b < NB; ++b) {
    // block b's loads (this wave's) are done once at most the loads of the
    // block issued after it are in flight (fewer for an odd block, which has
    // no scale loads); the barrier extends that to every wave's, and means
    // every wave is done computing block b - 1 (so also with the scale pair
    // slot that block b + 2 may load)
    if (b + 1 == NB)
      wait_then_barrier<0>();
    else if ((b + 1) & 1)
      xw ? wait_then_barrier<kWLoadsOdd + kXLoadsOdd>() : wait_then_barrier<kWLoadsOdd>();
    else
      xw ? wait_then_barrier<kWEven + kXLoads>() : wait_then_barrier<kWEven>();
    int sa[2][M][kRT];
    read_scales(b, sa);
    if (QS && (b & 3) == 3 && b + 1 < NB) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads above are done with the slot
      issue_scales((b + 1) / 4);
    }
    if (b + kStages - 1 < NB) issue(b + kStages - 1, (b + kStages - 1) % kStages);  // into b-1's slot
    compute(b, sa);
  }
  __syncthreads();  // the LDS is free for the caller (and its row table may change)
}

template <bool QS>
__global__ void __launch_bounds__(kThreads, 1) gemm13_mx_kernel(LayerArgs a) {
  const int tpe = (a.I + kRows13 - 1) / kRows13;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  // both loads in flight at once: the test reads both (off is never negative),
  // so the compiler cannot sink the second below it
  const int ne = a.counts[e], off = a.offsets[e];
  if (ne == 0 || off < 0) return;
  __shared__ SmemMx sm;
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
      gemm_pass_mx<QS, 2, 1, NT>(sm, wr, sr, wrow, srow, a.xq, a.xqs, nc, a.H, acc);
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
    switch ((nc + 15) / 16) {
      case 1: pass(IntC<1>{}); break;
      case 2: pass(IntC<2>{}); break;
      case 3: pass(IntC<3>{}); break;
      default: pass(IntC<4>{}); break;
    }
  }
}

template <bool QS>
__global__ void __launch_bounds__(kThreads, 1) gemm2_mx_kernel(LayerArgs a) {
  const int tpe = (a.H + kRows2 - 1) / kRows2;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  // both loads in flight at once: the test reads both (off is never negative),
  // so the compiler cannot sink the second below it
  const int ne = a.counts[e], off = a.offsets[e];
  if (ne == 0 || off < 0) return;
  __shared__ SmemMx sm;
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
      gemm_pass_mx<QS, 1, 2, NT>(sm, wr, sr, wrow, srow, a.hq, a.hqs, nc, a.I, acc);
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
      if (a.sal_part) saliency_tile<2, NT>(a, acc, act, sm.sal, off + c0, nc, rtile);
    };
    switch ((nc + 15) / 16) {
      case 1: pass(IntC<1>{}); break;
      case 2: pass(IntC<2>{}); break;
      case 3: pass(IntC<3>{}); break;
      default: pass(IntC<4>{}); break;
    }
  }
}

}  // namespace

namespace {
unsigned quant_blocks(int rows, int Kp) {
  return (unsigned)std::min<size_t>(((size_t)rows * Kp / 8 + 255) / 256, 4096);
}
static_assert(kRows2 == kSalRows, "saliency tiles are the w2 workgroup tiles");

}  // namespace

hipError_t launch_quant_mx8(const uint16_t* src, int rows, int K, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream) {
  hipLaunchKernelGGL(quant_mx8_kernel, dim3(quant_blocks(rows, K)), dim3(256), 0, stream, src, rows,
                     K, K, codes, scales);
  return hipGetLastError();
}

size_t mx8_padded(int K) { return (size_t)(K + kKB - 1) / kKB * kKB; }

// x is quantised first (stage 1 timing covers it with the w1/w3 GEMM), h after
// the w1/w3 GEMM (stage 2 covers it with the w2 GEMM).
hipError_t launch_prefill_mx8(const LayerArgs& a, hipStream_t stream) {
  const hipEvent_t* ev = a.ev;
  const dim3 blk(kThreads);
  const int P = a.T * a.k;
  const int Hp = (int)mx8_padded(a.H), Ip = (int)mx8_padded(a.I);
  const int t13 = a.E * ((a.I + kRows13 - 1) / kRows13), t2 = a.E * ((a.H + kRows2 - 1) / kRows2);
  launch_k(quant_mx8_kernel, dim3(quant_blocks(a.T, Hp)), dim3(256), 0, stream, ev_start(ev, 1),
           (hipEvent_t) nullptr, (const uint16_t*)a.x, a.T, a.H, Hp, a.xq, a.xqs);
  // four-block scale loads where K is whole blocks (at least two) and the scales 16-byte aligned
  auto qs = [](int K, const uint8_t* p, int64_t st) {
    return K % 256 == 0 && K >= 512 && (uintptr_t)p % 16 == 0 && st % 16 == 0;
  };
  const bool qs13 = qs(a.H, a.s1, a.stride[1]) && qs(a.H, a.s3, a.stride[3]);
  const bool qs2 = qs(a.I, a.s2, a.stride[5]);
  launch_k(qs13 ? gemm13_mx_kernel<true> : gemm13_mx_kernel<false>, dim3(xcd_grid(t13)), blk, 0,
           stream, (hipEvent_t) nullptr, ev_stop(ev, 1), a);
  launch_k(quant_mx8_kernel, dim3(quant_blocks(P, Ip)), dim3(256), 0, stream, ev_start(ev, 2),
           (hipEvent_t) nullptr, (const uint16_t*)a.h, P, a.I, Ip, a.hq, a.hqs);
  launch_k(qs2 ? gemm2_mx_kernel<true> : gemm2_mx_kernel<false>, dim3(xcd_grid(t2)), blk, 0, stream,
           (hipEvent_t) nullptr, ev_stop(ev, 2), a);
  return launch_combine(a, stream);
}

}  // namespace moe_fp4
