// Decode path: few tokens per step, so every selected expert is a GEMV that
// streams its packed weights once.  The DeepSeek-V4.1-Flash pages describe the
// cost of generating one token as reading every active expert weight once
// (ai-shiz.ru page, section on per-token arithmetic): this path is bound by HBM.
//
// One token (two launches a step):
//   gemv13_one_kernel  a persistent grid over the (chosen expert, row) units of
//                      w1/w3, taken in the ranking's order.  Wave 0 of every
//                      workgroup ranks the logits itself (the routing needs no
//                      launch of its own) and workgroup 0 publishes the
//                      result.  Half a wave reads the w1 row and half the w3
//                      row of a unit; FP4 is decoded in registers
//                      (v_cvt_scalef32_pk_bf16_fp4) and dotted with x from LDS
//                      (v_dot2c_f32_bf16, bf16 products exact in fp32); two
//                      units are in flight per wave; h = bf16(silu(G) * U).
//                      Optionally the shared expert's w1/w3 rows and the
//                      layer's RMS pre-norm ride along.
//   gemv2_one_kernel   one workgroup per CU over rows of y; every (chosen
//                      expert, 32-input group) pair of a row belongs to one
//                      lane, which holds its h values and gate in registers;
//                      rows stream through a 4-deep ring, the wave reduces
//                      with DPP and the wave partials are added in a fixed
//                      order: no atomics, y is bitwise reproducible.
//                      Optionally the shared expert's w2 rows ride along.
// Two to fifteen tokens: gemv13_few_kernel (the same units for every
// (token, expert) pair, the token rows in LDS) and gemv2_one_kernel per token.
// Other small shapes of up to sixteen tokens (the MFMA kernels gemv13_kernel
// and gemv2_combine_kernel): the token rows become the 16 columns of a
// 16x16x32 bf16 MFMA whose other operand is 16 weight rows decoded in
// registers; waves split the inputs (split-K) and meet in LDS.
#include <algorithm>
#include <mutex>
#include <vector>

#include "device_common.h"
#include "kernels.h"
#include "shared_gemv.h"
#include "topk.h"

namespace moe_fp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kBPW = 5;  // MFMA path: weight blocks (4 scale groups each) per wave in one batch
constexpr int kEB = 6;   // MFMA path: experts whose w2 loads are in flight together
constexpr int kB2 = 3;   // MFMA path: w2 blocks per wave and expert (I <= 8 * 3 * 128)
constexpr int kFusedVPL = 8;  // one-token routing inside the w1/w3 kernel: logits per lane (E <= 512)

__host__ __device__ constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DInfo {
  int e, off, ne;
};

__device__ __forceinline__ DInfo load_dinfo(const int32_t* dinfo, int d) {
  const u32x4 v = ld16(dinfo + 4 * d);
  return DInfo{(int)v[0], (int)v[1], (int)v[2]};
}

// =========================================================================== MFMA path
size_t lds13_bytes(int T, int H) {
  return align256((size_t)T * (H + 8) * 2) + (size_t)kWaves * 2 * 16 * 16 * 4;
}
size_t lds2_bytes(int P, int I) {
  return align256((size_t)P * (I + 8) * 2) + (size_t)kWaves * P * 16 * 4;
}

// G and U for 16 rows of one expert's w1/w3 and its (at most 16) tokens.
__global__ void __launch_bounds__(kThreads) gemv13_kernel(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const DInfo di = load_dinfo(a.dinfo, blockIdx.y);
  if (di.e < 0) return;
  const int e = di.e, off = di.off, ne = di.ne;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int c16 = lane & 15;  // A row (weight row) / B column (token) of this lane
  const int kb = lane >> 4;   // k-slot: which of the block's 4 scale groups
  const int r0 = blockIdx.x * 16;
  const int H = a.H, NG = H / 32, NB = (NG + 3) / 4;
  const int b0 = w * NB / kWaves, b1 = (w + 1) * NB / kWaves;
  const int XS = H + 8;  // LDS row stride (bf16): consecutive rows 4 banks apart
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + align256((size_t)a.T * XS * 2));

  const size_t wrow = (size_t)H / 2, srow = (size_t)H / 32;
  const uint8_t* w1r = a.w1 + (size_t)e * a.stride[0] + (size_t)(r0 + c16) * wrow;
  const uint8_t* s1r = a.s1 + (size_t)e * a.stride[1] + (size_t)(r0 + c16) * srow;
  const uint8_t* w3r = a.w3 + (size_t)e * a.stride[2] + (size_t)(r0 + c16) * wrow;
  const uint8_t* s3r = a.s3 + (size_t)e * a.stride[3] + (size_t)(r0 + c16) * srow;
  const u32x4 z4 = zero4();

  u32x4 q1[kBPW], q3[kBPW];
  uint32_t e1[kBPW], e3[kBPW];
  // Loads are unconditional, from an address that is always valid (group 0
  // when out of range), and zeroed afterwards: with no branches around them
  // all of them are in flight together and each wait is for the oldest.
  auto load = [&](int bb) {
#pragma unroll
    for (int j = 0; j < kBPW; ++j) {
      const int g = 4 * (bb + j) + kb;
      const bool ok = bb + j < b1 && g < NG;
      const int gg = ok ? g : 0;
      q1[j] = sel4(ok, ld16(w1r + (size_t)gg * 16));
      q3[j] = sel4(ok, ld16(w3r + (size_t)gg * 16));
      const uint32_t x1 = s1r[gg], x3 = s3r[gg];
      e1[j] = ok ? x1 : 0u;
      e3[j] = ok ? x3 : 0u;
    }
  };
  f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int bb) {
#pragma unroll
    for (int j = 0; j < kBPW; ++j) {
      if (bb + j < b1) {
        const int g = 4 * (bb + j) + kb;
        const bool bv = c16 < ne && g < NG;
        const float sc1 = ue8m0_to_f32(e1[j]), sc3 = ue8m0_to_f32(e3[j]);
        const uint16_t* xr = xs + c16 * XS + g * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 A1 = fp4x8_to_bf16x8(q1[j][i], sc1);
          const bf16x8 A3 = fp4x8_to_bf16x8(q3[j][i], sc3);
          const bf16x8 B = as_bf16x8(bv ? ld16(xr + 8 * i) : z4);
          acc1 = mfma16x16x32(A1, B, acc1);
          acc3 = mfma16x16x32(A3, B, acc3);
        }
      }
    }
  };

  load(b0);
  // x rows of this expert's tokens (sorted order) into LDS
  const int cpr = H / 8;  // 16-byte chunks per row
  for (int i = tid; i < ne * cpr; i += kThreads) {
    const int n = i / cpr, c = i - n * cpr;
    const int t = a.sorted_pairs[off + n] / a.k;
    st16(xs + n * XS + c * 8, ld16(a.x + (size_t)t * H + c * 8));
  }
  lds_barrier();
  compute(b0);
  for (int bb = b0 + kBPW; bb < b1; bb += kBPW) {
    load(bb);
    compute(bb);
  }

  // D[i][j]: i = weight row 4*kb + q, j = token c16
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    red[((w * 2 + 0) * 16 + 4 * kb + q) * 16 + c16] = acc1[q];
    red[((w * 2 + 1) * 16 + 4 * kb + q) * 16 + c16] = acc3[q];
  }
  lds_barrier();
  if (tid < 256) {
    const int i = tid & 15, j = tid >> 4;
    if (j < ne) {
      float G = 0.f, U = 0.f;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        G += red[((q * 2 + 0) * 16 + i) * 16 + j];
        U += red[((q * 2 + 1) * 16 + i) * 16 + j];
      }
      a.h[(size_t)(off + j) * a.I + r0 + i] = swiglu_bf16(G, U);
    }
  }
}

// y rows r0..r0+15 for every token: w2 for all distinct experts, then the
// gate-weighted combine.  part[w][slot][i] holds wave w's partial of Y_slot[r0+i].
__global__ void __launch_bounds__(kThreads) gemv2_combine_kernel(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int P = a.T * a.k;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int c16 = lane & 15, kb = lane >> 4;
  const int r0 = blockIdx.x * 16;
  const int I = a.I, NG = I / 32, NB = (NG + 3) / 4;
  const int b0 = w * NB / kWaves, b1 = (w + 1) * NB / kWaves;
  const int IS = I + 8;
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
  float* part = reinterpret_cast<float*>(smem + align256((size_t)P * IS * 2));
  const size_t wrow = (size_t)I / 2, srow = (size_t)I / 32;
  const int nd = a.meta[0];
  const u32x4 z4 = zero4();

  u32x4 q[kEB][kB2];
  uint32_t sv[kEB][kB2];
  auto load = [&](int d0) {
#pragma unroll
    for (int de = 0; de < kEB; ++de) {
      const int d = d0 + de;
      const int e = a.dinfo[4 * (d < nd ? d : 0)];
      const uint8_t* w2r = a.w2 + (size_t)e * a.stride[4] + (size_t)(r0 + c16) * wrow;
      const uint8_t* s2r = a.s2 + (size_t)e * a.stride[5] + (size_t)(r0 + c16) * srow;
#pragma unroll
      for (int j = 0; j < kB2; ++j) {
        const int g = 4 * (b0 + j) + kb;
        const bool ok = d < nd && b0 + j < b1 && g < NG;
        const int gg = ok ? g : 0;
        q[de][j] = sel4(ok, ld16(w2r + (size_t)gg * 16));
        const uint32_t x = s2r[gg];
        sv[de][j] = ok ? x : 0u;
      }
    }
  };
  auto compute = [&](int d0) {
#pragma unroll
    for (int de = 0; de < kEB; ++de) {
      const int d = d0 + de;
      if (d < nd) {
        const DInfo di = load_dinfo(a.dinfo, d);
        const int off = di.off, ne = di.ne;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kB2; ++j) {
          if (b0 + j < b1) {
            const int g = 4 * (b0 + j) + kb;
            const bool bv = c16 < ne && g < NG;
            const float sc = ue8m0_to_f32(sv[de][j]);
            const uint16_t* hr = hs + (off + c16) * IS + g * 32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16x8 A = fp4x8_to_bf16x8(q[de][j][i], sc);
              const bf16x8 B = as_bf16x8(bv ? ld16(hr + 8 * i) : z4);
              acc = mfma16x16x32(A, B, acc);
            }
          }
        }
        if (c16 < ne) {
          float* dst = part + ((size_t)w * P + off + c16) * 16 + 4 * kb;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dst[qq] = acc[qq];
        }
      }
    }
  };

  load(0);
  // every h row of the step (sorted order) into LDS
  const int cpr = I / 8;
  for (int i = tid; i < P * cpr; i += kThreads) {
    const int n = i / cpr, c = i - n * cpr;
    st16(hs + n * IS + c * 8, ld16(a.h + (size_t)n * I + c * 8));
  }
  lds_barrier();
  compute(0);
  for (int d0 = kEB; d0 < nd; d0 += kEB) {
    load(d0);
    compute(d0);
  }
  lds_barrier();
  for (int idx = tid; idx < a.T * 16; idx += kThreads) {
    const int t = idx >> 4, i = idx & 15;
    float s = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int p = t * a.k + j;
      const int slot = a.pair_slot[p];
      float v = 0.f;
#pragma unroll
      for (int qq = 0; qq < kWaves; ++qq) v += part[((size_t)qq * P + slot) * 16 + i];
      s += a.gates[p] * v;
    }
    float* yp = a.y + (size_t)t * a.H + r0 + i;
    *yp = a.accumulate ? *yp + s : s;
  }
}

// =========================================================================== one-token path
// In the w1/w3 kernels half a wave reads a row (half-lane j the 32-input
// groups j + 32 i).  The token's activations sit in LDS (read per unit, 16 bytes per group and dword; in registers they
// would cost 48 VGPRs and the kernel measured 0.7 us slower at H = 5120); in
// the w2 kernel each lane keeps its 32 h values in registers.  The weights are the only HBM
// stream, and the inner loop is the FP4 decode (v_cvt_scalef32_pk_bf16_fp4)
// and the dot products (v_dot2c_f32_bf16, bf16 products exact in fp32).

constexpr int kOneMaxXG = 4;      // x groups per lane: H <= 64 * 32 * 4 (w1/w3 slots <= 8)
constexpr int kOneMaxPL = 2;      // (slot, group) pairs per lane in the w2 kernel
constexpr int kOneRowsMax = 64;   // w2 rows per workgroup
constexpr int kOneDP = 4;         // w2 rows in flight per wave (measured best of 2..12)

int one_xg(int H) { return (H / 32 + kWave - 1) / kWave; }
// 16-byte slots a lane takes of one w1 row and one w3 row together
int one_ns(int H) { return (2 * (H / 32) + kWave - 1) / kWave; }
int one_pl(int I, int k) {
  const int pw = (k * (I / 32) + kWaves - 1) / kWaves;
  return (pw + kWave - 1) / kWave;
}
bool one_token_fits(int H, int I, int k) {
  return one_xg(H) <= kOneMaxXG && one_pl(I, k) <= kOneMaxPL;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The one-token w1/w3 kernel's tables, in LDS.  Its units are taken in the
// ranking's order: the expert of rank j (largest logit first) is de_rank[j],
// and its rows of h go to sorted slot slot_of[j], the number of chosen ids
// below it (each chosen expert holds exactly one pair).  de_w lists the
// chosen experts by ascending id (slot order).
struct OneTables {
  int de_rank[kMaxK], slot_of[kMaxK], de_w[kMaxK];
};

// Wave 0 of each workgroup ranks the logits; after round j it stores rank j's
// expert, so the other waves can start on the first ranks while it ranks the
// rest.
struct OneRanking {
  WaveRanking<kFusedVPL> rk;
  int my_e = 0;
  float my_v = 0.f, v0 = 0.f;

  __device__ __forceinline__ void round(int j, int lane, OneTables& tb) {
    uint32_t m;
    const int e = (int)rk.next(m);
    const float v = key_value(m);
    if (j == 0) v0 = v;
    if (j == lane) {
      my_e = e;
      my_v = v;
      tb.de_rank[j] = e;
    }
  }

  // After the last round: the slots, the ascending table, and (workgroup 0)
  // the routing result with the gates.
  __device__ __forceinline__ void finish(const LayerArgs& a, int lane, OneTables& tb) {
    const int k = a.k;
    const int key = lane < k ? my_e : 0x7FFFFFFF;
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(key, i) < key ? 1 : 0;
    if (lane < k) {
      tb.slot_of[lane] = rank;
      tb.de_w[rank] = my_e;
    }
    if (blockIdx.x == 0) {
      const float my_g = rank_gate(my_v, v0, k);
      if (lane < k) {
        const RouteArgs& r = a.route;
        r.idx[lane] = my_e;
        r.gates[lane] = my_g;
        r.sorted_pairs[rank] = lane;
        r.pair_slot[lane] = rank;
        r.slot_gate[rank] = my_g;
        r.slot_tok[rank] = 0;
        r.dinfo[4 * rank + 0] = my_e;
        r.dinfo[4 * rank + 1] = rank;
        r.dinfo[4 * rank + 2] = 1;
        r.dinfo[4 * rank + 3] = 0;
      }
    }
  }
};

// Workgroup 0's counts and offsets of the fused routing (after a barrier that
// makes wave 0's table visible).
__device__ __forceinline__ void publish_counts(const LayerArgs& a, const int (&de)[kMaxK]) {
  const RouteArgs& r = a.route;
  const int k = a.k, E = a.E;
  for (int x = threadIdx.x; x < E; x += kThreads) {
    int below = 0;
    while (below < k && de[below] < x) ++below;
    r.counts[x] = (below < k && de[below] == x) ? 1 : 0;
    r.offsets[x] = below;
  }
  if (threadIdx.x == 0) {
    r.offsets[E] = k;
    r.meta[0] = k;
  }
}

// G and U for every (chosen expert, row) unit.  The grid is persistent (what
// is resident at once); wave w of the grid takes units w, w + W, w + 2W, ...
// and keeps the next unit's loads in flight while it computes the current one.
// A unit is one row of w1 and the same row of w3, read as NS = H / 1024 slots
// (rounded up) of 16-byte loads: lanes 0-31 read the w1 row and lanes 32-63
// the w3 row, slot i of half-lane j the 32-input group j + 32 i, so a load
// covers 512 contiguous bytes of each row and at H = 5120 no lane idles.  Each
// slot brings its group's scale byte; in the last slot, lanes past the row's
// end re-read its last group and take the zero group of x.  A lane's sum is
// G's part (lanes 0-31) or U's (lanes 32-63).
//
// SH: the shared expert's w1/w3 rows too (sh: M = 2, T = 1, K = H).  They need
// no routing, so they take the first two ring slots of waves 0 .. N_s - 1: the
// first slot's loads go out before the first barrier, once the loads of x and
// the logits issued ahead of them are back, and fill the time in which routed
// rows cannot be addressed yet.  A shared row is two units of the
// same shape: part 0 the w1 row, part 1 the w3 row, slot i of lane l the
// 16-byte chunk l + 64 i of FP8 codes (K / 16 = NS 64 chunks at most) and its
// scale byte.  The routed units take the remaining slots in order.  All loads
// are global loads with per-lane addresses, the same instructions for both
// kinds, so the waits of the ring stay exact.  A part's sum runs through its
// chunks in the order shared_gemv_row takes them (fp8_chunk_dot each, x from
// LDS); then the wave sums and swiglu_bf16: the shared expert's own bits.
template <int NS, bool SH>
__global__ void __launch_bounds__(kThreads) gemv13_one_kernel(LayerArgs a, SharedArgs sh) {
  __shared__ OneTables tb;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int H = a.H, I = a.I, CPR = H / 32;

  // The token's x in LDS as 16-byte chunks (group g, dword q at 4 g + q),
  // followed by one zero group.  A lane's groups past the row end load a
  // duplicate weight chunk (clamped to the last group) and read the zero
  // group of x, so they add exactly nothing.  The logits and a bf16 x are
  // loaded together at entry (the logits by wave 0 alone), and x is stored
  // to LDS while wave 0 ranks.
  __shared__ u32x4 xl[kOneMaxXG * kWave * 4 + 4];
  static_assert(kOneMaxXG * kWave * 4 <= 2 * kThreads, "x chunks per thread");
  float lv[kFusedVPL];
  if (a.fused_route && w == 0) wave_load_logits<kFusedVPL>(a.logits, a.E, lane, lv);
  const int nc = CPR * 4, c0 = tid, c1 = tid + kThreads;
  const int cc0 = c0 < nc ? c0 : 0, cc1 = c1 < nc ? c1 : 0;
  u32x4 xv0 = zero4(), xv1 = zero4();
  float4 xf[4];  // a fp32 input row: chunks c0 and c1 (the pre-norm's ownership)
  static_assert(kThreads == kNormThreads, "pre-norm chunk ownership");
  if (a.xf) {
    xf[0] = *reinterpret_cast<const float4*>(a.xf + 8 * cc0);
    xf[1] = *reinterpret_cast<const float4*>(a.xf + 8 * cc0 + 4);
    xf[2] = *reinterpret_cast<const float4*>(a.xf + 8 * cc1);
    xf[3] = *reinterpret_cast<const float4*>(a.xf + 8 * cc1 + 4);
  } else {
    xv0 = ld16(a.x + 8 * cc0);
    xv1 = ld16(a.x + 8 * cc1);
  }

  // Work of the grid: S shared rows (two units each, in ring slots 0 and 1 of
  // waves 0 .. S - 1) and k I routed units.  Routed unit ru is row ru % I of
  // the expert of rank ru / I.
  constexpr int SP = SH ? 2 : 0;
  const int S = SH ? sh.N : 0;
  const int nunits = a.k * I;
  const int nw = gridDim.x * kWaves, wid = blockIdx.x * kWaves + w;
  const int V = SP * S + nunits;
  const int F = wid < V ? (V - 1 - wid) / nw + 1 : 0;  // units of this wave
  const bool mine_sh = wid < S;                         // slots 0 and 1 are a shared row
  auto routed_index = [&](int f) {
    return wid + f * nw - (f < SP ? f : SP) * S - (f < SP ? (wid < S ? wid : S) : 0);
  };

  // Wave 0 ranks the logits while the other waves stage x.  The first units
  // of this workgroup's waves need only the first `early` ranks (one where
  // they are all rows of the top expert): wave 0 stores those, the barrier
  // that publishes x publishes them, every wave issues its first unit, and
  // wave 0 ranks the rest while those loads are in flight; a second barrier
  // publishes the remaining ranks and the slots.  (Every wave ranking for
  // itself kept the SIMDs busy for 3-4 us: 16 waves a CU running the same
  // wave-wide reductions.)
  const int wg_last = min((int)(blockIdx.x + 1) * kWaves, nw < V ? nw : V) - 1;
  const int first_routed = wg_last - S;  // largest routed index in this workgroup's slot 0
  const int early = first_routed >= 0 ? first_routed / I + 1 : 0;
  OneRanking rank;
  if (w == 0) {
    if (a.fused_route) {
      rank.rk.init(lv, a.E, lane);
      for (int j = 0; j < early; ++j) rank.round(j, lane, tb);
    } else if (lane < a.k) {
      const int e = a.dinfo[4 * lane];
      tb.de_rank[lane] = e;
      tb.slot_of[lane] = lane;
      tb.de_w[lane] = e;
    }
  }

  const int snc = SH ? sh.K / 16 : 1;  // a shared row's 16-byte chunks
  float shG = 0.f;  // a shared row's G part, carried from part 0 to part 1

  struct Unit {
    u32x4 q[NS];
    uint32_t s[NS];
  };
  // a routed unit: lanes 0-31 read the w1 row, lanes 32-63 the w3 row; slot i
  // of half-lane hl is group hl + 32 i.  Only the last slot can pass the row's
  // end (32 (NS - 1) < CPR): it alone is clamped, the others are a fixed step
  // from the lane's first chunk.  A shared part's lane l reads chunks l + 64 i,
  // likewise clamped in the last slot only (64 (NS - 1) < 2 CPR).
  const bool hi = lane >= kWave / 2;
  const int hl = lane & (kWave / 2 - 1);
  const int g_last = hl + kWave / 2 * (NS - 1);
  const int gc_last = g_last < CPR ? g_last : CPR - 1;
  const int c_last = lane + kWave * (NS - 1);
  const int cc_last = c_last < snc ? c_last : snc - 1;
  auto issue = [&](int f, Unit& B) {
    const bool is_sh = SH && f < SP && mine_sh;
    const int ru = routed_index(f), j = ru / I, r = ru - j * I;
    const int e = is_sh ? 0 : uniform(tb.de_rank[j]);  // a shared unit reads no routing
    const uint8_t* wrow = (hi ? a.w3 + (size_t)e * a.stride[2] : a.w1 + (size_t)e * a.stride[0]) +
                          (size_t)r * (H / 2);
    const uint8_t* srow = (hi ? a.s3 + (size_t)e * a.stride[3] : a.s1 + (size_t)e * a.stride[1]) +
                          (size_t)r * CPR;
    int w0 = hl * 16, s0 = hl, wstep = kWave / 2 * 16, wl = gc_last * 16, sl = gc_last;
    if (SH && is_sh) {  // one row of a shared part
      wrow = sh.w[f] + (size_t)wid * sh.K;
      srow = sh.s[f] + (size_t)(wid / 32) * (sh.K / 32);
      w0 = lane * 16;
      s0 = lane / 2;
      wstep = kWave * 16;
      wl = cc_last * 16;
      sl = cc_last / 2;
    }
    const uint8_t* wp = wrow + w0;
    const uint8_t* sp = srow + s0;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
      B.q[i] = ld16(wp + wstep * i);
      B.s[i] = sp[kWave / 2 * i];  // 32 groups (routed) or 64 chunks (shared) on
    }
    B.q[NS - 1] = ld16(wrow + wl);
    B.s[NS - 1] = srow[sl];
  };
  auto compute = [&](int f, const Unit& B) {
    if (SH && f < SP && mine_sh) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int c = lane + kWave * i;
        if (c < snc) {
          const u32x4 xc[2] = {xl[2 * c], xl[2 * c + 1]};
          acc = fp8_chunk_dot(B.q[i], B.s[i], xc, acc);
        }
      }
      if (f == 0) {
        shG = acc;
      } else {
        const float r0 = wave_sum_f32(shG), r1 = wave_sum_f32(acc);
        if (lane == 0) sh.h[wid] = swiglu_bf16(r0, r1);
      }
      return;
    }
    const int ru = routed_index(f), j = ru / I, r = ru - j * I;
    float acc = 0.f;  // G's part in lanes 0-31, U's in lanes 32-63
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int g = hl + kWave / 2 * i;
      const int xg = i < NS - 1 || g < CPR ? g : CPR;  // past the row: zero group
      const float c = ue8m0_to_f32(B.s[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = dot8_bf16(fp4x8_to_bf16x8(B.q[i][q], c), as_bf16x8(xl[4 * xg + q]), acc);
    }
    float G, U;
    wave_half_sums_f32(acc, G, U);
    if (lane == 0) a.h[(size_t)uniform(tb.slot_of[j]) * I + r] = swiglu_bf16(G, U);
  };

  Unit A, B;
  // a shared row's first part needs neither the ranking nor x: out before the
  // first barrier
  const bool first_now = SH && F > 0 && mine_sh;
  if (first_now) issue(0, A);
  __builtin_amdgcn_sched_barrier(0);
  if (a.xf) {
    // the layer's input is the pre-norm of the fp32 row xf, computed as
    // moe_fp4_prenorm_bf16 computes it (same ownership and order: same bits)
    __shared__ float wsum[kNormThreads / 64];
    float ss = 0.f;
    if (c0 < nc) ss = chunk_sumsq(xf[0], xf[1], ss);
    if (c1 < nc) ss = chunk_sumsq(xf[2], xf[3], ss);
    const float r = block_rms(ss, H, a.eps, wsum);
    xv0 = chunk_to_bf16(xf[0], xf[1], r);
    xv1 = chunk_to_bf16(xf[2], xf[3], r);
  }
  if (c0 < nc) xl[c0] = xv0;
  if (c1 < nc) xl[c1] = xv1;
  if (tid < 4) xl[nc + tid] = zero4();
  lds_barrier();
  if (F > 0 && !first_now) issue(0, A);
  __builtin_amdgcn_sched_barrier(0);
  if (a.fused_route) {
    if (w == 0) {
      for (int j = early; j < a.k; ++j) rank.round(j, lane, tb);
      rank.finish(a, lane, tb);
    }
    lds_barrier();
    if (blockIdx.x == 0) publish_counts(a, tb.de_w);
  }
  if (F == 0) return;

  // Two register buffers; the loop body has no conditional loads, so each wait
  // is for the older buffer only and the next unit stays in flight.  The
  // scheduling barriers keep the compiler from sinking a unit's loads below
  // the computation they are meant to overlap.
  int f = 0;
  for (; f + 2 < F; f += 2) {
    issue(f + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(f, A);
    issue(f + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(f + 1, B);
  }
  if (F - f == 2) {
    issue(f + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(f, A);
    compute(f + 1, B);
  } else {
    compute(f, A);
  }
}

// ---------------------------------------------------------------- a few tokens
// The one-token kernels generalised to 2 <= T <= kFewMaxT tokens (routing by
// the routing kernels, before).  w1/w3: a unit is one row r of w1 and w3 for
// one sorted slot s (a (token, expert) pair); unit u = r P + s, so the slots
// of an expert that several tokens chose are consecutive units, taken by
// neighbouring waves of one workgroup at the same time: the row is read from
// HBM once and from the caches for the other slots.  Every token's x row
// sits in LDS (followed by a zero group, as in the one-token kernel): with
// 8-wave workgroups (two a CU) while that takes at most 64 KB, else 16-wave
// workgroups (one a CU, up to 160 KB), so a CU holds 16 waves either way.
constexpr int kFewMaxT = 15;
constexpr size_t kFewLdsBig = 160 * 1024;

size_t few13_lds(int T, int H, int k) {
  return (size_t)T * (H / 32 * 4 + 4) * 16 + (size_t)2 * T * k * 4;
}

template <int NS, int NW>
__global__ void __launch_bounds__(NW * kWave) gemv13_few_kernel(LayerArgs a) {
  constexpr int kThreads = NW * kWave, kWaves = NW;
  extern __shared__ __align__(16) uint8_t fsm[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int T = a.T, P = T * a.k, H = a.H, I = a.I, CPR = H / 32;
  const int RS = CPR * 4 + 4;  // 16-byte chunks a token row, the zero group included
  u32x4* xl = reinterpret_cast<u32x4*>(fsm);
  int* tab_e = reinterpret_cast<int*>(fsm + (size_t)T * RS * 16);  // expert of each slot
  int* tab_x = tab_e + P;                                           // its token's row in xl

  // the slot table: record d (distinct expert) covers slots off .. off + ne - 1
  const int nrec = P < a.E ? P : a.E;
  if (tid < nrec) {
    const u32x4 rec = ld16(a.dinfo + 4 * tid);
    const int e = (int)rec[0], off = (int)rec[1], ne = (int)rec[2];
    if (e >= 0)
      for (int j = 0; j < ne; ++j) tab_e[off + j] = e;
  }
  if (tid < P) tab_x[tid] = a.slot_tok[tid] * RS;
  // x rows, 8 chunks a thread in flight at a time
  const int nx = T * CPR * 4;
  for (int c0 = tid; c0 < nx; c0 += 8 * kThreads) {
    u32x4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = min(c0 + q * kThreads, nx - 1), t = c / (CPR * 4);
      v[q] = ld16(a.x + (size_t)t * H + 8 * (c - t * CPR * 4));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = c0 + q * kThreads, t = c / (CPR * 4);
      if (c < nx) xl[t * RS + (c - t * CPR * 4)] = v[q];
    }
  }
  if (tid < 4 * T) xl[(tid >> 2) * RS + CPR * 4 + (tid & 3)] = zero4();
  lds_barrier();

  const int nunits = P * I;
  const int nw = gridDim.x * kWaves, wid = blockIdx.x * kWaves + w;
  const int F = wid < nunits ? (nunits - 1 - wid) / nw + 1 : 0;
  if (F == 0) return;

  // the one-token kernel's units: lanes 0-31 the w1 row, lanes 32-63 the w3
  // row, slot i of half-lane hl group hl + 32 i, only the last slot clamped
  struct Unit {
    u32x4 q[NS];
    uint32_t s[NS];
  };
  const bool hi = lane >= kWave / 2;
  const int hl = lane & (kWave / 2 - 1);
  const int g_last = hl + kWave / 2 * (NS - 1);
  const int gc_last = g_last < CPR ? g_last : CPR - 1;
  auto issue = [&](int f, Unit& B) {
    const int u = wid + f * nw, r = u / P, sl = u - r * P;
    const int e = uniform(tab_e[sl]);
    const uint8_t* wrow = (hi ? a.w3 + (size_t)e * a.stride[2] : a.w1 + (size_t)e * a.stride[0]) +
                          (size_t)r * (H / 2);
    const uint8_t* srow = (hi ? a.s3 + (size_t)e * a.stride[3] : a.s1 + (size_t)e * a.stride[1]) +
                          (size_t)r * CPR;
    const uint8_t* wp = wrow + hl * 16;
    const uint8_t* sp = srow + hl;
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
      B.q[i] = ld16(wp + kWave / 2 * 16 * i);
      B.s[i] = sp[kWave / 2 * i];
    }
    B.q[NS - 1] = ld16(wrow + gc_last * 16);
    B.s[NS - 1] = srow[gc_last];
  };
  auto compute = [&](int f, const Unit& B) {
    const int u = wid + f * nw, r = u / P, sl = u - r * P;
    const u32x4* xr = xl + uniform(tab_x[sl]);
    float acc = 0.f;  // G's part in lanes 0-31, U's in lanes 32-63
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int g = hl + kWave / 2 * i;
      const int xg = i < NS - 1 || g < CPR ? g : CPR;  // past the row: zero group
      const float c = ue8m0_to_f32(B.s[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = dot8_bf16(fp4x8_to_bf16x8(B.q[i][q], c), as_bf16x8(xr[4 * xg + q]), acc);
    }
    float G, U;
    wave_half_sums_f32(acc, G, U);
    if (lane == 0) a.h[(size_t)sl * I + r] = swiglu_bf16(G, U);
  };

  // the two-buffer loop of the one-token kernel
  Unit A, B;
  issue(0, A);
  int f = 0;
  for (; f + 2 < F; f += 2) {
    issue(f + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(f, A);
    issue(f + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(f + 1, B);
  }
  if (F - f == 2) {
    issue(f + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(f, A);
    compute(f + 1, B);
  } else {
    compute(f, A);
  }
}

// y rows [m0, m1) of this workgroup for one token: every (pair, group) of the
// token's k pairs is owned by one lane of one wave (its 32 h values held in
// registers), so each w2 row costs each wave NPL 16-byte loads per lane; the
// lane sums gate * (chunk . h), the wave reduces with DPP, and the 8 wave
// partials of a row are added in a fixed order.  No atomics: y is bitwise
// reproducible.  One token (FEW false): the pairs are the sorted slots of the
// fused routing.  A few tokens (FEW true): workgroup (row block, token t), the
// pairs t k .. t k + k - 1 through pair_slot; a row block's workgroups for all
// tokens sit on one XCD (grid x a multiple of 8), so the w2 rows of an expert
// that several tokens chose are read from HBM about once.
//
// SC > 0 (one token): the shared expert's w2 rows [m0, m1) too (sh: M = 1,
// SC chunks a lane covering its whole row).  Wave w takes rows m0 + w + 8 i,
// kShRows at a time; their loads (and those of the shared h) go out at entry
// beside the routed ones, and they are evaluated after the routed rows as
// shared_gemv_row evaluates them (fp8_chunk_dot per chunk, then the wave sum),
// then added to the routed result: y = routed + shared, the order of the
// routed layer followed by the shared expert accumulating into y.
constexpr int kShRows = 3;
constexpr int kShMaxChunks = 4;  // chunks a lane of a shared w2 row in this kernel (K <= 4096)

template <int NPL, bool FEW, int SC = 0>
__device__ __forceinline__ void gemv2_one_body(const LayerArgs& a, int bid, int nblk, int tok,
                                               const SharedArgs& sh = SharedArgs{}) {
  __shared__ float part[kWaves][kOneRowsMax];
  __shared__ float shr[SC > 0 ? kOneRowsMax : 1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int H = a.H, I = a.I, CPR = I / 32;
  const int NP = a.k * CPR;
  // Where a row's pairs fit one wave (NP <= 64, e.g. one GPU's 288 rows of each
  // expert: 6 x 9 pairs), each wave takes whole rows m0 + w, m0 + w + 8, ...
  // with all its pairs and a row's sum is its wave's; otherwise the pairs are
  // split over the 8 waves, every wave takes every row, and the 8 partials of
  // a row are added in wave order.
  const bool rw = NPL == 1 && NP <= kWave;
  const int PW = rw ? NP : (NP + kWaves - 1) / kWaves, pw0 = rw ? 0 : w * PW;
  const int R = (H + nblk - 1) / nblk, m0 = bid * R;
  const int m1 = min(H, m0 + R);
  const int r0 = rw ? m0 + w : m0, rs = rw ? kWaves : 1;  // this wave's first row and row step
  if (m0 >= H) return;  // whole workgroup

  const uint8_t* wp[NPL];
  const uint8_t* sp[NPL];
  float gt[NPL];
  bf16x8 Hv[NPL][4];
  const bool routed = NP > 0;  // none: the shared expert's rows alone
  if (routed) {
    int ev[NPL], sl[NPL], gg[NPL];
    u32x4 hr[NPL][4];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int p = pw0 + lane + kWave * j;
      const int pc = (lane + kWave * j < PW && p < NP) ? p : 0;
      const int jj = pc / CPR;
      gg[j] = pc - jj * CPR;
      if (FEW) {
        const int pr = tok * a.k + jj;
        sl[j] = a.pair_slot[pr];
        ev[j] = a.route.idx[pr];
        gt[j] = a.gates[pr];
      } else {
        sl[j] = jj;
        ev[j] = a.dinfo[4 * sl[j]];
        gt[j] = a.slot_gate[sl[j]];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) hr[j][q] = ld16(a.h + (size_t)sl[j] * I + gg[j] * 32 + 8 * q);
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int p = pw0 + lane + kWave * j;
      const bool ok = lane + kWave * j < PW && p < NP;
      wp[j] = a.w2 + (size_t)ev[j] * a.stride[4] + gg[j] * 16;
      sp[j] = a.s2 + (size_t)ev[j] * a.stride[5] + gg[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) Hv[j][q] = as_bf16x8(sel4(ok, hr[j][q]));
    }
  }

  // the shared rows' loads: weights of up to kShRows rows, and the shared h
  // chunks (the same for every row)
  constexpr int SCN = SC > 0 ? SC : 1;
  const int NCs = SC > 0 ? sh.K / 16 : 0;
  u32x4 sw[kShRows][SCN], sx[SCN][2];
  uint32_t ss[kShRows][SCN];
  int scc[SCN];
  auto sh_load = [&](int m_first) {
#pragma unroll
    for (int j = 0; j < SCN; ++j) {
      const int c = lane + kWave * j;
      scc[j] = c < NCs ? c : NCs - 1;
    }
#pragma unroll
    for (int i = 0; i < kShRows; ++i) {
      const int n = min(m_first + kWaves * i, m1 - 1);  // past the end: a row already loaded
#pragma unroll
      for (int j = 0; j < SCN; ++j) {
        sw[i][j] = ld16(sh.w[0] + (size_t)n * sh.K + (size_t)scc[j] * 16);
        ss[i][j] = sh.s[0][(n / 32) * (sh.K / 32) + scc[j] / 2];
      }
    }
  };
  if constexpr (SC > 0) {
#pragma unroll
    for (int j = 0; j < SCN; ++j) {
      const int c = lane + kWave * j;
      const int cc = c < NCs ? c : NCs - 1;
      sx[j][0] = ld16(sh.act + (size_t)cc * 16);
      sx[j][1] = ld16(sh.act + (size_t)cc * 16 + 8);
    }
    sh_load(m0 + w);
  }

  const size_t wrow = I / 2;
  u32x4 qb[kOneDP][NPL];
  uint32_t sb[kOneDP][NPL];
  auto load = [&](int b, int m) {
    const int mc = m < m1 ? m : m1 - 1;  // past the end: a row already loaded
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      qb[b][j] = ld16(wp[j] + (size_t)mc * wrow);
      sb[b][j] = sp[j][(size_t)mc * CPR];
    }
  };
  // loads complete in issue order: issue the ring in the order it is consumed
  if (routed) {
#pragma unroll
  for (int b = 0; b < kOneDP; ++b) {
    load(b, r0 + rs * b);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int m = r0; m < m1; m += rs * kOneDP) {
#pragma unroll
    for (int b = 0; b < kOneDP; ++b) {
      const int mb = m + rs * b;
      if (mb < m1) {
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const float sc = ue8m0_to_f32(sb[b][j]);
          float t = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) t = dot8_bf16(fp4x8_to_bf16x8(qb[b][j][q], sc), Hv[j][q], t);
          p += gt[j] * t;
        }
        p = wave_sum_f32(p);
        if (lane == 0) part[rw ? 0 : w][mb - m0] = p;
      }
      load(b, mb + rs * kOneDP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  }
  if constexpr (SC > 0) {
    // the shared rows of this wave, kShRows at a time (one batch at the real
    // shape: 20 rows a workgroup)
    for (int mb = m0 + w; mb < m1; mb += kWaves * kShRows) {
      if (mb != m0 + w) sh_load(mb);
#pragma unroll
      for (int i = 0; i < kShRows; ++i) {
        const int n = mb + kWaves * i;
        if (n < m1) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < SCN; ++j)
            if (lane + kWave * j < NCs) acc = fp8_chunk_dot(sw[i][j], ss[i][j], sx[j], acc);
          acc = wave_sum_f32(acc);
          if (lane == 0) shr[n - m0] = acc;
        }
      }
    }
  }
  lds_barrier();
  if (tid < m1 - m0) {
    float* yp = a.y + (size_t)tok * H + m0 + tid;
    float v;
    if (routed) {
      float s = 0.f;
      if (rw) {
        s += part[0][tid];
      } else {
#pragma unroll
        for (int q = 0; q < kWaves; ++q) s += part[q][tid];
      }
      v = a.accumulate ? *yp + s : s;
      if constexpr (SC > 0) v = v + shr[tid];
    } else if constexpr (SC > 0) {
      v = a.accumulate ? *yp + shr[tid] : shr[tid];  // the shared expert's own y
    } else {
      v = a.accumulate ? *yp : 0.f;
    }
    *yp = v;
  }
}

// Workgroup b of nb takes rows b R .. (b + 1) R - 1 of y (R = H / nb rounded up).
template <int NPL, bool FEW, int SC>
__global__ void __launch_bounds__(kThreads) gemv2_one_kernel(LayerArgs a, SharedArgs sh) {
  gemv2_one_body<NPL, FEW, SC>(a, blockIdx.x, gridDim.x, FEW ? (int)blockIdx.y : 0, sh);
}

// Workgroups of `kernel` (`threads` threads, `lds` bytes of dynamic LDS) that the
// current device holds at once, and its compute units.  Cached per (device,
// kernel, lds).
struct Residency {
  int wgs, cus;
};
Residency residency(const void* kernel, size_t lds, int threads = kThreads) {
  struct Entry {
    int dev;
    const void* kernel;
    size_t lds;
    int threads;
    Residency r;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Residency{0, 0};
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& x : cache)
      if (x.dev == dev && x.kernel == kernel && x.lds == lds && x.threads == threads) return x.r;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return Residency{0, 0};
  const Residency r{cus * per_cu, cus};
  std::lock_guard<std::mutex> lock(mu);
  cache.push_back(Entry{dev, kernel, lds, threads, r});
  return r;
}

// The one-token w1/w3 kernel for NS = H / 1024 (rounded up) slots and SH: its
// address, or its launch.
template <int NS, bool SH>
const void* k13_one() { return reinterpret_cast<const void*>(gemv13_one_kernel<NS, SH>); }

template <bool SH>
const void* k13_one_sh(int ns) {
  switch (ns) {
    case 1: return k13_one<1, SH>();
    case 2: return k13_one<2, SH>();
    case 3: return k13_one<3, SH>();
    case 4: return k13_one<4, SH>();
    case 5: return k13_one<5, SH>();
    case 6: return k13_one<6, SH>();
    case 7: return k13_one<7, SH>();
    default: return k13_one<8, SH>();
  }
}
template <bool SH>
void launch13_one(int ns, dim3 g, const LayerArgs& a, const SharedArgs& sh, hipStream_t stream) {
  const dim3 blk(kThreads);
  const hipEvent_t e0 = ev_start(a.ev, 1), e1 = ev_stop(a.ev, 1);
  switch (ns) {
    case 1: launch_k(gemv13_one_kernel<1, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 2: launch_k(gemv13_one_kernel<2, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 3: launch_k(gemv13_one_kernel<3, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 4: launch_k(gemv13_one_kernel<4, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 5: launch_k(gemv13_one_kernel<5, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 6: launch_k(gemv13_one_kernel<6, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    case 7: launch_k(gemv13_one_kernel<7, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
    default: launch_k(gemv13_one_kernel<8, SH>, g, blk, 0, stream, e0, e1, a, sh); break;
  }
}
template <int NPL, bool FEW, int SC>
void launch2_one(dim3 g, const LayerArgs& a, const SharedArgs& sh, hipStream_t stream) {
  launch_k(gemv2_one_kernel<NPL, FEW, SC>, g, dim3(kThreads), 0, stream, ev_start(a.ev, 2),
           ev_stop(a.ev, 2), a, sh);
}

// Chunks a lane of a shared-expert row of K inputs takes when the one-token
// launches carry it (the whole row in one round, at most maxc), or 0 when they
// cannot.
int shared_one_chunks(int K, int maxc) {
  const int ncl = (K / 16 + kWave - 1) / kWave;
  return ncl <= maxc ? ncl : 0;
}
// A shared w1/w3 row of K = H inputs fits two units of the w1/w3 kernel (one
// a matrix, a chunk a slot).
bool shared13_fits(int K, int H) { return K == H && shared_one_chunks(K, one_ns(H)) > 0; }

hipError_t launch_one(const LayerArgs& a, hipStream_t stream) {
  const int ns = one_ns(a.H), npl = one_pl(a.I, a.k);
  const SharedArgs none{};
  // With a shared expert (a.shared13, a.shared2) its rows ride in the two
  // launches when they fit: a w1/w3 row in two units, a w2 row in one round
  // of kShMaxChunks chunks a lane, one wave for every shared w1/w3 row and
  // every wave below the row count owning ring slots 0 and 1 (W <= S + routed
  // units).  Otherwise the shared expert's own kernels run after the layer.
  bool shared = a.shared13 != nullptr;
  const int routed = a.k * a.I, S = shared ? a.shared13->N : 0;
  int sc2 = shared ? shared_one_chunks(a.shared2->K, kShMaxChunks) : 0;
  bool carry = shared && shared13_fits(a.shared13->K, a.H) && sc2 > 0;
  Residency res{};
  int want = 0;
  if (carry) {
    res = residency(k13_one_sh<true>(ns), 0);
    want = std::min(res.wgs, (S + routed) / kWaves);
    carry = res.wgs > 0 && want * kWaves >= S;
  }
  if (shared && !carry) {
    LayerArgs b = a;
    b.shared13 = b.shared2 = nullptr;
    const hipError_t e = launch_one(b, stream);
    if (e != hipSuccess) return e;
    const SharedArgs &s13 = *a.shared13, &s2 = *a.shared2;
    const uint8_t* const t[6] = {s13.w[0], s13.s[0], s13.w[1], s13.s[1], s2.w[0], s2.s[0]};
    return launch_shared(s13.act, t, 1, s13.K, s13.N, a.y, 1, s13.h, stream);
  }
  // w1/w3: as many workgroups as are resident
  if (!carry) {
    res = residency(k13_one_sh<false>(ns), 0);
    want = std::min(res.wgs, (routed + kWaves - 1) / kWaves);
  }
  if (res.wgs <= 0) return hipErrorInvalidValue;
  const dim3 g13(std::max(1, want));
  if (shared)
    launch13_one<true>(ns, g13, a, *a.shared13, stream);
  else
    launch13_one<false>(ns, g13, a, none, stream);
  // w2: one workgroup per compute unit, at most kOneRowsMax rows each
  const int n2 = std::max((a.H + kOneRowsMax - 1) / kOneRowsMax, std::min(a.H, res.cus));
  const dim3 g2(n2);
  if (!shared) {
    if (npl == 1)
      launch2_one<1, false, 0>(g2, a, none, stream);
    else
      launch2_one<2, false, 0>(g2, a, none, stream);
  } else if (sc2 <= 3) {
    if (npl == 1)
      launch2_one<1, false, 3>(g2, a, *a.shared2, stream);
    else
      launch2_one<2, false, 3>(g2, a, *a.shared2, stream);
  } else {
    if (npl == 1)
      launch2_one<1, false, kShMaxChunks>(g2, a, *a.shared2, stream);
    else
      launch2_one<2, false, kShMaxChunks>(g2, a, *a.shared2, stream);
  }
  return hipSuccess;
}

bool few_fits(int T, int H, int I, int k) {
  return T >= 2 && T <= kFewMaxT && one_token_fits(H, I, k) && few13_lds(T, H, k) <= kFewLdsBig;
}

// The few-token w1/w3 kernel for NS slots and the workgroup size the LDS
// allows; the dynamic LDS limit is raised once per (device, kernel).
template <int NS, int NW>
const void* k13_few() { return reinterpret_cast<const void*>(gemv13_few_kernel<NS, NW>); }
template <int NW>
hipError_t launch_few13(const LayerArgs& a, int ns, size_t lds, hipStream_t stream, int& cus) {
  const void* k = ns == 1   ? k13_few<1, NW>()
                  : ns == 2 ? k13_few<2, NW>()
                  : ns == 3 ? k13_few<3, NW>()
                  : ns == 4 ? k13_few<4, NW>()
                  : ns == 5 ? k13_few<5, NW>()
                  : ns == 6 ? k13_few<6, NW>()
                  : ns == 7 ? k13_few<7, NW>()
                            : k13_few<8, NW>();
  if (lds > kDecodeLds) {
    static std::mutex mu;
    static std::vector<std::pair<int, const void*>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(mu);
    if (std::find(done.begin(), done.end(), std::make_pair(dev, k)) == done.end()) {
      const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFewLdsBig);
      if (e != hipSuccess) return e;
      done.emplace_back(dev, k);
    }
  }
  const Residency res = residency(k, lds, NW * kWave);
  if (res.wgs <= 0) return hipErrorInvalidValue;
  cus = res.cus;
  const int units = a.T * a.k * a.I;
  const dim3 blk(NW * kWave), g(std::min(res.wgs, (units + NW - 1) / NW));
  const hipEvent_t e0 = ev_start(a.ev, 1), e1 = ev_stop(a.ev, 1);
  switch (ns) {
    case 1: launch_k(gemv13_few_kernel<1, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 2: launch_k(gemv13_few_kernel<2, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 3: launch_k(gemv13_few_kernel<3, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 4: launch_k(gemv13_few_kernel<4, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 5: launch_k(gemv13_few_kernel<5, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 6: launch_k(gemv13_few_kernel<6, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 7: launch_k(gemv13_few_kernel<7, NW>, g, blk, lds, stream, e0, e1, a); break;
    default: launch_k(gemv13_few_kernel<8, NW>, g, blk, lds, stream, e0, e1, a); break;
  }
  return hipSuccess;
}

hipError_t launch_few(const LayerArgs& a, hipStream_t stream) {
  const int ns = one_ns(a.H), npl = one_pl(a.I, a.k);
  const size_t lds = few13_lds(a.T, a.H, a.k);
  int cus = 0;
  const hipError_t e13 = lds <= kDecodeLds ? launch_few13<kWaves>(a, ns, lds, stream, cus)
                                           : launch_few13<2 * kWaves>(a, ns, lds, stream, cus);
  if (e13 != hipSuccess) return e13;
  // w2: (row block, token) workgroups; the row-block count a multiple of 8 so
  // that a row block's workgroups share an XCD
  int n2 = std::max((a.H + kOneRowsMax - 1) / kOneRowsMax, std::min(a.H, cus));
  n2 = (n2 + 7) / 8 * 8;
  const dim3 g2(n2, a.T);
  const SharedArgs none{};
  if (npl == 1)
    launch2_one<1, true, 0>(g2, a, none, stream);
  else
    launch2_one<2, true, 0>(g2, a, none, stream);
  return hipSuccess;
}

}  // namespace

bool decode_fits(int T, int H, int I, int k) {
  if (T == 1 && one_token_fits(H, I, k)) return true;
  if (few_fits(T, H, I, k)) return true;
  const int P = T * k;
  return T <= kDecodeMaxTokens && I <= kWaves * kB2 * 128 && lds13_bytes(T, H) <= kDecodeLds &&
         lds2_bytes(P, I) <= kDecodeLds;
}

bool decode_one_token(int T, int H, int I, int k) { return T == 1 && one_token_fits(H, I, k); }


int decode_family(int T, int H, int I, int k) {
  if (T == 1 && one_token_fits(H, I, k)) return 1;
  return few_fits(T, H, I, k) ? 2 : 3;
}

bool decode_fuses_route(int T, int H, int I, int E, int k) {
  return T == 1 && one_token_fits(H, I, k) && E <= kFusedVPL * kWave;
}

hipError_t launch_shared_one(const uint16_t* x, const uint8_t* const w[6], int H, int I, float* y,
                             int accumulate, uint16_t* h, hipStream_t stream, bool& done) {
  done = false;
  // the one-token kernels with no routed expert: a wave for every shared
  // w1/w3 row (two units: the w1 row, then the w3 row), the w2 rows in one
  // round of at most kShMaxChunks chunks a lane
  if (!one_token_fits(H, 32, 1) || !shared13_fits(H, H)) return hipSuccess;
  const int sc2 = shared_one_chunks(I, kShMaxChunks);
  if (sc2 == 0) return hipSuccess;
  const int ns = one_ns(H);
  const Residency res = residency(k13_one_sh<true>(ns), 0);
  if (res.wgs <= 0 || I % kWaves != 0 || I / kWaves > res.wgs) return hipSuccess;
  LayerArgs a{};
  a.H = H;
  a.I = 32;  // no routed unit reads it
  a.k = 0;
  a.E = 1;
  a.x = x;
  a.y = y;
  a.accumulate = accumulate;
  SharedArgs s13{};
  s13.act = x;
  s13.w[0] = w[0]; s13.s[0] = w[1]; s13.w[1] = w[2]; s13.s[1] = w[3];
  s13.N = I; s13.K = H; s13.T = 1; s13.h = h;
  SharedArgs s2{};
  s2.act = h;
  s2.w[0] = w[4]; s2.s[0] = w[5];
  s2.N = H; s2.K = I; s2.T = 1; s2.y = y; s2.accumulate = accumulate;
  launch13_one<true>(ns, dim3(I / kWaves), a, s13, stream);
  const dim3 g2(std::max((H + kOneRowsMax - 1) / kOneRowsMax, std::min(H, res.cus)));
  if (sc2 <= 3)
    launch2_one<1, false, 3>(g2, a, s2, stream);
  else
    launch2_one<1, false, kShMaxChunks>(g2, a, s2, stream);
  done = true;
  return hipGetLastError();
}

hipError_t launch_decode(const LayerArgs& a, hipStream_t stream) {
  const int P = a.T * a.k;
  const hipEvent_t* ev = a.ev;
  if (a.T == 1 && one_token_fits(a.H, a.I, a.k)) {
    const hipError_t e = launch_one(a, stream);
    if (e != hipSuccess) return e;
  } else if (few_fits(a.T, a.H, a.I, a.k)) {
    const hipError_t e = launch_few(a, stream);
    if (e != hipSuccess) return e;
  } else {
    const int dmax = P < a.E ? P : a.E;  // distinct experts can not exceed either
    const dim3 blk(kThreads), g13(a.I / 16, dmax), g2(a.H / 16);
    launch_k(gemv13_kernel, g13, blk, lds13_bytes(a.T, a.H), stream, ev_start(ev, 1), ev_stop(ev, 1),
             a);
    launch_k(gemv2_combine_kernel, g2, blk, lds2_bytes(P, a.I), stream, ev_start(ev, 2),
             ev_stop(ev, 2), a);
  }
  ev_empty(ev, 3, stream);  // the combine is part of the w2 kernels here
  return hipGetLastError();
}

}  // namespace moe_fp4
