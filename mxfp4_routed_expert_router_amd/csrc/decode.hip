// Decode path: few tokens per step, so every selected expert is a GEMV that
// streams its packed weights once.  The DeepSeek-V4.1-Flash pages describe the
// cost of generating one token as reading every active expert weight once
// (ai-shiz.ru page, section on per-token arithmetic): this path is bound by HBM.
//
// One or two tokens (the row-contiguous kernels):
//   gemv13_dot  one workgroup per (distinct expert, 16 rows of w1/w3); each of
//               its 8 waves owns two whole rows, so lane l of load j reads
//               16-byte chunk 64*j + l of those rows: one contiguous 1 KB per
//               instruction, the scale bytes contiguous too.  A lane decodes its
//               chunk (one UE8M0 group, 32 inputs) and takes the dot product with
//               the matching inputs of x from LDS on the VALU (v_dot2c_f32_bf16,
//               bf16 products exact in fp32); a row's sum is a fixed-order DPP
//               reduction, and h = bf16(silu(G) * U).  With one token the kernel
//               also ranks the logits itself (every workgroup, redundantly) and
//               one workgroup publishes the routing result, so a decode step is
//               two launches.
//   gemv2_dot   one workgroup per 16 rows of w2 covering every distinct expert;
//               each wave owns two rows and sums gate * (w2 row . h row) over the
//               experts chunk by chunk, then reduces over the wave: the combine
//               needs no atomics and y is bitwise reproducible.
// Three to sixteen tokens (the MFMA kernels): the token rows become the 16
// columns of a 16x16x32 bf16 MFMA whose other operand is 16 weight rows decoded
// in registers; waves split the inputs (split-K) and meet in LDS.
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
// Lane l of a wave owns the 32-input groups g = l + 64 i (i < NXG) of the rows
// it reads.  In the w1/w3 kernel the token's activations sit in LDS (read per
// unit, 16 bytes per group and dword; in registers they would cost 48 VGPRs
// and the kernel measured 0.7 us slower at H = 5120); in the w2 kernel each
// lane keeps its 32 h values in registers.  The weights are the only HBM
// stream, and the inner loop is the FP4 decode (v_cvt_scalef32_pk_bf16_fp4)
// and the dot products (v_dot2c_f32_bf16, bf16 products exact in fp32).

constexpr int kOneMaxXG = 4;      // x groups per lane: H <= 64 * 32 * 4
constexpr int kOneMaxPL = 2;      // (slot, group) pairs per lane in the w2 kernel
constexpr int kOneRowsMax = 64;   // w2 rows per workgroup
constexpr int kOneDP = 4;         // w2 rows in flight per wave (measured best of 2..12)

int one_xg(int H) { return (H / 32 + kWave - 1) / kWave; }
int one_pl(int I, int k) {
  const int pw = (k * (I / 32) + kWaves - 1) / kWaves;
  return (pw + kWave - 1) / kWave;
}
bool one_token_fits(int H, int I, int k) {
  return one_xg(H) <= kOneMaxXG && one_pl(I, k) <= kOneMaxPL;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The k chosen experts of the token by ascending id (slot d), as wave w sees
// them in its own row of the table.  With the routing fused, every wave ranks
// the logits itself (the same computation, so the same result in every wave):
// it can then issue its first unit's loads without waiting for any other wave.
// Each chosen expert holds exactly one pair, so the expert of rank j sits in
// sorted slot (number of chosen ids below it).  Wave 0 of workgroup 0
// publishes the routing result.
__device__ __forceinline__ void route_one_wave(const LayerArgs& a, const float (&lv)[kFusedVPL],
                                               int (&de)[kMaxK]) {
  const int lane = threadIdx.x & (kWave - 1), k = a.k;
  int my_e;
  float my_g;
  wave_topk_vals<kFusedVPL>(lv, a.E, k, lane, my_e, my_g);
  const int key = lane < k ? my_e : 0x7FFFFFFF;
  int rank = 0;
  for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(key, i) < key ? 1 : 0;
  if (lane < k) de[rank] = my_e;
  if (blockIdx.x == 0 && threadIdx.x < kWave && lane < k) {
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
// A unit is one row of w1 and the same row of w3: NXG load instructions each
// (lane l reads the 16-byte chunk of group l + 64 i), plus the scale bytes.
template <int NXG>
__global__ void __launch_bounds__(kThreads) gemv13_one_kernel(LayerArgs a) {
  __shared__ int de_w[kMaxK];  // the chosen experts in ascending order
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
  // Wave 0 ranks the logits while the other waves stage x; the barrier
  // below publishes both.  (Every wave ranking for itself, which needs no
  // barrier before its first loads, kept the SIMDs busy for 3-4 us: 16 waves
  // a CU running the same six wave-wide reductions.)
  if (w == 0) {
    if (a.fused_route)
      route_one_wave(a, lv, de_w);
    else if (lane < a.k)
      de_w[lane] = a.dinfo[4 * lane];
  }

  int gc[NXG], xo[NXG];
#pragma unroll
  for (int i = 0; i < NXG; ++i) {
    const int g = lane + kWave * i;
    gc[i] = g < CPR ? g : CPR - 1;
    xo[i] = g < CPR ? 4 * g : 4 * CPR;
  }
  const int nunits = a.k * I;
  const int nw = gridDim.x * kWaves, wid = blockIdx.x * kWaves + w;
  const int F = wid < nunits ? (nunits - 1 - wid) / nw + 1 : 0;  // units of this wave
  const int wbytes = I * (H / 2), sbytes = I * CPR;

  struct Unit {
    u32x4 q1[NXG], q3[NXG];
    uint32_t s1[NXG], s3[NXG];
  };
  auto issue = [&](int f, Unit& B) {
    const int u = wid + f * nw, d = u / I, r = u - d * I;
    const int e = uniform(de_w[d]);
    const __amdgpu_buffer_rsrc_t r1 = rsrc(a.w1 + (size_t)e * a.stride[0], wbytes);
    const __amdgpu_buffer_rsrc_t r3 = rsrc(a.w3 + (size_t)e * a.stride[2], wbytes);
    const __amdgpu_buffer_rsrc_t q1 = rsrc(a.s1 + (size_t)e * a.stride[1], sbytes);
    const __amdgpu_buffer_rsrc_t q3 = rsrc(a.s3 + (size_t)e * a.stride[3], sbytes);
    const int ow = r * (H / 2), os = r * CPR;
#pragma unroll
    for (int i = 0; i < NXG; ++i) {
      B.q1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, gc[i] * 16, ow, 0));
      B.q3[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r3, gc[i] * 16, ow, 0));
      B.s1[i] = __builtin_amdgcn_raw_buffer_load_b8(q1, gc[i], os, 0);
      B.s3[i] = __builtin_amdgcn_raw_buffer_load_b8(q3, gc[i], os, 0);
    }
  };
  auto compute = [&](int f, const Unit& B) {
    const int u = wid + f * nw, d = u / I, r = u - d * I;
    float G = 0.f, U = 0.f;
#pragma unroll
    for (int i = 0; i < NXG; ++i) {
      const float c1 = ue8m0_to_f32(B.s1[i]), c3 = ue8m0_to_f32(B.s3[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 xq = as_bf16x8(xl[xo[i] + q]);
        G = dot8_bf16(fp4x8_to_bf16x8(B.q1[i][q], c1), xq, G);
        U = dot8_bf16(fp4x8_to_bf16x8(B.q3[i][q], c3), xq, U);
      }
    }
    G = wave_sum_f32(G);
    U = wave_sum_f32(U);
    if (lane == 0) a.h[(size_t)d * I + r] = swiglu_bf16(G, U);
  };

  Unit A, B;
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
  if (a.fused_route && blockIdx.x == 0) publish_counts(a, de_w);
  if (F == 0) return;
  issue(0, A);
  __builtin_amdgcn_sched_barrier(0);

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

template <int NXG, int NW>
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

  int gc[NXG], xo[NXG];
#pragma unroll
  for (int i = 0; i < NXG; ++i) {
    const int g = lane + kWave * i;
    gc[i] = g < CPR ? g : CPR - 1;
    xo[i] = g < CPR ? 4 * g : 4 * CPR;
  }
  const int nunits = P * I;
  const int nw = gridDim.x * kWaves, wid = blockIdx.x * kWaves + w;
  const int F = wid < nunits ? (nunits - 1 - wid) / nw + 1 : 0;
  if (F == 0) return;
  const int wbytes = I * (H / 2), sbytes = I * CPR;

  struct Unit {
    u32x4 q1[NXG], q3[NXG];
    uint32_t s1[NXG], s3[NXG];
  };
  auto issue = [&](int f, Unit& B) {
    const int u = wid + f * nw, r = u / P, sl = u - r * P;
    const int e = uniform(tab_e[sl]);
    const __amdgpu_buffer_rsrc_t r1 = rsrc(a.w1 + (size_t)e * a.stride[0], wbytes);
    const __amdgpu_buffer_rsrc_t r3 = rsrc(a.w3 + (size_t)e * a.stride[2], wbytes);
    const __amdgpu_buffer_rsrc_t q1 = rsrc(a.s1 + (size_t)e * a.stride[1], sbytes);
    const __amdgpu_buffer_rsrc_t q3 = rsrc(a.s3 + (size_t)e * a.stride[3], sbytes);
    const int ow = r * (H / 2), os = r * CPR;
#pragma unroll
    for (int i = 0; i < NXG; ++i) {
      B.q1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, gc[i] * 16, ow, 0));
      B.q3[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r3, gc[i] * 16, ow, 0));
      B.s1[i] = __builtin_amdgcn_raw_buffer_load_b8(q1, gc[i], os, 0);
      B.s3[i] = __builtin_amdgcn_raw_buffer_load_b8(q3, gc[i], os, 0);
    }
  };
  auto compute = [&](int f, const Unit& B) {
    const int u = wid + f * nw, r = u / P, sl = u - r * P;
    const u32x4* xr = xl + uniform(tab_x[sl]);
    float G = 0.f, U = 0.f;
#pragma unroll
    for (int i = 0; i < NXG; ++i) {
      const float c1 = ue8m0_to_f32(B.s1[i]), c3 = ue8m0_to_f32(B.s3[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 xq = as_bf16x8(xr[xo[i] + q]);
        G = dot8_bf16(fp4x8_to_bf16x8(B.q1[i][q], c1), xq, G);
        U = dot8_bf16(fp4x8_to_bf16x8(B.q3[i][q], c3), xq, U);
      }
    }
    G = wave_sum_f32(G);
    U = wave_sum_f32(U);
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
template <int NPL, bool FEW>
__device__ __forceinline__ void gemv2_one_body(const LayerArgs& a, int bid, int nblk, int tok) {
  __shared__ float part[kWaves][kOneRowsMax];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = uniform(tid / kWave);
  const int H = a.H, I = a.I, CPR = I / 32;
  const int NP = a.k * CPR, PW = (NP + kWaves - 1) / kWaves;
  const int R = (H + nblk - 1) / nblk, m0 = bid * R;
  const int m1 = min(H, m0 + R);
  if (m0 >= H) return;  // whole workgroup

  const uint8_t* wp[NPL];
  const uint8_t* sp[NPL];
  float gt[NPL];
  bf16x8 Hv[NPL][4];
  {
    int ev[NPL], sl[NPL], gg[NPL];
    u32x4 hr[NPL][4];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int p = w * PW + lane + kWave * j;
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
      const int p = w * PW + lane + kWave * j;
      const bool ok = lane + kWave * j < PW && p < NP;
      wp[j] = a.w2 + (size_t)ev[j] * a.stride[4] + gg[j] * 16;
      sp[j] = a.s2 + (size_t)ev[j] * a.stride[5] + gg[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) Hv[j][q] = as_bf16x8(sel4(ok, hr[j][q]));
    }
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
#pragma unroll
  for (int b = 0; b < kOneDP; ++b) {
    load(b, m0 + b);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int m = m0; m < m1; m += kOneDP) {
#pragma unroll
    for (int b = 0; b < kOneDP; ++b) {
      if (m + b < m1) {
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
        if (lane == 0) part[w][m + b - m0] = p;
      }
      load(b, m + b + kOneDP);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();
  if (tid < m1 - m0) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s += part[q][tid];
    float* yp = a.y + (size_t)tok * H + m0 + tid;
    *yp = a.accumulate ? *yp + s : s;
  }
}

// Workgroup b of nb takes rows b R .. (b + 1) R - 1 of y (R = H / nb rounded up).
template <int NPL, bool FEW>
__global__ void __launch_bounds__(kThreads) gemv2_one_kernel(LayerArgs a) {
  gemv2_one_body<NPL, FEW>(a, blockIdx.x, gridDim.x, FEW ? (int)blockIdx.y : 0);
}

// The one-token w2 (workgroups below n2, as gemv2_one_kernel) and, in the same
// launch, the shared expert's w1/w3 rows, one wave a row (the rest): those need
// only x, and the w2 workgroups, one a compute unit, leave most of each CU's
// waves free while their row loads are in flight.
template <int NPL, int SC>
__global__ void __launch_bounds__(kThreads) gemv2_one_shared_kernel(LayerArgs a, SharedArgs s,
                                                                     int n2) {
  if ((int)blockIdx.x < n2) {
    gemv2_one_body<NPL, false>(a, blockIdx.x, n2, 0);
    return;
  }
  const int n = ((int)blockIdx.x - n2) * kWaves + (int)(threadIdx.x / kWave);
  if (n < s.N) shared_gemv_row<2, SC>(s, n, threadIdx.x & (kWave - 1));
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

template <int NXG>
const void* k13_one() { return reinterpret_cast<const void*>(gemv13_one_kernel<NXG>); }

hipError_t launch_one(const LayerArgs& a, hipStream_t stream) {
  const hipEvent_t* ev = a.ev;
  const int nxg = one_xg(a.H), npl = one_pl(a.I, a.k);
  const void* k13 = nxg == 1 ? k13_one<1>() : nxg == 2 ? k13_one<2>() : nxg == 3 ? k13_one<3>()
                                                                             : k13_one<4>();
  const Residency res = residency(k13, 0);
  if (res.wgs <= 0) return hipErrorInvalidValue;
  const int units = a.k * a.I;
  const dim3 blk(kThreads), g13(std::min(res.wgs, (units + kWaves - 1) / kWaves));
  const hipEvent_t e0 = ev_start(ev, 1), e1 = ev_stop(ev, 1);
  switch (nxg) {
    case 1: launch_k(gemv13_one_kernel<1>, g13, blk, 0, stream, e0, e1, a); break;
    case 2: launch_k(gemv13_one_kernel<2>, g13, blk, 0, stream, e0, e1, a); break;
    case 3: launch_k(gemv13_one_kernel<3>, g13, blk, 0, stream, e0, e1, a); break;
    default: launch_k(gemv13_one_kernel<4>, g13, blk, 0, stream, e0, e1, a); break;
  }
  // w2: one workgroup per compute unit, at most kOneRowsMax rows each
  const int n2 = std::max((a.H + kOneRowsMax - 1) / kOneRowsMax, std::min(a.H, res.cus));
  const dim3 g2(n2);
  if (a.shared13) {
    // the shared expert's w1/w3 rows ride along: one wave a row after the n2
    // w2 workgroups, with the chunk count its own kernel would take
    const SharedArgs& s = *a.shared13;
    const int ncl = std::min((s.K / 16 + kWave - 1) / kWave, kGvMaxChunks);
    const dim3 gs(n2 + (s.N + kWaves - 1) / kWaves);
#define MOE_W2S(NPL, SC) \
  launch_k(gemv2_one_shared_kernel<NPL, SC>, gs, blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a, s, n2)
#define MOE_W2S_NPL(NPL)                                                              \
  switch (ncl) {                                                                     \
    case 1: MOE_W2S(NPL, 1); break;                                                  \
    case 2: MOE_W2S(NPL, 2); break;                                                  \
    case 3: MOE_W2S(NPL, 3); break;                                                  \
    case 4: MOE_W2S(NPL, 4); break;                                                  \
    case 5: MOE_W2S(NPL, 5); break;                                                  \
    case 6: MOE_W2S(NPL, 6); break;                                                  \
    case 7: MOE_W2S(NPL, 7); break;                                                  \
    default: MOE_W2S(NPL, 8); break;                                                 \
  }
    if (npl == 1) {
      MOE_W2S_NPL(1)
    } else {
      MOE_W2S_NPL(2)
    }
#undef MOE_W2S_NPL
#undef MOE_W2S
    return hipSuccess;
  }
  if (npl == 1)
    launch_k(gemv2_one_kernel<1, false>, g2, blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a);
  else
    launch_k(gemv2_one_kernel<2, false>, g2, blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a);
  return hipSuccess;
}

bool few_fits(int T, int H, int I, int k) {
  return T >= 2 && T <= kFewMaxT && one_token_fits(H, I, k) && few13_lds(T, H, k) <= kFewLdsBig;
}

// The few-token w1/w3 kernel for NXG and the workgroup size the LDS allows;
// the dynamic LDS limit is raised once per (device, kernel).
template <int NW>
hipError_t launch_few13(const LayerArgs& a, int nxg, size_t lds, hipStream_t stream, int& cus) {
  const void* k = nxg == 1   ? reinterpret_cast<const void*>(gemv13_few_kernel<1, NW>)
                  : nxg == 2 ? reinterpret_cast<const void*>(gemv13_few_kernel<2, NW>)
                  : nxg == 3 ? reinterpret_cast<const void*>(gemv13_few_kernel<3, NW>)
                             : reinterpret_cast<const void*>(gemv13_few_kernel<4, NW>);
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
  switch (nxg) {
    case 1: launch_k(gemv13_few_kernel<1, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 2: launch_k(gemv13_few_kernel<2, NW>, g, blk, lds, stream, e0, e1, a); break;
    case 3: launch_k(gemv13_few_kernel<3, NW>, g, blk, lds, stream, e0, e1, a); break;
    default: launch_k(gemv13_few_kernel<4, NW>, g, blk, lds, stream, e0, e1, a); break;
  }
  return hipSuccess;
}

hipError_t launch_few(const LayerArgs& a, hipStream_t stream) {
  const hipEvent_t* ev = a.ev;
  const int nxg = one_xg(a.H), npl = one_pl(a.I, a.k);
  const size_t lds = few13_lds(a.T, a.H, a.k);
  int cus = 0;
  const hipError_t e13 = lds <= kDecodeLds ? launch_few13<kWaves>(a, nxg, lds, stream, cus)
                                           : launch_few13<2 * kWaves>(a, nxg, lds, stream, cus);
  if (e13 != hipSuccess) return e13;
  const dim3 blk(kThreads);
  // w2: (row block, token) workgroups; the row-block count a multiple of 8 so
  // that a row block's workgroups share an XCD
  int n2 = std::max((a.H + kOneRowsMax - 1) / kOneRowsMax, std::min(a.H, cus));
  n2 = (n2 + 7) / 8 * 8;
  const dim3 g2(n2, a.T);
  if (npl == 1)
    launch_k(gemv2_one_kernel<1, true>, g2, blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a);
  else
    launch_k(gemv2_one_kernel<2, true>, g2, blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a);
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

bool decode_fuses_route(int T, int H, int I, int E, int k) {
  return T == 1 && one_token_fits(H, I, k) && E <= kFusedVPL * kWave;
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
