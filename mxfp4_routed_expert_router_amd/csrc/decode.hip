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
#include "device_common.h"
#include "kernels.h"
#include "topk.h"

namespace moe_fp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kBPW = 5;  // MFMA path: weight blocks (4 scale groups each) per wave in one batch
constexpr int kEB = 6;   // MFMA path: experts whose w2 loads are in flight together
constexpr int kB2 = 3;   // MFMA path: w2 blocks per wave and expert (I <= 8 * 3 * 128)
constexpr int kDJ13 = 5;  // dot path: load instructions per wave and batch, w1/w3
constexpr int kDJ2 = 14;  // dot path: load instructions per wave and batch, w2
constexpr int kDX = 4;    // dot path: activation chunks per thread loaded ahead of the weights
constexpr int kDotMaxPairs = 32;   // dot path: token-expert pairs of a step (T <= 2, k <= 16)
constexpr int kFusedVPL = 8;       // fused routing: logits per lane (E <= 512)

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

// =========================================================================== dot path
// Activation rows in LDS for the dot kernels: each 32-input group (64 bytes)
// takes an 80-byte slot.  Lane l reads group l, so lane addresses step by 20
// dwords and a wave's 16-byte reads fall on every bank group evenly instead
// of a quarter of them (a 64-byte step).
constexpr int kGS = 40;  // bf16 per group slot
__host__ __device__ constexpr int grp_row(int K) { return (K / 32) * kGS; }  // bf16 per row
__device__ __forceinline__ int grp_chunk(int c) { return (c >> 2) * kGS + (c & 3) * 8; }

size_t lds13_dot_bytes(int T, int H) { return align256((size_t)T * grp_row(H) * 2); }
size_t lds2_dot_bytes(int P, int I) {
  return align256((size_t)P * grp_row(I) * 2) + (size_t)4 * kDotMaxPairs * 4;
}

// One token: rank the logits (every workgroup does, redundantly) and take
// this workgroup's expert, the d-th smallest id among the k chosen (each
// chosen expert holds exactly one pair, so its sorted slot is d).  Workgroup
// (0, 0) publishes the routing result for the later kernels.
__device__ DInfo fused_route(const LayerArgs& a, int d, int* s_e, float* s_g, int* s_sorted,
                             int* s_rank) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int k = a.k, E = a.E;
  if (tid < kWave) {
    wave_topk<kFusedVPL>(a.logits, E, k, lane, s_e, s_g);
    // rank of each chosen id among the chosen (they are distinct)
    const int my_e = lane < k ? s_e[lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(my_e, i) < my_e ? 1 : 0;
    if (lane < k) {
      s_sorted[rank] = my_e;
      s_rank[lane] = rank;
    }
  }
  lds_barrier();
  const int e = s_sorted[d];
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    const RouteArgs& r = a.route;
    if (tid < k) {
      const int rank = s_rank[tid];
      r.idx[tid] = s_e[tid];
      r.gates[tid] = s_g[tid];
      r.sorted_pairs[rank] = tid;
      r.pair_slot[tid] = rank;
      r.dinfo[4 * rank + 0] = s_e[tid];
      r.dinfo[4 * rank + 1] = rank;
      r.dinfo[4 * rank + 2] = 1;
      r.dinfo[4 * rank + 3] = 0;
    }
    for (int x = tid; x < E; x += kThreads) {
      int below = 0;
      while (below < k && s_sorted[below] < x) ++below;
      r.counts[x] = (below < k && s_sorted[below] == x) ? 1 : 0;
      r.offsets[x] = below;
    }
    if (tid == 0) {
      r.offsets[E] = k;
      r.meta[0] = k;
    }
  }
  return DInfo{e, d, 1};
}

template <int NT>
__global__ void __launch_bounds__(kThreads) gemv13_dot_kernel(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_e[kMaxK], s_sorted[kMaxK], s_rank[kMaxK];
  __shared__ float s_g[kMaxK];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int H = a.H, CPR = H / 32, C2 = 2 * CPR, XS = grp_row(H), C8 = H / 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);

  DInfo di;
  if (NT == 1 && a.fused_route) {
    // the token is row 0: its x loads need no routing and go out first
    u32x4 xr[kDX];
#pragma unroll
    for (int q = 0; q < kDX; ++q) {
      const int i = tid + q * kThreads;
      xr[q] = ld16(a.x + (size_t)(i < C8 ? i : 0) * 8);
    }
    di = fused_route(a, blockIdx.y, s_e, s_g, s_sorted, s_rank);
#pragma unroll
    for (int q = 0; q < kDX; ++q) {
      const int i = tid + q * kThreads;
      if (i < C8) st16(xs + grp_chunk(i), xr[q]);
    }
    for (int i = tid + kDX * kThreads; i < C8; i += kThreads)
      st16(xs + grp_chunk(i), ld16(a.x + (size_t)i * 8));
  } else {
    di = load_dinfo(a.dinfo, blockIdx.y);
    if (di.e < 0) return;
  }
  const int e = di.e, off = di.off, ne = di.ne;
  const int r = blockIdx.x * 16 + 2 * w;  // this wave's first row
  const uint8_t* w1b = a.w1 + (size_t)e * a.stride[0] + (size_t)r * (H / 2);
  const uint8_t* w3b = a.w3 + (size_t)e * a.stride[2] + (size_t)r * (H / 2);
  const uint8_t* s1b = a.s1 + (size_t)e * a.stride[1] + (size_t)r * CPR;
  const uint8_t* s3b = a.s3 + (size_t)e * a.stride[3] + (size_t)r * CPR;

  // Unfused: x rows of this expert's tokens.  Their loads go out before the
  // weight loads so that waiting for them never waits for the weight stream.
  int trow[NT];
  u32x4 xr[kDX];
  const bool stage = !(NT == 1 && a.fused_route);
  if (stage) {
#pragma unroll
    for (int t = 0; t < NT; ++t) trow[t] = a.sorted_pairs[off + (t < ne ? t : 0)] / a.k;
#pragma unroll
    for (int q = 0; q < kDX; ++q) {
      const int i = tid + q * kThreads;
      const bool ok = i < ne * C8;
      const int ii = ok ? i : 0, n = ii / C8, c = ii - n * C8;
      int t = trow[0];
#pragma unroll
      for (int u = 1; u < NT; ++u) t = n == u ? trow[u] : t;
      xr[q] = ld16(a.x + (size_t)t * H + c * 8);
    }
  }

  float a1[NT][2], a3[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) a1[t][0] = a1[t][1] = a3[t][0] = a3[t][1] = 0.f;
  for (int c0 = 0; c0 < C2; c0 += kDJ13 * kWave) {
    u32x4 q1[kDJ13], q3[kDJ13];
    uint32_t e1[kDJ13], e3[kDJ13];
#pragma unroll
    for (int j = 0; j < kDJ13; ++j) {
      const int c = c0 + j * kWave + lane;
      const bool ok = c < C2;
      const int cc = ok ? c : 0;
      q1[j] = sel4(ok, ld16(w1b + (size_t)cc * 16));
      q3[j] = sel4(ok, ld16(w3b + (size_t)cc * 16));
      const uint32_t x1 = s1b[cc], x3 = s3b[cc];
      e1[j] = ok ? x1 : 0u;
      e3[j] = ok ? x3 : 0u;
    }
    if (c0 == 0) {
      if (stage) {
#pragma unroll
        for (int q = 0; q < kDX; ++q) {
          const int i = tid + q * kThreads;
          if (i < ne * C8) {
            const int n = i / C8, c = i - n * C8;
            st16(xs + n * XS + grp_chunk(c), xr[q]);
          }
        }
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < kDJ13; ++j) {
      const int c = c0 + j * kWave + lane;
      const int rl = c >= CPR ? 1 : 0;
      const int g = c < C2 ? c - rl * CPR : 0;
      const float sc1 = ue8m0_to_f32(e1[j]), sc3 = ue8m0_to_f32(e3[j]);
      float p1[NT], p3[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) p1[t] = p3[t] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 A1 = fp4x8_to_bf16x8(q1[j][i], sc1);
        const bf16x8 A3 = fp4x8_to_bf16x8(q3[j][i], sc3);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 X = as_bf16x8(ld16(xs + t * XS + g * kGS + 8 * i));
          p1[t] = dot8_bf16(A1, X, p1[t]);
          p3[t] = dot8_bf16(A3, X, p3[t]);
        }
      }
      if (c < C2) {  // a lane past the end adds nothing (not even 0 * inf)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (rl) { a1[t][1] += p1[t]; a3[t][1] += p3[t]; }
          else { a1[t][0] += p1[t]; a3[t][0] += p3[t]; }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int rl = 0; rl < 2; ++rl) {
      const float G = wave_sum_f32(a1[t][rl]), U = wave_sum_f32(a3[t][rl]);
      if (lane == 0 && t < ne) a.h[(size_t)(off + t) * a.I + r + rl] = swiglu_bf16(G, U);
    }
}

// y rows m, m+1 of this wave for the step's tokens: sum over the distinct
// experts of gate * (w2 row . h row), chunk by chunk, then one DPP reduction.
// Chunk c of the wave enumerates (expert d, row, 32-input group) with d major;
// a load instruction spans at most two experts, whose ids are read with
// scalar loads.
template <int NT, int KH>
__global__ void __launch_bounds__(kThreads) gemv2_dot_kernel(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int P = a.T * a.k;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int I = a.I, CPR = I / 32, C2 = 2 * CPR, IS = grp_row(I), C8 = I / 8;
  const int m = blockIdx.x * 16 + 2 * w;  // this wave's first output row
  const int nd = a.meta[0];
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
  float* s_gate = reinterpret_cast<float*>(smem + align256((size_t)P * IS * 2));  // per slot
  int* s_tok = reinterpret_cast<int*>(s_gate + kDotMaxPairs);
  int* s_off = s_tok + kDotMaxPairs;  // per distinct expert
  int* s_ne = s_off + kDotMaxPairs;

  // h rows (all pairs of the step, sorted order): loads first
  u32x4 hr[KH];
#pragma unroll
  for (int q = 0; q < KH; ++q) {
    const int i = tid + q * kThreads;
    hr[q] = ld16(a.h + (size_t)(i < P * C8 ? i : 0) * 8);
  }
  const int total = nd * C2;
  float acc[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = 0.f;
  for (int c0 = 0; c0 < total; c0 += kDJ2 * kWave) {
    u32x4 q[kDJ2];
    uint32_t ev[kDJ2];
#pragma unroll
    for (int j = 0; j < kDJ2; ++j) {
      const int cb = c0 + j * kWave;  // uniform
      const int c = cb + lane;
      const bool ok = c < total;
      int e, cr;
      if (C2 >= kWave) {  // uniform: the instruction spans at most two experts
        const int dlo = min(cb / C2, nd - 1);
        const int dhi = min(dlo + 1, nd - 1);
        const int elo = a.dinfo[4 * dlo], ehi = a.dinfo[4 * dhi];
        const bool hi = c >= (dlo + 1) * C2;
        e = hi ? ehi : elo;
        cr = ok ? c - (hi ? dhi : dlo) * C2 : 0;
      } else {            // narrow w2 rows: look the expert up per lane
        const int cc = ok ? c : 0, dd = cc / C2;
        e = a.dinfo[4 * dd];
        cr = cc - dd * C2;
      }
      q[j] = sel4(ok, ld16(a.w2 + (size_t)e * a.stride[4] + (size_t)m * (I / 2) + (size_t)cr * 16));
      const uint32_t x = a.s2[(size_t)e * a.stride[5] + (size_t)m * CPR + cr];
      ev[j] = ok ? x : 0u;
    }
    if (c0 == 0) {
#pragma unroll
      for (int qq = 0; qq < KH; ++qq) {
        const int i = tid + qq * kThreads;
        if (i < P * C8) {
          const int n = i / C8, c = i - n * C8;
          st16(hs + n * IS + grp_chunk(c), hr[qq]);
        }
      }
      for (int i = tid + KH * kThreads; i < P * C8; i += kThreads) {
        const int n = i / C8, c = i - n * C8;
        st16(hs + n * IS + grp_chunk(c), ld16(a.h + (size_t)i * 8));
      }
      for (int s = tid; s < P; s += kThreads) {
        const int p = a.sorted_pairs[s];
        s_gate[s] = a.gates[p];
        s_tok[s] = p / a.k;
      }
      for (int dd = tid; dd < nd; dd += kThreads) {
        const DInfo di = load_dinfo(a.dinfo, dd);
        s_off[dd] = di.off;
        s_ne[dd] = di.ne;
      }
      lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < kDJ2; ++j) {
      const int cb = c0 + j * kWave;  // uniform
      const int c = cb + lane;
      const bool ok = c < total;
      const int cc = ok ? c : 0;
      int dd;
      if (C2 >= kWave) {  // same bracketing as the loads
        const int dlo = min(cb / C2, nd - 1);
        dd = cc >= (dlo + 1) * C2 ? dlo + 1 : dlo;
      } else {
        dd = cc / C2;
      }
      const int cr = cc - dd * C2;
      const int rl = cr >= CPR ? 1 : 0;
      const int g = cr - rl * CPR;
      const int off = s_off[dd], nex = s_ne[dd];
      const float sc = ue8m0_to_f32(ev[j]);
      bf16x8 A[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) A[i] = fp4x8_to_bf16x8(q[j][i], sc);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        if (ok && u < nex) {
          const int s = off + u;
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) p = dot8_bf16(A[i], as_bf16x8(ld16(hs + s * IS + g * kGS + 8 * i)), p);
          const float gp = s_gate[s] * p;
          const int t = s_tok[s];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            if (t == tt) {
              if (rl) acc[tt][1] += gp; else acc[tt][0] += gp;
            }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int rl = 0; rl < 2; ++rl) {
      const float Y = wave_sum_f32(acc[t][rl]);
      if (lane == 0 && t < a.T) {
        float* yp = a.y + (size_t)t * a.H + m + rl;
        *yp = a.accumulate ? *yp + Y : Y;
      }
    }
}

// One or two tokens take the row-contiguous kernels (x staged ahead of the
// weights needs T * H <= 8 * kDX * kThreads); up to 16, the MFMA kernels.
bool use_dot(int T, int H) { return T <= 2 && T * (H / 8) <= kDX * kThreads; }

}  // namespace

bool decode_fits(int T, int H, int I, int k) {
  const int P = T * k;
  if (use_dot(T, H))
    return P <= kDotMaxPairs && lds13_dot_bytes(T, H) <= kDecodeLds &&
           lds2_dot_bytes(P, I) <= kDecodeLds;
  return T <= kDecodeMaxTokens && I <= kWaves * kB2 * 128 && lds13_bytes(T, H) <= kDecodeLds &&
         lds2_bytes(P, I) <= kDecodeLds;
}

bool decode_fuses_route(int T, int H, int E) {
  return T == 1 && use_dot(T, H) && E <= kFusedVPL * kWave;
}

hipError_t launch_decode(const LayerArgs& a, hipStream_t stream) {
  const int P = a.T * a.k;
  const int dmax = P < a.E ? P : a.E;  // distinct experts can not exceed either
  const hipEvent_t* ev = a.stage_events;
  const dim3 blk(kThreads), g13(a.I / 16, dmax), g2(a.H / 16);
  if (!use_dot(a.T, a.H)) {
    hipLaunchKernelGGL(gemv13_kernel, g13, blk, lds13_bytes(a.T, a.H), stream, a);
    if (ev) (void)hipEventRecord(ev[0], stream);
    hipLaunchKernelGGL(gemv2_combine_kernel, g2, blk, lds2_bytes(P, a.I), stream, a);
  } else {
    const size_t l13 = lds13_dot_bytes(a.T, a.H), l2 = lds2_dot_bytes(P, a.I);
    const bool small_h = P * (a.I / 8) <= 4 * kThreads;
    if (a.T == 1) {
      hipLaunchKernelGGL(gemv13_dot_kernel<1>, g13, blk, l13, stream, a);
      if (ev) (void)hipEventRecord(ev[0], stream);
      if (small_h)
        hipLaunchKernelGGL((gemv2_dot_kernel<1, 4>), g2, blk, l2, stream, a);
      else
        hipLaunchKernelGGL((gemv2_dot_kernel<1, 8>), g2, blk, l2, stream, a);
    } else {
      hipLaunchKernelGGL(gemv13_dot_kernel<2>, g13, blk, l13, stream, a);
      if (ev) (void)hipEventRecord(ev[0], stream);
      if (small_h)
        hipLaunchKernelGGL((gemv2_dot_kernel<2, 4>), g2, blk, l2, stream, a);
      else
        hipLaunchKernelGGL((gemv2_dot_kernel<2, 8>), g2, blk, l2, stream, a);
    }
  }
  if (ev) {
    (void)hipEventRecord(ev[1], stream);
    (void)hipEventRecord(ev[2], stream);
  }
  return hipGetLastError();
}

}  // namespace moe_fp4
