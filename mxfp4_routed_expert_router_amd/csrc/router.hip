// Router logits: logits[t][e] = sum_c x[t][c] * Wr[e][c], with x bf16 [T][H],
// the router weight Wr [E][H] and logits fp32 [T][E].  The 10100.com page
// (section on the expert-capacity bottleneck) lists the router among the
// resident dense weights without giving its format; Wr is taken as bf16.
// bf16 products are exact in fp32; sums are fp32.  Every logit is produced by
// one wave in a fixed order, so the logits -- and the routing taken from
// them -- are the same bits on every run.
//
//   router_gemv_kernel  T <= 4: one wave per expert row, four rows a
//                       workgroup.  Lane l takes the 16-byte chunks l + 64 j
//                       of the row (whole 128-byte lines per load), all issued
//                       before the first use; the token rows are read the same
//                       way (L2-served after the first wave) and the wave
//                       reduces with DPP.
//   router_gemm_kernel  T > 4: 64 experts x 64 tokens per workgroup, four
//                       waves of 16 experts; K in blocks of 64 staged through
//                       a double-buffered LDS tile; 16x16x32 bf16 MFMA.
#include "device_common.h"
#include "kernels.h"

namespace moe_fp4 {
namespace {

constexpr int kGemvMaxT = 4;
constexpr int kGemvChunks = 16;  // 16-byte chunks per lane in flight (H <= 8192 in one round)

constexpr int kGemvRows = 4;  // expert rows (waves) per workgroup

__global__ void __launch_bounds__(kGemvRows * kWave) router_gemv_kernel(const uint16_t* __restrict__ x,
                                                                         const uint16_t* __restrict__ w,
                                                                         float* __restrict__ logits,
                                                                         int T, int H, int E) {
  const int e = blockIdx.x * kGemvRows + (int)(threadIdx.x / kWave), lane = threadIdx.x & (kWave - 1);
  if (e >= E) return;  // whole wave
  const int NC = H / 8;                                   // chunks per row
  const int NCL = (NC + kWave - 1) / kWave;               // chunks per lane
  const uint16_t* const wr = w + (size_t)e * H;
  float acc[kGemvMaxT] = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < NCL; g0 += kGemvChunks) {
    int cc[kGemvChunks];
    u32x4 wv[kGemvChunks];
#pragma unroll
    for (int j = 0; j < kGemvChunks; ++j) {
      const int c = lane + kWave * (g0 + j);
      cc[j] = c < NC ? c : NC - 1;  // past the row end: a duplicate chunk, not summed
      if (g0 + j < NCL) wv[j] = ld16(wr + (size_t)cc[j] * 8);
    }
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
      if (t >= T) break;
      const uint16_t* const xr = x + (size_t)t * H;
      u32x4 xv[kGemvChunks];
#pragma unroll
      for (int j = 0; j < kGemvChunks; ++j)
        if (g0 + j < NCL) xv[j] = ld16(xr + (size_t)cc[j] * 8);
#pragma unroll
      for (int j = 0; j < kGemvChunks; ++j)
        if (g0 + j < NCL && lane + kWave * (g0 + j) < NC)
          acc[t] = dot8_bf16(as_bf16x8(wv[j]), as_bf16x8(xv[j]), acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvMaxT; ++t) {
    if (t >= T) break;
    const float s = wave_sum_f32(acc[t]);
    if (lane == 0) logits[(size_t)t * E + e] = s;
  }
}

constexpr int kRT = 64;        // experts and tokens per workgroup tile
constexpr int kRK = 64;        // inputs per K block
constexpr int kRS = kRK + 8;   // LDS row stride in bf16: 16 rows hit 16 different bank groups
constexpr int kRThreads = 4 * kWave;

__global__ void __launch_bounds__(kRThreads) router_gemm_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                float* __restrict__ logits, int T,
                                                                int H, int E) {
  __shared__ uint16_t sw[2][kRT][kRS];
  __shared__ uint16_t sx[2][kRT][kRS];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int c16 = lane & 15, kq = lane >> 4;
  const int e0 = blockIdx.x * kRT, t0 = blockIdx.y * kRT;
  const int NK = (H + kRK - 1) / kRK;

  // staging: thread tid moves chunks id = tid + 256 u (u < 2) of each tile:
  // row id / 8, 8 inputs at 8 (id % 8).  Rows past E or T read the last row
  // (results not stored); inputs past H are stored as zeros.
  const uint16_t* wrow[2];
  const uint16_t* xrow[2];
  int col[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + kRThreads * u, r = id / 8;
    col[u] = 8 * (id % 8);
    wrow[u] = w + (size_t)min(e0 + r, E - 1) * H;
    xrow[u] = x + (size_t)min(t0 + r, T - 1) * H;
  }
  u32x4 rw[2], rx[2];
  auto load = [&](int kb) {
    kb = kb < NK ? kb : NK - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kb * kRK + col[u];
      const int kc = k < H ? k : H - 8;
      rw[u] = ld16(wrow[u] + kc);
      rx[u] = ld16(xrow[u] + kc);
    }
  };
  auto store = [&](int kb, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + kRThreads * u, r = id / 8;
      const bool ok = kb * kRK + col[u] < H;
      st16(&sw[buf][r][col[u]], sel4(ok, rw[u]));
      st16(&sx[buf][r][col[u]], sel4(ok, rx[u]));
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  store(0, 0);
  lds_barrier();
  for (int kb = 0; kb < NK; ++kb) {
    const int buf = kb & 1;
    load(kb + 1);
#pragma unroll
    for (int ks = 0; ks < kRK / 32; ++ks) {
      const bf16x8 A = as_bf16x8(ld16(&sw[buf][16 * wv + c16][32 * ks + 8 * kq]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 B = as_bf16x8(ld16(&sx[buf][16 * nt + c16][32 * ks + 8 * kq]));
        acc[nt] = mfma16x16x32(A, B, acc[nt]);
      }
    }
    store(kb + 1, buf ^ 1);  // the other buffer was last read in block kb - 1
    lds_barrier();
  }
  // acc[nt][q]: expert e0 + 16 wv + 4 kq + q, token t0 + 16 nt + c16
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = t0 + 16 * nt + c16;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 16 * wv + 4 * kq + q;
      if (e < E) logits[(size_t)t * E + e] = acc[nt][q];
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w, float* logits, int T, int H,
                                int E, hipStream_t stream) {
  if (T <= kGemvMaxT)
    hipLaunchKernelGGL(router_gemv_kernel, dim3((E + kGemvRows - 1) / kGemvRows), dim3(kGemvRows * kWave),
                       0, stream, x, w, logits, T, H, E);
  else
    hipLaunchKernelGGL(router_gemm_kernel, dim3((E + kRT - 1) / kRT, (T + kRT - 1) / kRT),
                       dim3(kRThreads), 0, stream, x, w, logits, T, H, E);
  return hipGetLastError();
}

}  // namespace moe_fp4
