// The shared expert: one per layer beside the routed ones (ai-shiz.ru page,
// section "what the model is"), kept in FP8 (10100.com page, plan two), with
// the model's main weights stored as FP8 in 32 x 32 blocks (ai-shiz.ru page,
// same section).  Taken as a SwiGLU expert of the routed experts' form:
//   w1, w3 [I][H] and w2 [H][I] E4M3 codes, s1, s3 [I/32][H/32] and s2
//   [H/32][I/32] UE8M0 scales, one per 32 x 32 block;
//   h = bf16(silu(W1 x) * (W3 x)), y (+)= W2 h, no gate.
// An E4M3 value times a power of two is exact in bf16, so the weights are
// decoded to bf16 (v_cvt_scalef32_pk_bf16_fp8) and every product is exact in
// fp32, as on the routed path.
//
// One token, where the shapes fit, runs on the one-token decode kernels with no
// routed expert (launch_shared_one, decode.hip).  Otherwise:
//   shared_gemv_kernel<M, C>  T <= 4: one wave per output row; lane l takes the
//                          16-byte chunks l + 64 j of the row (16 codes each,
//                          whole lines per load), the wave reduces with DPP.
//   shared_gemm_kernel<M>  T > 4: 64 rows x 64 tokens per workgroup, four
//                          waves of 16 rows; K in blocks of 64 through a
//                          double-buffered LDS tile, the FP8 codes decoded as
//                          they are staged; 16x16x32 bf16 MFMA.
// M = 2: w1 and w3 with the SwiGLU epilogue into h; M = 1: w2, y (+)= W2 h.
#include "device_common.h"
#include "kernels.h"
#include "shared_gemv.h"

namespace moe_fp4 {
namespace {

template <int M, int kGvChunks>
__global__ void __launch_bounds__(4 * kWave) shared_gemv_kernel(SharedArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;  // whole wave
  shared_gemv_row<M, kGvChunks>(a, n, lane);
}

constexpr int kST = 64;        // rows and tokens per workgroup tile
constexpr int kSK = 64;        // inputs per K block
constexpr int kSS = kSK + 8;   // LDS row stride in bf16 (16 rows on 16 bank groups)
constexpr int kSThreads = 4 * kWave;

template <int M>
__global__ void __launch_bounds__(kSThreads) shared_gemm_kernel(SharedArgs a) {
  __shared__ uint16_t sw[2][M][kST][kSS];
  __shared__ uint16_t sx[2][kST][kSS];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int c16 = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * kST, t0 = blockIdx.y * kST;
  const int K = a.K, NK = (K + kSK - 1) / kSK;

  // activations: chunks id = tid + 256 u (u < 2): row id / 8, 8 inputs at 8 (id % 8)
  const uint16_t* xrow[2];
  int xcol[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + kSThreads * u;
    xcol[u] = 8 * (id % 8);
    xrow[u] = a.act + (size_t)min(t0 + id / 8, a.T - 1) * K;
  }
  // weights: row tid / 4, 16 codes at 16 (tid % 4) of the block, per matrix
  const int wr = tid / 4, wcol = 16 * (tid % 4);
  const int wn = min(n0 + wr, a.N - 1);
  u32x4 rx[2], rw[M];
  uint32_t rs[M];
  auto load = [&](int kb) {
    kb = kb < NK ? kb : NK - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kb * kSK + xcol[u];
      rx[u] = ld16(xrow[u] + (k < K ? k : K - 8));
    }
    const int k = kb * kSK + wcol, kc = k < K ? k : K - 16;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      rw[m] = ld16(a.w[m] + (size_t)wn * K + kc);
      rs[m] = a.s[m][(wn / 32) * (K / 32) + kc / 32];
    }
  };
  auto store = [&](int kb, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + kSThreads * u;
      st16(&sx[buf][id / 8][xcol[u]], sel4(kb * kSK + xcol[u] < K, rx[u]));
    }
    const bool ok = kb * kSK + wcol < K;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      bf16x8 lo, hi;
      fp8x16_to_bf16(sel4(ok, rw[m]), ue8m0_to_f32(rs[m]), lo, hi);
      st16(&sw[buf][m][wr][wcol], __builtin_bit_cast(u32x4, lo));
      st16(&sw[buf][m][wr][wcol + 8], __builtin_bit_cast(u32x4, hi));
    }
  };

  f32x4 acc[M][4];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  store(0, 0);
  lds_barrier();
  for (int kb = 0; kb < NK; ++kb) {
    const int buf = kb & 1;
    load(kb + 1);
#pragma unroll
    for (int ks = 0; ks < kSK / 32; ++ks) {
      bf16x8 A[M];
#pragma unroll
      for (int m = 0; m < M; ++m) A[m] = as_bf16x8(ld16(&sw[buf][m][16 * wv + c16][32 * ks + 8 * kq]));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8 B = as_bf16x8(ld16(&sx[buf][16 * nt + c16][32 * ks + 8 * kq]));
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m][nt] = mfma16x16x32(A[m], B, acc[m][nt]);
      }
    }
    store(kb + 1, buf ^ 1);  // the other buffer was last read in block kb - 1
    lds_barrier();
  }
  // acc[m][nt][q]: row n0 + 16 wv + 4 kq + q, token t0 + 16 nt + c16
  const int nr = n0 + 16 * wv + 4 * kq;
  if (nr >= a.N) return;  // N is a multiple of 32: the 4 rows are all in or all out
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int t = t0 + 16 * nt + c16;
    if (t >= a.T) continue;
    if constexpr (M == 2) {
      uint16_t hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = swiglu_bf16(acc[0][nt][q], acc[1][nt][q]);
      *reinterpret_cast<uint2*>(a.h + (size_t)t * a.N + nr) =
          uint2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
    } else {
      float4* const yp = reinterpret_cast<float4*>(a.y + (size_t)t * a.N + nr);
      float4 o = {acc[0][nt][0], acc[0][nt][1], acc[0][nt][2], acc[0][nt][3]};
      if (a.accumulate) {
        const float4 p = *yp;
        o = float4{p.x + o.x, p.y + o.y, p.z + o.z, p.w + o.w};
      }
      *yp = o;
    }
  }
}

template <int M, int C>
void launch_gemv(const SharedArgs& s, hipStream_t stream) {
  hipLaunchKernelGGL(HIP_KERNEL_NAME(shared_gemv_kernel<M, C>), dim3((s.N + 3) / 4), dim3(4 * kWave),
                     0, stream, s);
}

template <int M>
void launch_one_gemm(const SharedArgs& s, hipStream_t stream) {
  if (s.T <= kGvMaxT) {
    const int ncl = (s.K / 16 + kWave - 1) / kWave;  // chunks per lane
    switch (ncl < kGvMaxChunks ? ncl : kGvMaxChunks) {
      case 1: launch_gemv<M, 1>(s, stream); break;
      case 2: launch_gemv<M, 2>(s, stream); break;
      case 3: launch_gemv<M, 3>(s, stream); break;
      case 4: launch_gemv<M, 4>(s, stream); break;
      case 5: launch_gemv<M, 5>(s, stream); break;
      case 6: launch_gemv<M, 6>(s, stream); break;
      case 7: launch_gemv<M, 7>(s, stream); break;
      default: launch_gemv<M, 8>(s, stream); break;
    }
  } else
    hipLaunchKernelGGL(shared_gemm_kernel<M>, dim3((s.N + kST - 1) / kST, (s.T + kST - 1) / kST),
                       dim3(kSThreads), 0, stream, s);
}

}  // namespace

hipError_t launch_shared(const uint16_t* x, const uint8_t* const w[6], int T, int H, int I,
                         float* y, int accumulate, uint16_t* h, hipStream_t stream) {
  if (T == 1) {
    bool done = false;
    const hipError_t e = launch_shared_one(x, w, H, I, y, accumulate, h, stream, done);
    if (done || e != hipSuccess) return e;
  }
  SharedArgs s13{};
  s13.act = x;
  s13.w[0] = w[0]; s13.s[0] = w[1]; s13.w[1] = w[2]; s13.s[1] = w[3];
  s13.N = I; s13.K = H; s13.T = T; s13.h = h;
  launch_one_gemm<2>(s13, stream);
  SharedArgs s2{};
  s2.act = h;
  s2.w[0] = w[4]; s2.s[0] = w[5];
  s2.N = H; s2.K = I; s2.T = T; s2.y = y; s2.accumulate = accumulate;
  launch_one_gemm<1>(s2, stream);
  return hipGetLastError();
}

hipError_t launch_shared_w2(const uint16_t* h, const uint8_t* w2, const uint8_t* s2, int T, int H,
                            int I, float* y, int accumulate, hipStream_t stream) {
  SharedArgs s{};
  s.act = h;
  s.w[0] = w2; s.s[0] = s2;
  s.N = H; s.K = I; s.T = T; s.y = y; s.accumulate = accumulate;
  launch_one_gemm<1>(s, stream);
  return hipGetLastError();
}

}  // namespace moe_fp4
