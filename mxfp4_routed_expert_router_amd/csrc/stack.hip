// Pre-normalisation for a residual stack of MoE layers.  The layers chained as
// x_{l+1} = x_l + moe_l(x_l) overflow within a few layers because the SwiGLU
// expert is quadratic in its input; normalising each layer's input to unit RMS
// (then rounding to the bf16 the experts take) keeps the chain finite.
#include "device_common.h"
#include "kernels.h"

namespace moe_fp4 {
namespace {

// One 512-thread workgroup per token row: u = bf16(x / sqrt(mean(x^2) + eps)).
// Thread t holds the 8-value chunks t, t + 512, ... (H <= 16384: at most 4) in
// registers; the sum of squares runs in the fixed order of chunk_sumsq and
// block_rms, so u is reproducible bit for bit and equal to the pre-norm fused
// into the one-token decode kernel.
constexpr int kNormChunks = 4;

__global__ void __launch_bounds__(kNormThreads) prenorm_kernel(const float* __restrict__ x,
                                                               uint16_t* __restrict__ u, int H,
                                                               float eps) {
  __shared__ float wsum[kNormThreads / 64];
  const float* xr = x + (size_t)blockIdx.x * H;
  const int nc = H / 8, t = threadIdx.x;
  float4 f[2 * kNormChunks];
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = t + kNormThreads * i, cc = c < nc ? c : 0;
    f[2 * i] = *reinterpret_cast<const float4*>(xr + 8 * cc);
    f[2 * i + 1] = *reinterpret_cast<const float4*>(xr + 8 * cc + 4);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i)
    if (t + kNormThreads * i < nc) ss = chunk_sumsq(f[2 * i], f[2 * i + 1], ss);
  const float r = block_rms(ss, H, eps, wsum);
  u32x4* ur = reinterpret_cast<u32x4*>(u + (size_t)blockIdx.x * H);
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = t + kNormThreads * i;
    if (c < nc) ur[c] = chunk_to_bf16(f[2 * i], f[2 * i + 1], r);
  }
}

}  // namespace

hipError_t launch_prenorm(const float* x, uint16_t* u, int T, int H, float eps, hipStream_t stream) {
  if (H / 8 > kNormThreads * kNormChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prenorm_kernel, dim3(T), dim3(kNormThreads), 0, stream, x, u, H, eps);
  return hipGetLastError();
}

}  // namespace moe_fp4
