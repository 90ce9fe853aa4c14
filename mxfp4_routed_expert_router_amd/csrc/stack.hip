// Pre-normalisation for a residual stack of MoE layers.  The layers chained as
// x_{l+1} = x_l + moe_l(x_l) overflow within a few layers because the SwiGLU
// expert is quadratic in its input; normalising each layer's input to unit RMS
// (then rounding to the bf16 the experts take) keeps the chain finite.
#include "device_common.h"
#include "kernels.h"

namespace moe_fp4 {
namespace {

// One workgroup per token row: u = bf16(x / sqrt(mean(x^2) + eps)).  The sum of
// squares is reduced in a fixed order (row_rms), so u is reproducible bit for bit.
__global__ void __launch_bounds__(256) prenorm_kernel(const float* __restrict__ x,
                                                      uint16_t* __restrict__ u, int H, float eps) {
  __shared__ float wsum[4];
  const float* xr = x + (size_t)blockIdx.x * H;
  const float r = row_rms(xr, H, eps, wsum);
  uint16_t* ur = u + (size_t)blockIdx.x * H;
  for (int m = threadIdx.x; m < H; m += 256) ur[m] = f32_to_bf16_rne(xr[m] / r);
}

}  // namespace

hipError_t launch_prenorm(const float* x, uint16_t* u, int T, int H, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(prenorm_kernel, dim3(T), dim3(256), 0, stream, x, u, H, eps);
  return hipGetLastError();
}

}  // namespace moe_fp4
