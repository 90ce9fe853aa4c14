// The shared expert's row GEMV (one wave per output row), used by the shared
// expert's own kernels and by the one-token decode's w2 launch, which runs the
// shared w1/w3 rows beside the routed w2 rows.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace moe_fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 16 E4M3 codes (byte i = code i) times `scale` -> bf16 codes 0..7 and 8..15.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& v, float scale, bf16x8& lo,
                                               bf16x8& hi) {
  bf16x2_t p[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    p[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], scale, false);
    p[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[d], scale, true);
  }
  lo = bf16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  hi = bf16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}


// acc + (16 E4M3 codes times their block scale byte) . (16 bf16 inputs, two
// 16-byte chunks): the first eight products, then the last eight, each through
// dot8_bf16.  Every kernel that evaluates a shared-expert row does its chunks
// through this, so they give the same bits.
__device__ __forceinline__ float fp8_chunk_dot(const u32x4& w, uint32_t scale_byte,
                                               const u32x4 (&x)[2], float acc) {
  bf16x8 lo, hi;
  fp8x16_to_bf16(w, ue8m0_to_f32(scale_byte), lo, hi);
  acc = dot8_bf16(lo, as_bf16x8(x[0]), acc);
  return dot8_bf16(hi, as_bf16x8(x[1]), acc);
}

constexpr int kGvMaxT = 4;
constexpr int kGvMaxChunks = 8;  // 16-byte chunks per lane and round (K <= 8192 in one round)

// Output row n of SharedArgs a, one wave: lane l takes the 16-byte chunks
// l + 64 j of the row (16 codes each, whole lines per load), the wave reduces
// with DPP.  kGvChunks: chunks per lane and round, the smallest that covers K
// in one round (registers are sized by it).
template <int M, int kGvChunks>
__device__ __forceinline__ void shared_gemv_row(const SharedArgs& a, int n, int lane) {
  const int K = a.K, T = a.T, NC = K / 16, NCL = (NC + kWave - 1) / kWave;
  const int srow = (n / 32) * (K / 32);
  float acc[M][kGvMaxT];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int t = 0; t < kGvMaxT; ++t) acc[m][t] = 0.f;
  for (int g0 = 0; g0 < NCL; g0 += kGvChunks) {
    int cc[kGvChunks];
    u32x4 wv[M][kGvChunks];
    uint32_t sv[M][kGvChunks];
#pragma unroll
    for (int j = 0; j < kGvChunks; ++j) {
      const int c = lane + kWave * (g0 + j);
      cc[j] = c < NC ? c : NC - 1;  // past the row end: a duplicate chunk, not summed
      if (g0 + j < NCL)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          wv[m][j] = ld16(a.w[m] + (size_t)n * K + (size_t)cc[j] * 16);
          sv[m][j] = a.s[m][srow + cc[j] / 2];
        }
    }
#pragma unroll
    for (int t = 0; t < kGvMaxT; ++t) {
      if (t >= T) break;
      const uint16_t* const xr = a.act + (size_t)t * K;
      u32x4 xv[kGvChunks][2];
#pragma unroll
      for (int j = 0; j < kGvChunks; ++j)
        if (g0 + j < NCL) {
          xv[j][0] = ld16(xr + (size_t)cc[j] * 16);
          xv[j][1] = ld16(xr + (size_t)cc[j] * 16 + 8);
        }
#pragma unroll
      for (int j = 0; j < kGvChunks; ++j)
        if (g0 + j < NCL && lane + kWave * (g0 + j) < NC)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[m][t] = fp8_chunk_dot(wv[m][j], sv[m][j], xv[j], acc[m][t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kGvMaxT; ++t) {
    if (t >= T) break;
    const float r0 = wave_sum_f32(acc[0][t]);
    if constexpr (M == 2) {
      const float r1 = wave_sum_f32(acc[1][t]);
      if (lane == 0) a.h[(size_t)t * a.N + n] = swiglu_bf16(r0, r1);
    } else {
      if (lane == 0) {
        float* const yp = a.y + (size_t)t * a.N + n;
        *yp = a.accumulate ? *yp + r0 : r0;
      }
    }
  }
}

}  // namespace moe_fp4
