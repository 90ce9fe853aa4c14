// Saliency side output of the prefill w2 GEMMs (the pruning signal of the
// 10100.com page, section on choosing experts by frequency or saliency:
// router weight times the L2 norm of the expert's output, summed over the
// tokens).  Each w2 workgroup tile reduces the squares of its rows per token
// into sal_part; launch_saliency takes the square roots and the gate-weighted
// sums per expert, in a fixed order.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe_fp4 {

// Saliency partial of one w2 tile, called by all threads of a 512-thread
// workgroup after a pass: acc[m][rt][nt] holds the wave's rows 16 rt + 4 (l/16)
// .. +3 (valid where act[rt]) for tokens 16 nt + l % 16.  Each wave's sum of
// squares per token is reduced over its lanes, the 8 wave sums of a token are
// added in wave order, and the total goes to sal_part[(slot0 + token) * tiles
// + tile] for tokens < nc.  red: 8 x 64 floats of LDS.
template <int RT, int NT>
__device__ __forceinline__ void saliency_tile(const LayerArgs& a, const f32x4 (&acc)[1][RT][NT],
                                              const bool (&act)[RT], float* red, int slot0, int nc,
                                              int tile) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float ss = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      if (act[rt])
#pragma unroll
        for (int q = 0; q < 4; ++q) ss += acc[0][rt][nt][q] * acc[0][rt][nt][q];
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16) red[w * 64 + 16 * nt + lane] = ss;
  }
  __syncthreads();
  if (tid < nc) {
    float s = 0.f;
    for (int q = 0; q < 8; ++q) s += red[q * 64 + tid];
    a.sal_part[(size_t)(slot0 + tid) * a.sal_tiles + tile] = s;
  }
  __syncthreads();
}

}  // namespace moe_fp4
