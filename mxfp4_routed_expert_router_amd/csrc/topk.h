// Router top-k shared by the routing kernels and the fused one-token decode
// kernel: one wave ranks one token's E logits (larger first, ties to the lower
// expert index, -0 equal to +0, NaN last) and forms the softmax over the k
// chosen logits.
#pragma once

#include "device_common.h"

namespace moe_fp4 {

// Monotone map of a float onto uint32: larger float -> larger key; -0 maps to
// the key of +0; NaN maps to 1, below the key of -inf (0x007FFFFF).  Key 0
// marks a slot that is empty or already chosen.
__device__ __forceinline__ uint32_t order_key(float v) {
  // selects only: a branch here would let the compiler sink the logit loads
  // into it, each then waited for before the next is issued
  uint32_t u = __float_as_uint(v);
  u = (u << 1) == 0u ? 0u : u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 1u : key;
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Lane l's logits l, l+64, ... of one token row.  The loads are unconditional
// (a clamped index, the value discarded past E): inside a branch each one would
// be waited for before the next is issued.
template <int VPL>
__device__ __forceinline__ void wave_load_logits(const float* __restrict__ lrow, int E, int lane,
                                                 float (&vals)[VPL]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    vals[i] = lrow[e < E ? e : E - 1];
  }
}

// A ranking in progress: one wave holds the E logits of one token (lane l the
// keys of logits l, l+64, ... as wave_load_logits leaves them), and each call
// of next() takes the largest remaining one: the wave-wide maximum key (DPP),
// among lanes holding it the lowest expert id, which is then cleared.  Rounds
// can be spread over a kernel's prologue.  Requires all 64 lanes active.
template <int VPL>
struct WaveRanking {
  uint32_t keys[VPL];
  int lane;

  __device__ __forceinline__ void init(const float (&vals)[VPL], int E, int lane_) {
    lane = lane_;
#pragma unroll
    for (int i = 0; i < VPL; ++i)  // a mask, not a select: see wave_load_logits
      keys[i] = order_key(vals[i]) & (0u - (uint32_t)(lane + kWave * i < E));
  }

  // The expert of the next rank (uniform over the wave); its key in m.
  __device__ __forceinline__ uint32_t next(uint32_t& m) {
    uint32_t bk = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (keys[i] > bk) { bk = keys[i]; bi = i; }  // strict: lower slot (lower id) wins ties
    m = wave_max_u32(bk);
    const uint64_t tied = __ballot(bk == m);
    uint32_t e_win;
    if (__popcll(tied) == 1) {
      e_win = (uint32_t)__builtin_amdgcn_readlane(lane + kWave * bi,
                                                  (int)(__ffsll((long long)tied) - 1));
    } else {
      e_win = wave_min_u32(bk == m ? (uint32_t)(lane + kWave * bi) : 0xFFFFFFFFu);
    }
    // clear the taken key: a select in every lane, no branch
    const uint32_t kill = (int)(e_win & (kWave - 1)) == lane ? 1u << (e_win >> 6) : 0u;
#pragma unroll
    for (int i = 0; i < VPL; ++i) keys[i] = (kill >> i) & 1u ? 0u : keys[i];
    return e_win;
  }
};

// The softmax over the k chosen logits: lane j < k holds the logit of rank j
// (my_v), v0 is the largest.  One exp per lane, and the denominator summed in
// rank order from the lanes' terms.
__device__ __forceinline__ float rank_gate(float my_v, float v0, int k) {
  const float ev = expf(my_v - v0);
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ev), j));
  return ev / s;
}

// One wave ranks the E logits of one token (vals as wave_load_logits leaves
// them); lane j < k receives the expert of rank j and its gate.  Requires
// k <= E and all 64 lanes active.
template <int VPL>
__device__ __forceinline__ void wave_topk_vals(const float (&vals)[VPL], int E, int k, int lane,
                                               int& e_out, float& g_out) {
  WaveRanking<VPL> rk;
  rk.init(vals, E, lane);
  int my_e = 0;
  float my_v = 0.f, v0 = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t m;
    const uint32_t e_win = rk.next(m);
    const float v = key_value(m);
    if (j == 0) v0 = v;
    if (j == lane) { my_e = (int)e_win; my_v = v; }
  }
  e_out = my_e;
  g_out = rank_gate(my_v, v0, k);
}

// As wave_topk_vals, loading the logits itself.
template <int VPL>
__device__ __forceinline__ void wave_topk_regs(const float* __restrict__ lrow, int E, int k,
                                               int lane, int& e_out, float& g_out) {
  float vals[VPL];
  wave_load_logits<VPL>(lrow, E, lane, vals);
  wave_topk_vals<VPL>(vals, E, k, lane, e_out, g_out);
}

// As wave_topk_regs, writing the k experts and gates to idx_out / g_out.
template <int VPL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lrow, int E, int k, int lane,
                                          int32_t* __restrict__ idx_out, float* __restrict__ g_out) {
  int e;
  float g;
  wave_topk_regs<VPL>(lrow, E, k, lane, e, g);
  if (lane < k) {
    idx_out[lane] = e;
    g_out[lane] = g;
  }
}

}  // namespace moe_fp4
