// Device-side helpers shared by the moe_fp4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// UE8M0 scale byte -> fp32 2^(e-127): byte 0 is 2^-127 (an fp32 subnormal)
// and 255 is NaN, as in the OCP MX format.  The library supports e in
// [2, 252], where every scaled E2M1 value is a normal number.
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  const uint32_t b = e == 0u ? 0x00400000u : e == 255u ? 0x7FC00000u : e << 23;
  return __uint_as_float(b);
}

// Eight E2M1 codes packed in one dword (code 2i in the low nibble of byte i,
// code 2i+1 in its high nibble) -> eight bf16 values times `scale`, in code
// order.  v_cvt_scalef32_pk_bf16_fp4 converts the two codes of one byte.
// Every E2M1 value times a power of two in the supported scale range is exact
// in bf16, so no rounding happens here.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// silu(g) * u in fp32, then one rounding to bf16.  silu(g) = g * sigmoid(g).
// For g < 0 the exponential is taken of g itself (never overflows), and below
// g = -64 of g + 64 (exact for g >= -128), the product being multiplied by
// fp32(e^-64) at the end: e^g would otherwise be an fp32 subnormal with few
// significant bits while silu(g) * u can still be a normal bf16 (|u| is large
// when the scales are).  The relative error stays within a few fp32 ulps.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
  constexpr float kExpM64 = 0x1.969d48p-93f;   // e^-64 rounded to fp32
  if (g >= 0.0f) return f32_to_bf16_rne(g / (1.0f + expf(-g)) * u);
  const bool deep = g < -64.0f;
  const float e = expf(deep ? g + 64.0f : g);  // e^g, times e^64 when deep
  const float s = deep ? e : e / (1.0f + e);   // sigmoid(g) (1 + e^g rounds to 1 when deep)
  const float h = (g * s) * u;
  return f32_to_bf16_rne(deep ? h * kExpM64 : h);
}

// 16x16x32 bf16 MFMA: D[i][j] += sum_k A[i][k] B[k][j].  Lane l supplies
// A row (l % 16) and B column (l % 16), each with the 8 k-values of k-slot
// (l / 16); it receives D rows 4*(l/16) .. +3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global or LDS load as a native vector (selects on it stay in registers;
// a ternary on HIP's struct-typed uint4 can be lowered through the stack).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ u32x4 sel4(bool ok, const u32x4& v) {
  return u32x4{ok ? v[0] : 0u, ok ? v[1] : 0u, ok ? v[2] : 0u, ok ? v[3] : 0u};
}

// Workgroup barrier for LDS traffic only.  __syncthreads() fences every address
// space, which makes each wave wait for all of its outstanding global loads
// (vmcnt(0)) before the barrier and so drains any prefetch in flight; this one
// waits only for the wave's own LDS operations (lgkmcnt(0)).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- wave-wide reductions with DPP: the four lanes of a quad exchange with
// quad_perm, rows of 16 with row_ror, and the four row results are read into
// scalar registers.  The result is uniform across the wave.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax32(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax32(v, dpp_u32<0x124>(v));  // row_ror:4
  v = umax32(v, dpp_u32<0x128>(v));  // row_ror:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return umax32(umax32(r0, r1), umax32(r2, r3));
}

// Sum over the 64 lanes of a wave in a fixed association order (quad, row,
// then rows 0+1 and 2+3), so the result is the same bits on every run.
// Uniform across the wave.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// The sums over lanes 0-31 (lo) and 32-63 (hi) of a wave, with the same DPP
// steps as wave_sum_f32: lo = row 0 + row 1, hi = row 2 + row 3.  Uniform.
__device__ __forceinline__ void wave_half_sums_f32(float v, float& lo, float& hi) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  lo = r0 + r1;
  hi = r2 + r3;
}

// sum_{i<8} a[i] * b[i] + c with bf16 products exact in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const bf16x8& b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[0], a[1]}, bf16x2{b[0], b[1]}, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[2], a[3]}, bf16x2{b[2], b[3]}, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[4], a[5]}, bf16x2{b[4], b[5]}, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[6], a[7]}, bf16x2{b[6], b[7]}, c, false);
  return c;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = umin32(v, dpp_u32<0xB1>(v));
  v = umin32(v, dpp_u32<0x4E>(v));
  v = umin32(v, dpp_u32<0x124>(v));
  v = umin32(v, dpp_u32<0x128>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return umin32(umin32(r0, r1), umin32(r2, r3));
}

// Pre-normalisation u = bf16(x / rms) of one fp32 row, rms = sqrt(mean(x^2) +
// eps), by a 512-thread workgroup.  Thread t owns the 8-value chunks t,
// t + 512, t + 1024, ... (chunk c holds elements 8 c .. 8 c + 7) and keeps
// them in registers, so the row is read once.  The sum of squares runs over
// the thread's chunks in that order and each chunk's values in order; each
// wave then reduces with the fixed DPP tree of wave_sum_f32, and the 8 wave
// sums are added in wave order.  The standalone pre-norm and the one fused
// into the one-token decode kernel both use these, so both give the same bits.
constexpr int kNormThreads = 512;

__device__ __forceinline__ float chunk_sumsq(const float4& a, const float4& b, float ss) {
  ss += a.x * a.x;
  ss += a.y * a.y;
  ss += a.z * a.z;
  ss += a.w * a.w;
  ss += b.x * b.x;
  ss += b.y * b.y;
  ss += b.z * b.z;
  ss += b.w * b.w;
  return ss;
}

// The workgroup's rms from each thread's partial sum ss (every thread of the
// 512 must call it: it has a barrier).  wsum: 8 floats of LDS.
__device__ __forceinline__ float block_rms(float ss, int H, float eps, float* wsum) {
  ss = wave_sum_f32(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  lds_barrier();  // wsum is the only data shared; loads in flight stay in flight
  float tot = wsum[0];
#pragma unroll
  for (int i = 1; i < kNormThreads / 64; ++i) tot += wsum[i];
  return sqrtf(tot / (float)H + eps);
}

// Eight values times 1 / r, rounded to bf16 and packed in order.
__device__ __forceinline__ u32x4 chunk_to_bf16(const float4& a, const float4& b, float r) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = (uint32_t)f32_to_bf16_rne(v[2 * j] / r) | ((uint32_t)f32_to_bf16_rne(v[2 * j + 1] / r) << 16);
  return o;
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Grouped-GEMM workgroups are dealt to the 8 XCDs round robin; give each XCD a
// contiguous run of `n` logical tiles, so that the tiles of one expert share an
// XCD's L2.  Returns false for padding blocks.
__device__ __forceinline__ bool xcd_tile(int n, int& logical) {
  const int per = (n + 7) / 8;
  const int slot = blockIdx.x >> 3;
  logical = (blockIdx.x & 7) * per + slot;
  return slot < per && logical < n;
}
inline unsigned xcd_grid(int n) { return (unsigned)(((n + 7) / 8) * 8); }

}  // namespace moe_fp4
