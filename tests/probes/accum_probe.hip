// Accumulation probes for the parity tests (test infrastructure, not part of
// the layer library).  Each kernel runs one matrix-core or dot-product
// instruction of the kind the layer's kernels chain, on inputs the test
// chooses, and returns the fp32 result, so that the test can measure how far
// one instruction's result may stray from the exact sum of its terms.  The h
// checks bound a kernel's fp32 evaluation of G and U by chaining these
// per-instruction bounds along its longest accumulation path.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

// d[i] = a[i].lo * b[i].lo + a[i].hi * b[i].hi + c[i]  (v_dot2c_f32_bf16)
__global__ void dot2_kernel(const uint32_t* a, const uint32_t* b, const float* c, float* d, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const bf16x2 x = __builtin_bit_cast(bf16x2, a[i]);
  const bf16x2 y = __builtin_bit_cast(bf16x2, b[i]);
  d[i] = __builtin_amdgcn_fdot2_f32_bf16(x, y, c[i], false);
}

// One 16x16x32 bf16 MFMA per wave: D = C + A B for A [16][32], B [32][16]
// (bf16 bits, row-major) and C, D [16][16] fp32.  Lane l supplies A row l % 16
// and B column l % 16 with k-values 8 (l / 16) .. +7; it holds D rows
// 4 (l / 16) .. +3 of column l % 16.
__global__ void mfma_bf16_kernel(const uint16_t* A, const uint16_t* B, const float* C, float* D,
                                 int n) {
  const int p = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (p >= n) return;
  const int l = threadIdx.x & 63, r = l & 15, kb = l >> 4;
  const uint16_t* Ap = A + (size_t)p * 512;
  const uint16_t* Bp = B + (size_t)p * 512;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(__bf16, Ap[r * 32 + 8 * kb + j]);
    b[j] = __builtin_bit_cast(__bf16, Bp[(8 * kb + j) * 16 + r]);
  }
  f32x4 acc;
  for (int q = 0; q < 4; ++q) acc[q] = C[(size_t)p * 256 + (4 * kb + q) * 16 + r];
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  for (int q = 0; q < 4; ++q) D[(size_t)p * 256 + (4 * kb + q) * 16 + r] = acc[q];
}

// One scaled 16x16x128 MFMA per wave with E2M1 A and E4M3 B:
// D = C + sum_k A[i][k] 2^(sa[i][k/32]-127) B[k][j] 2^(sb[j][k/32]-127).
// A: [16][64] bytes (two codes a byte, low nibble = even k); sa [16][4];
// B: [16][128] bytes, column-major by token j (B[k][j] at j * 128 + k);
// sb [16][4].  Lane l supplies A row l % 16, k = 32 (l/16) .. +31 (16 bytes)
// with scale sa[l % 16][l / 16], and B column l % 16, k = 16 (l/16) .. +15 and
// 64 + 16 (l/16) .. +15, with scale sb[l % 16][l / 16].
__global__ void mfma_scale_kernel(const uint8_t* A, const uint8_t* sa, const uint8_t* B,
                                  const uint8_t* sb, const float* C, float* D, int n) {
  const int p = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (p >= n) return;
  const int l = threadIdx.x & 63, r = l & 15, kb = l >> 4;
  const uint32_t* Ap = reinterpret_cast<const uint32_t*>(A + (size_t)p * 1024 + r * 64 + 16 * kb);
  const uint32_t* B0 = reinterpret_cast<const uint32_t*>(B + (size_t)p * 2048 + r * 128 + 16 * kb);
  const uint32_t* B1 = reinterpret_cast<const uint32_t*>(B + (size_t)p * 2048 + r * 128 + 64 + 16 * kb);
  const i32x8 av = {(int)Ap[0], (int)Ap[1], (int)Ap[2], (int)Ap[3], 0, 0, 0, 0};
  const i32x8 bv = {(int)B0[0], (int)B0[1], (int)B0[2], (int)B0[3],
                    (int)B1[0], (int)B1[1], (int)B1[2], (int)B1[3]};
  const int s_a = sa[(size_t)p * 64 + r * 4 + kb], s_b = sb[(size_t)p * 64 + r * 4 + kb];
  f32x4 acc;
  for (int q = 0; q < 4; ++q) acc[q] = C[(size_t)p * 256 + (4 * kb + q) * 16 + r];
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 0, 0, s_a, 0, s_b);
  for (int q = 0; q < 4; ++q) D[(size_t)p * 256 + (4 * kb + q) * 16 + r] = acc[q];
}

}  // namespace

extern "C" {
int probe_dot2(const uint32_t* a, const uint32_t* b, const float* c, float* d, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(dot2_kernel, dim3((n + 255) / 256), dim3(256), 0, 0, a, b, c, d, n);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
int probe_mfma_bf16(const uint16_t* A, const uint16_t* B, const float* C, float* D, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3((n + 3) / 4), dim3(256), 0, 0, A, B, C, D, n);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
int probe_mfma_scale(const uint8_t* A, const uint8_t* sa, const uint8_t* B, const uint8_t* sb,
                     const float* C, float* D, int n) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_scale_kernel, dim3((n + 3) / 4), dim3(256), 0, 0, A, sa, B, sb, C, D, n);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
}
