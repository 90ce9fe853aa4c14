// Seeded synthetic expert-weight generator, device side.
//
// Input generation only: nothing here is part of the MoE arithmetic.  This is
// the device twin of gen_host.c and produces the same bytes: the counter-based
// SplitMix64 stream described there (Steele, Lea & Flood, OOPSLA 2014, with the
// finaliser constants of Vigna's splitmix64.c).  Generating on the device lets
// multi-gigabyte weight sets (one 384-expert layer is 7.2 GB, a 40-layer pruned
// stack 104 GB) be made in HBM directly instead of being staged from the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t sm64_at(uint64_t state, uint64_t i) {
  return sm64_mix(state + (i + 1) * kGamma);
}

// One thread writes one 8-byte word of uniform bytes (kind 0).
__global__ void fill_bytes_words(uint8_t* __restrict__ dst, int32_t n_exp, int64_t words_per_expert,
                                 int64_t expert_stride, uint64_t seed, uint32_t layer,
                                 uint32_t expert0, uint32_t tensor) {
  const int64_t total = (int64_t)n_exp * words_per_expert;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = g / words_per_expert;
    const int64_t w = g - e * words_per_expert;
    const uint64_t ctr = ((uint64_t)layer << 32) | ((uint64_t)(expert0 + e) << 8) | (tensor & 0xFF);
    const uint64_t st = sm64_at(seed, ctr);
    *reinterpret_cast<uint64_t*>(dst + e * expert_stride + w * 8) = sm64_at(st, (uint64_t)w);
  }
}

// One thread writes one byte (kind 0 unaligned fallback, or kind 1 scales).
__global__ void fill_bytes_single(uint8_t* __restrict__ dst, int32_t n_exp, int64_t bytes_per_expert,
                                  int64_t expert_stride, uint64_t seed, uint32_t layer,
                                  uint32_t expert0, uint32_t tensor, int kind, int lo, int hi) {
  const int64_t total = (int64_t)n_exp * bytes_per_expert;
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = g / bytes_per_expert;
    const int64_t o = g - e * bytes_per_expert;
    const uint64_t ctr = ((uint64_t)layer << 32) | ((uint64_t)(expert0 + e) << 8) | (tensor & 0xFF);
    const uint64_t st = sm64_at(seed, ctr);
    uint8_t v;
    if (kind == 0) {
      v = (uint8_t)(sm64_at(st, (uint64_t)(o >> 3)) >> (8 * (o & 7)));
    } else {
      v = (uint8_t)(lo + (int)(((sm64_at(st, (uint64_t)o) >> 32) * span) >> 32));
    }
    dst[e * expert_stride + o] = v;
  }
}

}  // namespace

// Fill n_exp experts of one weight tensor.  Expert i (0-based within this call)
// is generator expert expert0+i and lands at dst + i*expert_stride.
// kind 0: uniform bytes; kind 1: scale bytes in [lo, hi].  Returns a hipError_t.
extern "C" int synth_fill_tensor_dev(uint8_t* dst, int32_t n_exp, int64_t bytes_per_expert,
                                     int64_t expert_stride, uint64_t seed, uint32_t layer,
                                     uint32_t expert0, uint32_t tensor, int kind, int lo, int hi,
                                     void* stream) {
  if (n_exp <= 0 || bytes_per_expert <= 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int threads = 256;
  const bool words = kind == 0 && bytes_per_expert % 8 == 0 && expert_stride % 8 == 0 &&
                     (reinterpret_cast<uintptr_t>(dst) & 7) == 0;
  if (words) {
    const int64_t wpe = bytes_per_expert / 8;
    int64_t blocks = ((int64_t)n_exp * wpe + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_bytes_words, dim3((unsigned)blocks), dim3(threads), 0, s, dst, n_exp,
                       wpe, expert_stride, seed, layer, expert0, tensor);
  } else {
    int64_t blocks = ((int64_t)n_exp * bytes_per_expert + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_bytes_single, dim3((unsigned)blocks), dim3(threads), 0, s, dst, n_exp,
                       bytes_per_expert, expert_stride, seed, layer, expert0, tensor, kind, lo, hi);
  }
  return (int)hipGetLastError();
}
