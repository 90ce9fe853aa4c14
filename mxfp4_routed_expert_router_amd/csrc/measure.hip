// Measurement companion of the layer library (libmoe_fp4_measure.so, loaded by
// the benchmark only): a plain streaming read, so that the decode kernels'
// bandwidth can be set beside what one kernel reading the same number of bytes
// reaches on this GPU, not only beside the nominal HBM peak.
//
// Workgroup g of G reads the 16 KB chunks g, g + G, g + 2G, ... of the buffer:
// thread t loads 16 bytes at t * 16 + j * blockDim * 16 for j < UNROLL (all
// loads of a chunk in flight before the first is used), and folds every dword
// into an xor that it stores once, so no load can be dropped.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16, uint32_t* sink) {
  const size_t per = (size_t)blockDim.x * UNROLL;  // 16-byte loads per chunk
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c * per < n16; c += gridDim.x) {
    const size_t base = c * per + threadIdx.x;
    u32x4 v[UNROLL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const size_t i = base + (size_t)j * blockDim.x;
      v[j] = buf[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {
// Read `bytes` (a multiple of 16) at `buf` with `grid` workgroups of `threads`
// threads (64..1024, a multiple of 64), `unroll` (4, 8 or 16) loads in flight
// per thread; `sink` holds grid * threads uint32.  `start` / `stop` (may be
// null) are recorded by the dispatch itself, so their elapsed time is the
// kernel's duration.  Returns 0, 1 on bad arguments, 2 on a launch error.
int moe_fp4_measure_stream_read(const void* buf, size_t bytes, int grid, int threads, int unroll,
                                uint32_t* sink, hipEvent_t start, hipEvent_t stop,
                                hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || grid <= 0 || threads < 64 || threads > 1024 ||
      threads % 64)
    return 1;
  const size_t n16 = bytes / 16;
  const auto* p = static_cast<const u32x4*>(buf);
  switch (unroll) {
    case 4:
      hipExtLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(threads), 0, stream, start, stop,
                            0u, p, n16, sink);
      break;
    case 8:
      hipExtLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(threads), 0, stream, start, stop,
                            0u, p, n16, sink);
      break;
    case 16:
      hipExtLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(threads), 0, stream, start, stop,
                            0u, p, n16, sink);
      break;
    default:
      return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
}
