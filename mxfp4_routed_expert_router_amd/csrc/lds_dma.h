// Direct global->LDS loads for the grouped-GEMM main loops (gfx950, wave64).
//
// global_load_lds_dwordx4 / _dword write lane l's 16 or 4 bytes to LDS at
// M0 + 16 l or M0 + 4 l, so the blocks a loop keeps in flight cost no
// registers.  The loads are issued from inline assembly and the loops wait for
// them themselves (s_waitcnt vmcnt(n), n = this wave's loads still allowed in
// flight, counted by the loop): the compiler cannot tell which LDS bytes such
// a load writes and would otherwise wait for all of them before every LDS
// read.  A loop that uses these must issue no other global loads, so that its
// counts are exact; vector memory loads complete in issue order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
// The LDS base goes in as an m0 operand: the compiler sets m0 itself and knows
// that the instruction reads it.
__device__ __forceinline__ void lds_load16(uint32_t lds_base, const void* g) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}
// The same with the non-temporal hint, for data read once (weights): the L2
// keeps it at low priority, so reused activation rows stay resident.
__device__ __forceinline__ void lds_load16_nt(uint32_t lds_base, const void* g) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_load4(uint32_t lds_base, const void* g) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}
// Wait until at most N of this wave's loads are in flight, then meet the
// workgroup.  The memory clobber keeps the compiler's LDS accesses on their side.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Byte offset in a 16-row weight tile of 128 bytes a row (2 KB) of row r's
// 16-byte chunk c: rows 0-7 fill the first 1 KB, rows 8-15 the second, chunk
// slot c ^ (r & 7) ^ (r >> 3).  The reads of 16 lanes (16 rows, one chunk)
// then hit 16 different 16-byte bank groups.  One global_load_lds_dwordx4
// fills one half: lane l takes row 8 h + l / 8, slot l % 8, i.e. chunk
// (l % 8) ^ (l / 8) ^ h -- 8 lanes read each row's whole 128-byte line.
__device__ __forceinline__ int woff(int r, int c) {
  return (r >> 3) * 1024 + (r & 7) * 128 + ((c ^ (r & 7) ^ (r >> 3)) << 4);
}
__device__ __forceinline__ int wtile_chunk(int lane, int h) { return (lane & 7) ^ (lane >> 3) ^ h; }

}  // namespace moe_fp4
