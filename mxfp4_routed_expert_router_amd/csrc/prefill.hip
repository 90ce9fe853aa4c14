// Prefill path (register-fed GEMMs here; prefill_lds.hip holds LDS-fed ones,
// used where K is a multiple of 256): a chunk of many tokens, so each expert's weights are read once
// and reused by every token routed to it -- the reason prefill is far faster per
// token than decode (ai-shiz.ru page, section on prefill; the 10100.com page uses
// 2048-token prefill chunks, section on KV and prefill workspace).  Per expert
// this is a small-M grouped GEMM; at DeepSeek-V4.1-Flash shapes (about 32 tokens
// per expert) it stays bound by the weight stream from HBM, with the MFMA units
// well below their peak.
//
//   gemm13   workgroup = (expert, 128 rows of w1/w3): 8 waves x 16 rows.  K advances in blocks of 128 inputs
//            (4 scale groups).  Each wave keeps its next kPF blocks of packed
//            weights in flight in a register ring; the gathered token rows of x
//            for a block are fetched kPF blocks ahead into registers as well and
//            written to a double-buffered LDS tile one block ahead, so every
//            wait is for the oldest loads and the prefetch never drains.  The
//            weights are decoded in registers straight into MFMA A operands.
//            Epilogue: h = bf16(silu(G) U).
//   gemm2    workgroup = (expert, 256 rows of w2): 8 waves x 32 rows (two
//            16-row MFMA tiles per wave); B = the expert's h rows.
//            Epilogue: ypair = gate * Y (fp32), one row per (token, expert) pair.
//   combine  y[t] = sum_j ypair[slot(t, j)], j ascending: deterministic.
// Workgroups are dealt to the eight XCDs so that the row tiles of one expert
// share an XCD and its L2 serves their common token rows.
#include "device_common.h"
#include "kernels.h"
#include "saliency.h"

namespace moe_fp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kRT13 = 1;                  // 16-row MFMA tiles per wave, w1/w3 pass
constexpr int kRT2 = 2;                   // 16-row MFMA tiles per wave, w2 pass
constexpr int kRows13 = 16 * kRT13 * kWaves;  // weight rows per workgroup
constexpr int kRows2 = 16 * kRT2 * kWaves;
constexpr int kTok = 64;                  // tokens per pass
constexpr int kKB = 128;                  // inputs per K block (4 scale groups)
constexpr int kXS = kKB + 8;              // LDS row stride in bf16: rows 4 banks apart
constexpr int kPF13 = 3;                  // K blocks in flight per wave, w1/w3 pass
constexpr int kPF2 = 4;                   // K blocks in flight per wave, w2 pass
constexpr int kXC = (kTok * kKB / 8) / kThreads;  // 16-byte activation chunks per thread, block

struct Smem {
  uint16_t xs[2][kTok][kXS];
  int row[kTok];
  float sal[kWaves * 64];  // saliency reduction (saliency.h)
};



// One pass over all K for up to NT*16 staged token rows (sm.row[n] for n < nc,
// row length ld in src): acc[m][rt][nt] = W_m[rows of tile rt] . X^T[tokens of nt].
// M weight matrices share the activation tile.  Row tiles with act[rt] false
// read a valid chunk they do not use (scale 0) but the wave still takes part
// in the staging and the barriers.  NT (16-token column tiles) is a template
// argument so that the MFMA loop has no branches: a branch around MFMAs makes
// the compiler copy the accumulators at every join.
template <int M, int kPF, int kRT, int NT>
__device__ __forceinline__ void gemm_pass(Smem& sm, const uint8_t* const (&wr)[M][kRT],
                                          const uint8_t* const (&sr)[M][kRT], const bool (&act)[kRT],
                                          const uint16_t* __restrict__ src, int ld, int nc, int K,
                                          f32x4 (&acc)[M][kRT][NT]) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int c16 = lane & 15, kb = lane >> 4;
  const int NG = K / 32, NB = (K + kKB - 1) / kKB;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[m][rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 q[kPF][M][kRT];
  uint32_t sv[kPF][M][kRT];
  u32x4 xv[kPF][kXC];
  // Every load is issued unconditionally from an address that is always valid
  // (out-of-range blocks, rows or tokens read row 0 / token 0 / block 0), and
  // validity is applied where the value is used: a weight chunk past the end
  // gets scale 0 (every E2M1 code times 0 is 0), an activation chunk past the
  // end is stored to LDS as zeros.  A select on a loaded register right after
  // its load would make the compiler wait for it there (and at the loop's back
  // edge), draining the prefetch; with no branches and no selects around the
  // loads each wait is for the oldest block only.
  auto w_ok = [&](int b, int rt) { return b < NB && act[rt] && 4 * b + kb < NG; };
  auto x_ok = [&](int b, int u) {
    const int id = tid + u * kThreads;
    const int n = id / (kKB / 8), c = id % (kKB / 8);
    return b < NB && n < nc && b * kKB + c * 8 < K;
  };
  auto issue_w = [&](int b, int s) {
    const int g = 4 * b + kb;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int gg = w_ok(b, rt) ? g : 0;
        q[s][m][rt] = ld16(wr[m][rt] + (size_t)gg * 16);
        sv[s][m][rt] = sr[m][rt][gg];
      }
  };
  auto issue_x = [&](int b, int s) {
#pragma unroll
    for (int u = 0; u < kXC; ++u) {
      const int id = tid + u * kThreads;
      const int n = id / (kKB / 8), c = id % (kKB / 8);
      const bool ok = x_ok(b, u);
      xv[s][u] = ld16(src + (size_t)sm.row[ok ? n : 0] * ld + (ok ? b * kKB + c * 8 : 0));
    }
  };
  auto write_x = [&](int s, int buf, int b) {
#pragma unroll
    for (int u = 0; u < kXC; ++u) {
      const int id = tid + u * kThreads;
      const int n = id / (kKB / 8), c = id % (kKB / 8);
      st16(&sm.xs[buf][n][c * 8], sel4(x_ok(b, u), xv[s][u]));
    }
  };
  auto compute = [&](int s, int buf, int b) {
    float sc[M][kRT];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) sc[m][rt] = w_ok(b, rt) ? ue8m0_to_f32(sv[s][m][rt]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 A[M][kRT];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) A[m][rt] = fp4x8_to_bf16x8(q[s][m][rt][i], sc[m][rt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 B = as_bf16x8(ld16(&sm.xs[buf][16 * nt + c16][kb * 32 + 8 * i]));
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) acc[m][rt][nt] = mfma16x16x32(A[m][rt], B, acc[m][rt][nt]);
      }
    }
  };

  // Prologue: blocks 0..kPF-1 in flight, block 0's activations in LDS.  The
  // loop body is the same for every block; blocks past the end (at most
  // kPF - 1 of them in the last round) compute on zeros.
#pragma unroll
  for (int s = 0; s < kPF; ++s) {
    issue_x(s, s);
    issue_w(s, s);
  }
  write_x(0, 0, 0);
  for (int b0 = 0; b0 < NB; b0 += kPF) {
#pragma unroll
    for (int s = 0; s < kPF; ++s) {
      const int b = b0 + s;
      lds_barrier();  // block b's tile is in LDS; the other buffer is free
      write_x((s + 1) % kPF, (b + 1) & 1, b + 1);
      compute(s, b & 1, b);
      issue_x(b + kPF, s);
      issue_w(b + kPF, s);
    }
  }
  lds_barrier();
}

__global__ void __launch_bounds__(kThreads, 1) gemm13_kernel(LayerArgs a) {
  const int tpe = (a.I + kRows13 - 1) / kRows13;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  // both loads in flight at once: the test reads both (off is never negative),
  // so the compiler cannot sink the second below it
  const int ne = a.counts[e], off = a.offsets[e];
  if (ne == 0 || off < 0) return;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int c16 = lane & 15, kb = lane >> 4;
  const int rw = rtile * kRows13 + w * (16 * kRT13);  // this wave's first row
  const size_t wrow = (size_t)a.H / 2, srow = (size_t)a.H / 32;
  bool act[kRT13];
  const uint8_t* wr[2][kRT13];
  const uint8_t* sr[2][kRT13];
#pragma unroll
  for (int rt = 0; rt < kRT13; ++rt) {
    const int r = rw + 16 * rt;
    act[rt] = r < a.I;
    const size_t ro = (size_t)(act[rt] ? r + c16 : 0);
    wr[0][rt] = a.w1 + (size_t)e * a.stride[0] + ro * wrow;
    sr[0][rt] = a.s1 + (size_t)e * a.stride[1] + ro * srow;
    wr[1][rt] = a.w3 + (size_t)e * a.stride[2] + ro * wrow;
    sr[1][rt] = a.s3 + (size_t)e * a.stride[3] + ro * srow;
  }
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (tid < nc) sm.row[tid] = a.slot_tok[off + c0 + tid];
    lds_barrier();
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[2][kRT13][NT];
      gemm_pass<2, kPF13, kRT13, NT>(sm, wr, sr, act, a.x, a.H, nc, a.H, acc);
#pragma unroll
      for (int rt = 0; rt < kRT13; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int tok = 16 * nt + c16;
          if (act[rt] && tok < nc) {
            uint16_t hv[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) hv[qq] = swiglu_bf16(acc[0][rt][nt][qq], acc[1][rt][nt][qq]);
            const uint2 pk = {(uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                              (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
            *reinterpret_cast<uint2*>(a.h + (size_t)(off + c0 + tok) * a.I + rw + 16 * rt + 4 * kb) = pk;
          }
        }
    };
    switch ((nc + 15) / 16) {
      case 1: pass(IntC<1>{}); break;
      case 2: pass(IntC<2>{}); break;
      case 3: pass(IntC<3>{}); break;
      default: pass(IntC<4>{}); break;
    }
  }
}

__global__ void __launch_bounds__(kThreads, 1) gemm2_kernel(LayerArgs a) {
  const int tpe = (a.H + kRows2 - 1) / kRows2;
  int logical;
  if (!xcd_tile(a.E * tpe, logical)) return;
  const int e = logical / tpe, rtile = logical - e * tpe;
  // both loads in flight at once: the test reads both (off is never negative),
  // so the compiler cannot sink the second below it
  const int ne = a.counts[e], off = a.offsets[e];
  if (ne == 0 || off < 0) return;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int c16 = lane & 15, kb = lane >> 4;
  const int rw = rtile * kRows2 + w * (16 * kRT2);
  const size_t wrow = (size_t)a.I / 2, srow = (size_t)a.I / 32;
  bool act[kRT2];
  const uint8_t* wr[1][kRT2];
  const uint8_t* sr[1][kRT2];
#pragma unroll
  for (int rt = 0; rt < kRT2; ++rt) {
    const int r = rw + 16 * rt;
    act[rt] = r < a.H;
    const size_t ro = (size_t)(act[rt] ? r + c16 : 0);
    wr[0][rt] = a.w2 + (size_t)e * a.stride[4] + ro * wrow;
    sr[0][rt] = a.s2 + (size_t)e * a.stride[5] + ro * srow;
  }
  for (int c0 = 0; c0 < ne; c0 += kTok) {
    const int nc = min(kTok, ne - c0);
    if (tid < nc) sm.row[tid] = off + c0 + tid;
    lds_barrier();
    auto pass = [&](auto nt_const) {
      constexpr int NT = decltype(nt_const)::value;
      f32x4 acc[1][kRT2][NT];
      gemm_pass<1, kPF2, kRT2, NT>(sm, wr, sr, act, a.h, a.I, nc, a.I, acc);
#pragma unroll
      for (int rt = 0; rt < kRT2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int tok = 16 * nt + c16;
          if (act[rt] && tok < nc) {
            const int s = off + c0 + tok;
            const float gate = a.slot_gate[s];
            const f32x4 v = acc[0][rt][nt];
            const float4 o = {gate * v[0], gate * v[1], gate * v[2], gate * v[3]};
            *reinterpret_cast<float4*>(a.ypair + (size_t)s * a.H + rw + 16 * rt + 4 * kb) = o;
          }
        }
      if (a.sal_part) saliency_tile<kRT2, NT>(a, acc, act, sm.sal, off + c0, nc, rtile);
    };
    switch ((nc + 15) / 16) {
      case 1: pass(IntC<1>{}); break;
      case 2: pass(IntC<2>{}); break;
      case 3: pass(IntC<3>{}); break;
      default: pass(IntC<4>{}); break;
    }
  }
}

// y[t] = (y[t] if accumulating) + sum_j ypair[pair_slot[t*k + j]], j ascending.
__global__ void __launch_bounds__(256) combine_kernel(LayerArgs a) {
  const int t = blockIdx.y;
  const int m4 = blockIdx.x * 256 + threadIdx.x;
  if (m4 * 4 >= a.H) return;
  float4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.k; ++j) {
    const int slot = a.pair_slot[t * a.k + j];
    const float4 v = *reinterpret_cast<const float4*>(a.ypair + (size_t)slot * a.H + m4 * 4);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  float4* yp = reinterpret_cast<float4*>(a.y + (size_t)t * a.H + m4 * 4);
  if (a.accumulate) {
    const float4 o = *yp;
    s.x = o.x + s.x; s.y = o.y + s.y; s.z = o.z + s.z; s.w = o.w + s.w;
  }
  *yp = s;
}

// saliency[e] += sum over e's sorted slots (ascending) of gate * sqrt(sum of the
// slot's tile partials, in tile order); one wave per expert, lanes strided over
// the slots and reduced in a fixed DPP order.
__global__ void __launch_bounds__(kWave) saliency_kernel(LayerArgs a, float* __restrict__ sal) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int n = a.counts[e], off = a.offsets[e];
  float v = 0.f;
  for (int i = lane; i < n; i += kWave) {
    const float* p = a.sal_part + (size_t)(off + i) * a.sal_tiles;
    float ss = 0.f;
    for (int t = 0; t < a.sal_tiles; ++t) ss += p[t];
    v += a.slot_gate[off + i] * sqrtf(ss);
  }
  v = wave_sum_f32(v);
  if (lane == 0) sal[e] += v;
}

// h rows from sorted (by-expert) order to pair order, for the debug entry point.
__global__ void unsort_h_kernel(const uint16_t* __restrict__ hs, const int32_t* __restrict__ slot,
                                int P, int I, uint16_t* __restrict__ out) {
  const size_t n = (size_t)P * I;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x) {
    const size_t p = q / I, c = q - p * I;
    out[q] = hs[(size_t)slot[p] * I + c];
  }
}

}  // namespace

hipError_t launch_combine(const LayerArgs& a, hipStream_t stream) {
  launch_k(combine_kernel, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, stream, ev_start(a.ev, 3),
           ev_stop(a.ev, 3), a);
  return hipGetLastError();
}

hipError_t launch_prefill(const LayerArgs& a, hipStream_t stream) {
  const dim3 blk(kThreads);
  const hipEvent_t* ev = a.ev;
  const int t13 = a.E * ((a.I + kRows13 - 1) / kRows13), t2 = a.E * ((a.H + kRows2 - 1) / kRows2);
  const uint8_t* const s13[2] = {a.s1, a.s3};
  const int64_t st13[2] = {a.stride[1], a.stride[3]};
  // (each launcher returns hipGetLastError(), which also clears the error:
  // its result is the only report of a failed launch)
  hipError_t e;
  if (prefill_lds_takes(a.H, s13, st13, 2)) {
    e = launch_gemm13_lds(a, stream, ev_start(ev, 1), ev_stop(ev, 1));
  } else {
    launch_k(gemm13_kernel, dim3(xcd_grid(t13)), blk, 0, stream, ev_start(ev, 1), ev_stop(ev, 1), a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (prefill_lds_takes(a.I, &a.s2, &a.stride[5], 1)) {
    e = launch_gemm2_lds(a, stream, ev_start(ev, 2), ev_stop(ev, 2));
  } else {
    launch_k(gemm2_kernel, dim3(xcd_grid(t2)), blk, 0, stream, ev_start(ev, 2), ev_stop(ev, 2), a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return launch_combine(a, stream);
}

hipError_t launch_saliency(const LayerArgs& a, float* saliency, hipStream_t stream) {
  hipLaunchKernelGGL(saliency_kernel, dim3(a.E), dim3(kWave), 0, stream, a, saliency);
  return hipGetLastError();
}

static_assert(kRows2 == kSalRows, "saliency tiles are the w2 workgroup tiles");

hipError_t launch_unsort_h(const LayerArgs& a, uint16_t* h_out, hipStream_t stream) {
  const int P = a.T * a.k;
  size_t blocks = ((size_t)P * a.I + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(unsort_h_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.h,
                     a.pair_slot, P, a.I, h_out);
  return hipGetLastError();
}

}  // namespace moe_fp4
