// Router (top-k + softmax over the chosen logits) and token permutation grouped
// by expert (histogram, exclusive scan, stable scatter).
//
// What is computed follows the 10100.com page's description of the layer (each
// token picks 6 of the 384 routed experts of a layer) with the readings stated
// in include/moe_fp4.h: larger logit first, ties to the lower expert index, -0
// equal to +0, NaN last; gates are a softmax over the k chosen logits.  Every
// output is a deterministic function of the logits: the ranking is exact integer
// comparison and the scatter orders pairs by (expert, pair id) without relying on
// the order in which atomics land.
#include "device_common.h"
#include "kernels.h"
#include "topk.h"

namespace moe_fp4 {
namespace {

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ gates) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves leave together
  wave_topk<VPL>(logits + (size_t)t * E, E, k, lane, idx + (size_t)t * k, gates + (size_t)t * k);
}

// Inclusive scan across a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

template <int NTH>
struct PermSmem {
  static constexpr int kWaves = NTH / kWave;
  int cnt[kMaxExperts];
  int base[kMaxExperts];
  uint8_t wcnt[kWaves][kMaxExperts];
  int wsum[2 * kWave + 1];
};

// Exclusive scan of kMaxExperts values; thread t owns entries
// t*PER .. t*PER+PER-1 in `vals`, which it gets back as exclusive prefixes.
template <int NTH>
__device__ void block_excl_scan_e(int (&vals)[kMaxExperts / NTH], int* s_wsum, int* total) {
  constexpr int PER = kMaxExperts / NTH, NW = NTH / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int mine = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) mine += vals[q];
  const int inc = wave_incl_scan(mine, lane);
  if (lane == kWave - 1) s_wsum[w] = inc;
  lds_barrier();
  if (w == 0) {
    const int x = lane < NW ? s_wsum[lane] : 0;
    const int xi = wave_incl_scan(x, lane);
    if (lane < NW) s_wsum[kWave + lane] = xi - x;
    if (lane == NW - 1) s_wsum[2 * kWave] = xi;
  }
  lds_barrier();
  int run = inc - mine + s_wsum[kWave + w];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int v = vals[q];
    vals[q] = run;
    run += v;
  }
  *total = s_wsum[2 * kWave];
  lds_barrier();
}

template <int NTH>
__device__ void scatter_range(const int32_t* idx, int p0, int p1, int E, int k,
                              int32_t* sorted_pairs, int32_t* pair_slot, const float* gsrc,
                              float* slot_gate, int32_t* slot_tok, PermSmem<NTH>& sm);

// Histogram, scan and stable scatter of the P pairs of `idx` (LDS or global)
// by one NTH-thread block.  Pairs are taken in chunks of NTH in pair order;
// inside a chunk a pair's position is base[e] + (pairs of e in earlier waves of
// the chunk) + (pairs of e in earlier lanes of its wave), so the result is the
// stable order whatever the timing of the LDS atomics in the histogram.
// With `slot_gate` non-null, also writes per sorted slot the pair's gate
// (read from `gsrc`, LDS or global) and token (pair id / k).
template <int NTH>
__device__ void block_permute(const int32_t* idx, int P, int E, int k, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot,
                              int32_t* dinfo, int32_t* meta, const float* gsrc, float* slot_gate,
                              int32_t* slot_tok, PermSmem<NTH>& sm) {
  constexpr int NW = NTH / kWave, PER = kMaxExperts / NTH;
  const int tid = threadIdx.x;
  for (int e = tid; e < kMaxExperts; e += NTH) {
    sm.cnt[e] = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) sm.wcnt[q][e] = 0;
  }
  lds_barrier();
  for (int p = tid; p < P; p += NTH) atomicAdd(&sm.cnt[idx[p]], 1);
  lds_barrier();
  // offsets, and the ascending list of experts that received pairs
  int c[PER], f[PER], cc[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    cc[q] = c[q] = sm.cnt[tid * PER + q];
    f[q] = c[q] > 0 ? 1 : 0;
  }
  int total = 0, nd = 0;
  block_excl_scan_e<NTH>(c, sm.wsum, &total);
  block_excl_scan_e<NTH>(f, sm.wsum, &nd);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = tid * PER + q;
    if (e < E) {
      counts[e] = cc[q];
      offsets[e] = c[q];
      sm.base[e] = c[q];
      if (cc[q] > 0 && dinfo) {
        dinfo[4 * f[q] + 0] = e;
        dinfo[4 * f[q] + 1] = c[q];
        dinfo[4 * f[q] + 2] = cc[q];
        dinfo[4 * f[q] + 3] = 0;
      }
    }
  }
  if (tid == 0) {
    offsets[E] = total;
    if (meta) meta[0] = nd;
  }
  // records past the last distinct expert (up to the grid the expert kernels
  // launch, min(P, E)) say "no expert"
  if (dinfo)
    for (int x = nd + tid; x < (P < E ? P : E); x += NTH) dinfo[4 * x] = -1;
  lds_barrier();
  scatter_range<NTH>(idx, 0, P, E, k, sorted_pairs, pair_slot, gsrc, slot_gate, slot_tok, sm);
}

// Stable scatter of pairs p0 .. p1-1 (sm.base[e] = the sorted position of the
// first of them routed to expert e; sm.wcnt zero), in chunks of NTH in pair
// order: inside a chunk a pair's position is base[e] + (pairs of e in earlier
// waves of the chunk) + (pairs of e in earlier lanes of its wave), the lanes
// holding the same expert found by 11 ballots on the expert id's bits.
template <int NTH>
__device__ void scatter_range(const int32_t* idx, int p0, int p1, int E, int k,
                              int32_t* sorted_pairs, int32_t* pair_slot, const float* gsrc,
                              float* slot_gate, int32_t* slot_tok, PermSmem<NTH>& sm) {
  constexpr int NW = NTH / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  for (int c0 = p0; c0 < p1; c0 += NTH) {
    const int p = c0 + tid;
    const bool valid = p < p1;
    const int e = valid ? idx[p] : -1;
    // lanes of this wave holding the same expert
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (valid && rank == 0) sm.wcnt[w][e] = (uint8_t)__popcll(peers);
    lds_barrier();
    if (valid) {
      int pos = sm.base[e] + rank;
      for (int q = 0; q < w; ++q) pos += sm.wcnt[q][e];
      sorted_pairs[pos] = p;
      pair_slot[p] = pos;
      if (slot_gate) {
        slot_gate[pos] = gsrc[p];
        slot_tok[pos] = p / k;
      }
    }
    lds_barrier();
    if (c0 + NTH < p1) {  // advance the per-expert bases for the next chunk
      for (int x = tid; x < E; x += NTH) {
        int add = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          add += sm.wcnt[q][x];
          sm.wcnt[q][x] = 0;
        }
        sm.base[x] += add;
      }
      lds_barrier();
    }
  }
}

constexpr int kPermThreads = 1024;
constexpr int kPermLdsPairs = 16384;  // expert ids staged in LDS up to this many pairs

__global__ void __launch_bounds__(kPermThreads)
permute_kernel(const int32_t* __restrict__ idx, const float* __restrict__ gates, int P, int E,
               int k, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot,
               int32_t* dinfo, int32_t* meta, float* slot_gate, int32_t* slot_tok) {
  __shared__ PermSmem<kPermThreads> sm;
  __shared__ int32_t s_idx[kPermLdsPairs];
  const int32_t* src = idx;
  if (P <= kPermLdsPairs) {
    for (int p = threadIdx.x; p < P; p += kPermThreads) s_idx[p] = idx[p];
    lds_barrier();
    src = s_idx;
  }
  block_permute<kPermThreads>(src, P, E, k, counts, offsets, sorted_pairs, pair_slot, dinfo, meta,
                              gates, slot_gate, slot_tok, sm);
}

// Large batches inside the forward path (which has workspace for the per-block
// counts): the permutation over many workgroups.  Block b owns the pairs
// [b R, (b+1) R) in pair order.
//   perm_hist_kernel     per-block expert histograms -> bcnt[b][e]
//   perm_scan_kernel     counts, offsets, the distinct-expert records, and
//                        bcnt[b][e] <- offsets[e] + pairs of e in blocks < b
//   perm_scatter_kernel  each block scatters its pairs stably from bcnt[b][.]
// The result is the same stable order as the single-block kernel's.
constexpr int kPermBlockThreads = 256;

__global__ void __launch_bounds__(kPermBlockThreads)
perm_hist_kernel(const int32_t* __restrict__ idx, int P, int E, int R, int32_t* __restrict__ bcnt) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x, p0 = blockIdx.x * R, p1 = min(P, p0 + R);
  for (int e = tid; e < E; e += kPermBlockThreads) cnt[e] = 0;
  lds_barrier();
  for (int p = p0 + tid; p < p1; p += kPermBlockThreads) atomicAdd(&cnt[idx[p]], 1);
  lds_barrier();
  for (int e = tid; e < E; e += kPermBlockThreads) bcnt[(size_t)blockIdx.x * E + e] = cnt[e];
}

constexpr int kPermScanThreads = kMaxExperts;

__global__ void __launch_bounds__(kPermScanThreads)
perm_scan_kernel(int32_t* __restrict__ bcnt, int NB, int P, int E, int32_t* counts,
                 int32_t* offsets, int32_t* dinfo, int32_t* meta) {
  __shared__ PermSmem<kPermScanThreads> sm;
  const int e = threadIdx.x;
  // Up to kScanRegs blocks the column of expert e is read once, all loads in
  // flight together, and kept in registers until its base is known; past that,
  // in rounds of eight loads, the prefix stored and the base added after.
  constexpr int kScanRegs = 64;
  const bool in_regs = NB <= kScanRegs;
  int col[kScanRegs];
  int run = 0;
  if (e < E) {
    if (in_regs) {
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b) {  // unconditional loads: all in flight at once
        const int v = bcnt[(size_t)min(b, NB - 1) * E + e];
        col[b] = b < NB ? v : 0;
      }
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b) {
        const int c = col[b];
        col[b] = run;
        run += c;
      }
    } else {
      int b = 0;
      for (; b + 8 <= NB; b += 8) {  // eight independent loads in flight
        int c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = bcnt[(size_t)(b + j) * E + e];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bcnt[(size_t)(b + j) * E + e] = run;
          run += c[j];
        }
      }
      for (; b < NB; ++b) {
        const int c = bcnt[(size_t)b * E + e];
        bcnt[(size_t)b * E + e] = run;
        run += c;
      }
    }
  }
  int c[1] = {run}, f[1] = {run > 0 ? 1 : 0};
  int total = 0, nd = 0;
  block_excl_scan_e<kPermScanThreads>(c, sm.wsum, &total);
  block_excl_scan_e<kPermScanThreads>(f, sm.wsum, &nd);
  if (e < E) {
    counts[e] = run;
    offsets[e] = c[0];
    if (run > 0) {
      dinfo[4 * f[0] + 0] = e;
      dinfo[4 * f[0] + 1] = c[0];
      dinfo[4 * f[0] + 2] = run;
      dinfo[4 * f[0] + 3] = 0;
    }
    if (in_regs) {
#pragma unroll
      for (int b = 0; b < kScanRegs; ++b)
        if (b < NB) bcnt[(size_t)b * E + e] = col[b] + c[0];
    } else {
      for (int b = 0; b < NB; ++b) bcnt[(size_t)b * E + e] += c[0];
    }
  }
  if (e == 0) {
    offsets[E] = total;
    meta[0] = nd;
  }
  for (int x = nd + e; x < (P < E ? P : E); x += kPermScanThreads) dinfo[4 * x] = -1;
}

__global__ void __launch_bounds__(kPermBlockThreads)
perm_scatter_kernel(const int32_t* __restrict__ idx, const float* __restrict__ gates, int P, int E,
                    int k, int R, const int32_t* __restrict__ bcnt, int32_t* sorted_pairs,
                    int32_t* pair_slot, float* slot_gate, int32_t* slot_tok) {
  __shared__ PermSmem<kPermBlockThreads> sm;
  const int tid = threadIdx.x, p0 = blockIdx.x * R, p1 = min(P, p0 + R);
  for (int e = tid; e < E; e += kPermBlockThreads) {
    sm.base[e] = bcnt[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < kPermBlockThreads / kWave; ++q) sm.wcnt[q][e] = 0;
  }
  lds_barrier();
  scatter_range<kPermBlockThreads>(idx, p0, p1, E, k, sorted_pairs, pair_slot, gates, slot_gate,
                                   slot_tok, sm);
}

// Few tokens (T <= kFewRouteTokens <= 64, at most kFewRoutePairs pairs): the 16
// waves rank the tokens (wave w: tokens w, w + 16, ...) and set bit t of expert
// e's token mask for each choice; a token's k experts are distinct, so expert
// e's pairs in pair order are its tokens in token order.  Thread x then counts
// expert x's pairs (popcount of its mask) and one block scan gives, packed in
// one int, its first sorted slot and its distinct-expert record index; pair
// (t, j) lands in slot first(e) + popcount(mask(e) below bit t).  That is the
// stable (expert, pair id) order of the many-token permutation.
constexpr int kFewRouteThreads = 1024;
static_assert(kFewRouteThreads == kMaxExperts, "one expert a thread");
static_assert(kFewRouteTokens <= 64, "a 64-bit token mask per expert");
static_assert(kFewRoutePairs <= kMaxExperts, "slots and records packed in 16 bits each");

template <int VPL>
__global__ void __launch_bounds__(kFewRouteThreads)
route_few_kernel(const float* __restrict__ logits, int T, int E, int k, int32_t* idx, float* gates,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot,
                 int32_t* dinfo, int32_t* meta, float* slot_gate, int32_t* slot_tok) {
  __shared__ unsigned long long tmask[kMaxExperts];  // bit t: token t chose expert x
  __shared__ int first[kMaxExperts];                 // first sorted slot of expert x
  __shared__ int wsum[2 * kWave + 1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int P = T * k;
  // every logit row of the wave's tokens is loaded before the first is ranked
  constexpr int NW = kFewRouteThreads / kWave, kTPW = (kFewRouteTokens + NW - 1) / NW;
  float lv[kTPW][VPL];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int t = w + NW * j;
    wave_load_logits<VPL>(logits + (size_t)(t < T ? t : 0) * E, E, lane, lv[j]);
  }
  tmask[tid] = 0ull;
  lds_barrier();
  int pe[kTPW];  // lane j < k: the expert and gate of rank j of the wave's token j
  float pg[kTPW];
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int t = w + NW * j;
    pe[j] = 0;
    pg[j] = 0.f;
    if (t < T) {
      wave_topk_vals<VPL>(lv[j], E, k, lane, pe[j], pg[j]);
      if (lane < k) {
        atomicOr(&tmask[pe[j]], 1ull << t);
        idx[t * k + lane] = pe[j];
        gates[t * k + lane] = pg[j];
      }
    }
  }
  lds_barrier();
  const unsigned long long m = tid < E ? tmask[tid] : 0ull;
  const int c = __popcll(m);
  int v[1] = {c | (c ? 1 << 16 : 0)};
  int tot;
  block_excl_scan_e<kFewRouteThreads>(v, wsum, &tot);
  const int f = v[0] & 0xFFFF, d = v[0] >> 16, nd = tot >> 16;
  first[tid] = f;
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = f;
    if (dinfo && c) {
      dinfo[4 * d + 0] = tid;
      dinfo[4 * d + 1] = f;
      dinfo[4 * d + 2] = c;
      dinfo[4 * d + 3] = 0;
    }
  }
  // records past the last distinct expert (up to min(P, E)) say "no expert"
  if (dinfo && tid >= nd && tid < (P < E ? P : E)) dinfo[4 * tid] = -1;
  if (tid == 0) {
    offsets[E] = P;
    if (meta) meta[0] = nd;
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < kTPW; ++j) {
    const int t = w + NW * j;
    if (t < T && lane < k) {
      const int e = pe[j], p = t * k + lane;
      const int sl = first[e] + __popcll(tmask[e] & ((1ull << t) - 1ull));
      pair_slot[p] = sl;
      sorted_pairs[sl] = p;
      if (slot_tok) slot_tok[sl] = t;
      if (slot_gate) slot_gate[sl] = pg[j];
    }
  }
}

int vpl_for(int E) {
  const int v = (E + kWave - 1) / kWave;
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 6 ? 6 : v <= 8 ? 8 : 16;
}

}  // namespace

int perm_pairs_per_block(int P) {
  const int chunks = (P + kPermBlockThreads - 1) / kPermBlockThreads;
  const int per = (chunks + kPermBlocksMax - 1) / kPermBlocksMax;  // chunks per block
  return per * kPermBlockThreads;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int P = a.T * a.k;
  const int vpl = vpl_for(a.E);
  if (a.T <= kFewRouteTokens && P <= kFewRoutePairs) {
#define MOE_ROUTE_FEW(V)                                                                         \
  launch_k(route_few_kernel<V>, dim3(1), dim3(kFewRouteThreads), 0, stream, ev_start(a.ev, 0),   \
           ev_stop(a.ev, 0), a.logits, a.T, a.E, a.k, a.idx, a.gates, a.counts, a.offsets,       \
           a.sorted_pairs, a.pair_slot, a.dinfo, a.meta, a.slot_gate, a.slot_tok)
    switch (vpl) {
      case 1: MOE_ROUTE_FEW(1); break;
      case 2: MOE_ROUTE_FEW(2); break;
      case 4: MOE_ROUTE_FEW(4); break;
      case 6: MOE_ROUTE_FEW(6); break;
      case 8: MOE_ROUTE_FEW(8); break;
      default: MOE_ROUTE_FEW(16); break;
    }
#undef MOE_ROUTE_FEW
  } else {
    // more than 64 tokens or 1024 pairs: one wave per token, then the
    // permutation (several workgroups with the forward path's scratch, else one)
    const int wpb = 4;
    const dim3 grid((a.T + wpb - 1) / wpb), block(wpb * kWave);
#define MOE_TOPK(V) \
  launch_k(topk_kernel<V>, grid, block, 0, stream, ev_start(a.ev, 0), (hipEvent_t) nullptr, \
           a.logits, a.T, a.E, a.k, a.idx, a.gates)
    switch (vpl) {
      case 1: MOE_TOPK(1); break;
      case 2: MOE_TOPK(2); break;
      case 4: MOE_TOPK(4); break;
      case 6: MOE_TOPK(6); break;
      case 8: MOE_TOPK(8); break;
      default: MOE_TOPK(16); break;
    }
#undef MOE_TOPK
    if (a.perm_scratch && a.dinfo && a.slot_gate) {
      const int R = perm_pairs_per_block(P), NB = (P + R - 1) / R;
      launch_k(perm_hist_kernel, dim3(NB), dim3(kPermBlockThreads), 0, stream,
               (hipEvent_t) nullptr, (hipEvent_t) nullptr, (const int32_t*)a.idx, P, a.E, R,
               a.perm_scratch);
      launch_k(perm_scan_kernel, dim3(1), dim3(kPermScanThreads), 0, stream, (hipEvent_t) nullptr,
               (hipEvent_t) nullptr, a.perm_scratch, NB, P, a.E, a.counts, a.offsets, a.dinfo,
               a.meta);
      launch_k(perm_scatter_kernel, dim3(NB), dim3(kPermBlockThreads), 0, stream,
               (hipEvent_t) nullptr, ev_stop(a.ev, 0), (const int32_t*)a.idx,
               (const float*)a.gates, P, a.E, a.k, R, (const int32_t*)a.perm_scratch,
               a.sorted_pairs, a.pair_slot, a.slot_gate, a.slot_tok);
    } else {
      launch_k(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, (hipEvent_t) nullptr,
               ev_stop(a.ev, 0), (const int32_t*)a.idx, (const float*)a.gates, P, a.E, a.k,
               a.counts, a.offsets, a.sorted_pairs, a.pair_slot, a.dinfo, a.meta, a.slot_gate,
               a.slot_tok);
    }
  }
  return hipGetLastError();
}

}  // namespace moe_fp4
