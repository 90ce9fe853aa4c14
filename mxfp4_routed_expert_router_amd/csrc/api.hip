// C-ABI of the moe_fp4 library: argument validation, workspace layout and
// dispatch to the route / decode / prefill kernels.  Every check runs on the
// host before the first HIP call, so a rejected call enqueues nothing.
#include "../../include/moe_fp4.h"

#include <mutex>
#include <new>

#include "kernels.h"

using namespace moe_fp4;

namespace {

constexpr size_t kAlign = 256;
constexpr float kStackEps = 1e-6f;  // the residual stack's pre-norm epsilon

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool dims_ok(const moe_fp4_dims& d) {
  return d.T >= 1 && d.T <= 65535 && d.E >= 1 && d.E <= kMaxExperts && d.k >= 1 && d.k <= d.E &&
         d.k <= kMaxK && d.H >= 32 && d.H <= 16384 && d.H % 32 == 0 && d.I >= 32 &&
         d.I <= 16384 && d.I % 32 == 0;
}

// AUTO takes the GEMV path up to this many tokens: at H = 5120, I = 2304,
// top-6 of 384 the few-token GEMV kernels and the small-batch grouped GEMMs
// take 148 and 150 us per call at T = 8, but 210 against 189 us at T = 12 and
// 256 against 215 us at T = 15 (graph replay, one MI355X).
constexpr int kAutoDecodeMaxT = 8;

// Mode that a call actually runs, or -1 if the dims do not allow it.
int resolve_mode(const moe_fp4_dims& d, int mode) {
  const bool decode_ok = decode_fits(d.T, d.H, d.I, d.k);
  switch (mode) {
    case MOE_FP4_MODE_AUTO:
      return decode_ok && d.T <= kAutoDecodeMaxT ? MOE_FP4_MODE_DECODE : MOE_FP4_MODE_PREFILL;
    case MOE_FP4_MODE_DECODE: return decode_ok ? MOE_FP4_MODE_DECODE : -1;
    case MOE_FP4_MODE_PREFILL: return MOE_FP4_MODE_PREFILL;
    case MOE_FP4_MODE_PREFILL_MXFP8:  // one scaled MFMA covers 128 inputs
      return d.H % 128 == 0 && d.I % 128 == 0 ? MOE_FP4_MODE_PREFILL_MXFP8 : -1;
    default: return -1;
  }
}

int sal_tiles(int H) { return (H + kSalRows - 1) / kSalRows; }

// Workspace sections, each 256-byte aligned.
struct WsLayout {
  size_t logits, idx, gates, counts, offsets, sorted, slot, slot_gate, slot_tok, dinfo, meta, perm,
      h, ypair, sal, xq, xqs, hq, hqs, u, total;
};

WsLayout layout(const moe_fp4_dims& d, int rmode) {
  const size_t P = (size_t)d.T * d.k;
  WsLayout L{};
  size_t o = 0;
  L.logits = o;   o = align_up(o + (size_t)d.T * d.E * 4);  // moe_fp4_forward_routed
  L.idx = o;      o = align_up(o + P * 4);
  L.gates = o;    o = align_up(o + P * 4);
  L.counts = o;   o = align_up(o + (size_t)d.E * 4);
  L.offsets = o;  o = align_up(o + (size_t)(d.E + 1) * 4);
  L.sorted = o;   o = align_up(o + P * 4);
  L.slot = o;     o = align_up(o + P * 4);
  L.slot_gate = o; o = align_up(o + P * 4);
  L.slot_tok = o; o = align_up(o + P * 4);
  L.dinfo = o;    o = align_up(o + (size_t)d.E * 16);
  L.meta = o;     o = align_up(o + 64);
  L.perm = o;     // per-block expert counts of the multi-block permutation
  if (P > (size_t)kFewRoutePairs) o = align_up(o + (size_t)kPermBlocksMax * d.E * 4);
  L.h = o;        o = align_up(o + P * (size_t)d.I * 2);
  L.ypair = o;
  L.u = o;  // pre-normed input of moe_fp4_forward_residual: ypair's space in the prefill modes
  if (rmode == MOE_FP4_MODE_DECODE) o = align_up(o + (size_t)d.T * d.H * 2);
  const bool mx = rmode == MOE_FP4_MODE_PREFILL_MXFP8;
  if (rmode == MOE_FP4_MODE_PREFILL || mx) {
    o = align_up(o + P * (size_t)d.H * 4);
    L.sal = o;  // saliency tile partials (moe_fp4_forward_saliency)
    o = align_up(o + P * (size_t)sal_tiles(d.H) * 4);
  }
  if (mx) {
    const size_t Hp = mx8_padded(d.H), Ip = mx8_padded(d.I);
    L.xq = o;  o = align_up(o + (size_t)d.T * Hp);
    L.xqs = o; o = align_up(o + (size_t)d.T * Hp / 32);
    L.hq = o;  o = align_up(o + P * Ip);
    L.hqs = o; o = align_up(o + P * Ip / 32);
  }
  L.total = o;
  return L;
}

// Workspace of moe_fp4_route: the records the many-workgroup permutation
// writes besides the caller's outputs; none up to kFewRoutePairs pairs.
struct RouteWs {
  size_t dinfo, meta, slot_gate, slot_tok, perm, total;
};
RouteWs route_layout(const moe_fp4_dims& d) {
  RouteWs L{};
  const size_t P = (size_t)d.T * d.k;
  if (d.T <= kFewRouteTokens && P <= (size_t)kFewRoutePairs) return L;
  size_t o = 0;
  L.dinfo = o;     o = align_up(o + (size_t)d.E * 16);
  L.meta = o;      o = align_up(o + 64);
  L.slot_gate = o; o = align_up(o + P * 4);
  L.slot_tok = o;  o = align_up(o + P * 4);
  L.perm = o;      o = align_up(o + (size_t)kPermBlocksMax * d.E * 4);
  L.total = o;
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Exactly one of logits and w_router is given; with w_router the logits are
// computed into the workspace first.
// With saliency (prefill modes only) the per-expert saliency is added to it.
// With x_resid (x null, y = x_resid) the layer's input is the pre-norm of
// x_resid and its output is added to it.
int forward_impl(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                 const uint16_t* w_router, const moe_fp4_weights* w, float* y, int mode, int flags,
                 void* ws, size_t ws_bytes, hipStream_t stream, uint16_t* h_out,
                 moe_fp4_route_out* route_out, const hipEvent_t* events,
                 float* saliency = nullptr, float* x_resid = nullptr,
                 const SharedArgs* shared13 = nullptr, const SharedArgs* shared2 = nullptr,
                 bool validate_only = false) {
  if (x_resid) {
    if (x) return MOE_FP4_EINVAL;
    y = x_resid;
    flags |= MOE_FP4_ACCUMULATE;
  }
  if (!dims || !(x || x_resid) || !(logits || w_router) || !w || !y || !ws) return MOE_FP4_EINVAL;
  if (!w->w1 || !w->s1 || !w->w3 || !w->s3 || !w->w2 || !w->s2) return MOE_FP4_EINVAL;
  if (route_out && (!route_out->topk_idx || !route_out->gates || !route_out->counts ||
                    !route_out->offsets || !route_out->sorted_pairs || !route_out->pair_slot))
    return MOE_FP4_EINVAL;
  for (int i = 0; i < 6; ++i)
    if (w->expert_stride[i] < 0) return MOE_FP4_EINVAL;
  const moe_fp4_dims d = *dims;
  if (d.T < 1 || d.H < 1 || d.I < 1 || d.E < 1 || d.k < 1 || d.k > d.E) return MOE_FP4_EINVAL;
  if (!dims_ok(d)) return MOE_FP4_EUNSUPPORTED;
  if (flags & ~MOE_FP4_ACCUMULATE) return MOE_FP4_EUNSUPPORTED;
  const int rmode = resolve_mode(d, saliency && mode == MOE_FP4_MODE_AUTO ? MOE_FP4_MODE_PREFILL
                                                                            : mode);
  if (rmode < 0 || (saliency && rmode == MOE_FP4_MODE_DECODE)) return MOE_FP4_EUNSUPPORTED;
  if (saliency && !aligned(saliency, 4)) return MOE_FP4_EALIGN;

  // per-expert tensor sizes in bytes, in the order w1, s1, w3, s3, w2, s2
  const int64_t per[6] = {(int64_t)d.I * d.H / 2, (int64_t)d.I * d.H / 32,
                          (int64_t)d.I * d.H / 2, (int64_t)d.I * d.H / 32,
                          (int64_t)d.H * d.I / 2, (int64_t)d.H * d.I / 32};
  int64_t stride[6];
  for (int i = 0; i < 6; ++i) stride[i] = w->expert_stride[i] ? w->expert_stride[i] : per[i];
  if (!aligned(x_resid ? (const void*)x_resid : (const void*)x, 16) || !aligned(y, 16) ||
      !aligned(ws, kAlign) || !aligned(w->w1, 16) ||
      !aligned(w->w3, 16) || !aligned(w->w2, 16) || stride[0] % 16 || stride[2] % 16 ||
      stride[4] % 16 || (h_out && !aligned(h_out, 4)) || (w_router && !aligned(w_router, 16)))
    return MOE_FP4_EALIGN;
  // the MXFP8 GEMMs read the scales a dword at a time
  if (rmode == MOE_FP4_MODE_PREFILL_MXFP8 &&
      (!aligned(w->s1, 4) || !aligned(w->s3, 4) || !aligned(w->s2, 4) || stride[1] % 4 ||
       stride[3] % 4 || stride[5] % 4))
    return MOE_FP4_EALIGN;
  const WsLayout L = layout(d, rmode);
  if (ws_bytes < L.total || validate_only) return MOE_FP4_EWORKSPACE;

  // the pre-norm: inside the w1/w3 kernel on the one-token path, else a
  // kernel of its own into the workspace
  const bool prenorm_fused =
      x_resid && rmode == MOE_FP4_MODE_DECODE && decode_one_token(d.T, d.H, d.I, d.k);
  if (x_resid && !prenorm_fused) {
    uint16_t* const u = at<uint16_t>(ws, L.u);
    if (launch_prenorm(x_resid, u, d.T, d.H, kStackEps, stream) != hipSuccess) return MOE_FP4_EHIP;
    x = u;
  }
  if (w_router) {
    float* const lg = at<float>(ws, L.logits);
    if (launch_router_logits(x, w_router, lg, d.T, d.H, d.E, stream) != hipSuccess)
      return MOE_FP4_EHIP;
    logits = lg;
  }
  RouteArgs r{};
  r.logits = logits;
  r.T = d.T; r.E = d.E; r.k = d.k;
  r.idx = at<int32_t>(ws, L.idx);
  r.gates = at<float>(ws, L.gates);
  r.counts = at<int32_t>(ws, L.counts);
  r.offsets = at<int32_t>(ws, L.offsets);
  r.sorted_pairs = at<int32_t>(ws, L.sorted);
  r.pair_slot = at<int32_t>(ws, L.slot);
  r.dinfo = at<int32_t>(ws, L.dinfo);
  r.meta = at<int32_t>(ws, L.meta);
  r.slot_gate = at<float>(ws, L.slot_gate);
  r.slot_tok = at<int32_t>(ws, L.slot_tok);
  if ((size_t)d.T * d.k > (size_t)kFewRoutePairs) r.perm_scratch = at<int32_t>(ws, L.perm);
  // A one-token decode ranks the logits inside its first expert kernel.
  const bool fused = rmode == MOE_FP4_MODE_DECODE && decode_fuses_route(d.T, d.H, d.I, d.E, d.k);
  r.ev = events;
  if (fused)
    ev_empty(events, 0, stream);  // routing runs inside the w1/w3 kernel
  else if (launch_route(r, stream) != hipSuccess)
    return MOE_FP4_EHIP;

  LayerArgs a{};
  a.T = d.T; a.H = d.H; a.I = d.I; a.E = d.E; a.k = d.k;
  a.x = x;
  a.w1 = w->w1; a.s1 = w->s1; a.w3 = w->w3; a.s3 = w->s3; a.w2 = w->w2; a.s2 = w->s2;
  for (int i = 0; i < 6; ++i) a.stride[i] = stride[i];
  a.counts = r.counts; a.offsets = r.offsets; a.sorted_pairs = r.sorted_pairs;
  a.pair_slot = r.pair_slot; a.dinfo = r.dinfo; a.meta = r.meta; a.gates = r.gates;
  a.slot_gate = r.slot_gate; a.slot_tok = r.slot_tok;
  a.h = at<uint16_t>(ws, L.h);
  const bool mx = rmode == MOE_FP4_MODE_PREFILL_MXFP8;
  a.ypair = rmode == MOE_FP4_MODE_PREFILL || mx ? at<float>(ws, L.ypair) : nullptr;
  if (mx) {
    a.xq = at<uint8_t>(ws, L.xq);
    a.xqs = at<uint8_t>(ws, L.xqs);
    a.hq = at<uint8_t>(ws, L.hq);
    a.hqs = at<uint8_t>(ws, L.hqs);
  }
  a.y = y;
  a.accumulate = (flags & MOE_FP4_ACCUMULATE) ? 1 : 0;
  a.ev = events;
  a.fused_route = fused ? 1 : 0;
  a.route = r;
  a.logits = logits;
  if (prenorm_fused) {
    a.xf = x_resid;
    a.eps = kStackEps;
  }
  a.shared13 = shared13;
  a.shared2 = shared2;
  if (saliency) {
    a.sal_part = at<float>(ws, L.sal);
    a.sal_tiles = sal_tiles(d.H);
  }
  const hipError_t err = rmode == MOE_FP4_MODE_DECODE ? launch_decode(a, stream)
                         : mx                          ? launch_prefill_mx8(a, stream)
                                                       : launch_prefill(a, stream);
  if (err != hipSuccess) return MOE_FP4_EHIP;
  if (saliency && launch_saliency(a, saliency, stream) != hipSuccess) return MOE_FP4_EHIP;

  if (h_out && launch_unsort_h(a, h_out, stream) != hipSuccess) return MOE_FP4_EHIP;
  if (route_out) {
    const size_t P = (size_t)d.T * d.k;
    const struct { void* dst; const void* src; size_t n; } cp[6] = {
        {route_out->topk_idx, r.idx, P * 4},       {route_out->gates, r.gates, P * 4},
        {route_out->counts, r.counts, (size_t)d.E * 4},
        {route_out->offsets, r.offsets, (size_t)(d.E + 1) * 4},
        {route_out->sorted_pairs, r.sorted_pairs, P * 4},
        {route_out->pair_slot, r.pair_slot, P * 4}};
    for (const auto& c : cp)
      if (hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return MOE_FP4_EHIP;
  }
  return MOE_FP4_OK;
}

// Checks of the shared expert's arguments (T and H from dims).
int shared_check(const moe_fp4_dims& d, const uint16_t* x, const moe_fp4_shared_weights* sw,
                 const float* y) {
  if (!x || !sw || !y || !sw->w1 || !sw->s1 || !sw->w3 || !sw->s3 || !sw->w2 || !sw->s2)
    return MOE_FP4_EINVAL;
  if (d.T < 1 || d.H < 1 || sw->I < 1) return MOE_FP4_EINVAL;
  if (d.T > 65535 || d.H < 32 || d.H > 16384 || d.H % 32 || sw->I < 32 || sw->I > 16384 ||
      sw->I % 32)
    return MOE_FP4_EUNSUPPORTED;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(sw->w1, 16) || !aligned(sw->w3, 16) ||
      !aligned(sw->w2, 16))
    return MOE_FP4_EALIGN;
  return MOE_FP4_OK;
}
const uint8_t* const* shared_tensors(const moe_fp4_shared_weights* sw, const uint8_t* (&t)[6]) {
  t[0] = sw->w1; t[1] = sw->s1; t[2] = sw->w3; t[3] = sw->s3; t[4] = sw->w2; t[5] = sw->s2;
  return t;
}

// The workspace of moe_fp4_forward_noalloc: one array per GPU, held until the
// process ends.  Host code never uses its name as an address (on the host it
// is a stand-in symbol): the device address comes from hipGetSymbolAddress,
// taken once per device and kept in scratch_ptr.
constexpr size_t kScratchBytes = MOE_FP4_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's scratch address, or null (and *err set) on failure.
void* device_scratch(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_fp4_forward_noalloc(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                            const moe_fp4_weights* w, float* y, int mode, int flags,
                            hipStream_t stream) {
  // Every check of moe_fp4_forward, with a stand-in workspace address that
  // passes its alignment rule and is never used: forward_impl returns
  // EWORKSPACE at its workspace check when everything before it passed.
  // Then the size rule.  All of it before the first HIP call.
  const int rc = forward_impl(dims, x, logits, nullptr, w, y, mode, flags,
                              reinterpret_cast<void*>(kAlign), 0, stream, nullptr, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, /*validate_only=*/true);
  if (rc != MOE_FP4_EWORKSPACE) return rc;
  if (layout(*dims, resolve_mode(*dims, mode)).total > kScratchBytes) return MOE_FP4_EWORKSPACE;
  hipError_t err = hipSuccess;
  void* ws = device_scratch(&err);
  if (!ws) return MOE_FP4_EHIP;
  return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, kScratchBytes, stream,
                      nullptr, nullptr, nullptr);
}

int moe_fp4_workspace_size(const moe_fp4_dims* dims, int mode, size_t* bytes) {
  if (!dims || !bytes) return MOE_FP4_EINVAL;
  if (!dims_ok(*dims)) return MOE_FP4_EUNSUPPORTED;
  const int rmode = resolve_mode(*dims, mode);
  if (rmode < 0) return MOE_FP4_EUNSUPPORTED;
  *bytes = layout(*dims, rmode).total;
  return MOE_FP4_OK;
}

int moe_fp4_plan(const moe_fp4_dims* dims, int mode, int* path) {
  if (!dims || !path) return MOE_FP4_EINVAL;
  const moe_fp4_dims d = *dims;
  if (!dims_ok(d)) return MOE_FP4_EUNSUPPORTED;
  const int rmode = resolve_mode(d, mode);
  if (rmode < 0) return MOE_FP4_EUNSUPPORTED;
  if (rmode == MOE_FP4_MODE_DECODE) {
    const int fam = decode_family(d.T, d.H, d.I, d.k);
    *path = fam == 1 ? MOE_FP4_PATH_DECODE_ONE : fam == 2 ? MOE_FP4_PATH_DECODE_FEW
                                                          : MOE_FP4_PATH_DECODE_MFMA;
  } else {
    *path = rmode == MOE_FP4_MODE_PREFILL_MXFP8 ? MOE_FP4_PATH_PREFILL_MXFP8 : MOE_FP4_PATH_PREFILL;
  }
  return MOE_FP4_OK;
}

namespace {
int route_dims(const moe_fp4_dims* dims) {
  if (!dims) return MOE_FP4_EINVAL;
  const moe_fp4_dims d = *dims;
  if (d.T < 1 || d.E < 1 || d.k < 1 || d.k > d.E) return MOE_FP4_EINVAL;
  if (d.T > 65535 || d.E > kMaxExperts || d.k > kMaxK) return MOE_FP4_EUNSUPPORTED;
  return MOE_FP4_OK;
}
}  // namespace

int moe_fp4_route_workspace_size(const moe_fp4_dims* dims, size_t* bytes) {
  if (!bytes) return MOE_FP4_EINVAL;
  const int rc = route_dims(dims);
  if (rc != MOE_FP4_OK) return rc;
  *bytes = route_layout(*dims).total;
  return MOE_FP4_OK;
}

int moe_fp4_route(const moe_fp4_dims* dims, const float* logits, moe_fp4_route_out* out,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dims || !logits || !out || !out->topk_idx || !out->gates || !out->counts ||
      !out->offsets || !out->sorted_pairs || !out->pair_slot)
    return MOE_FP4_EINVAL;
  const int rc = route_dims(dims);
  if (rc != MOE_FP4_OK) return rc;
  const moe_fp4_dims d = *dims;
  if (!aligned(logits, 4) || (ws && !aligned(ws, kAlign))) return MOE_FP4_EALIGN;
  const RouteWs L = route_layout(d);
  if (L.total > 0 && (!ws || ws_bytes < L.total)) return MOE_FP4_EWORKSPACE;
  RouteArgs r{};
  r.logits = logits;
  r.T = d.T; r.E = d.E; r.k = d.k;
  r.idx = out->topk_idx; r.gates = out->gates; r.counts = out->counts; r.offsets = out->offsets;
  r.sorted_pairs = out->sorted_pairs; r.pair_slot = out->pair_slot;
  if (L.total > 0) {
    // large batches: the permutation spread over many workgroups, with its
    // per-workgroup counts and per-slot records in the workspace
    r.dinfo = at<int32_t>(ws, L.dinfo);
    r.meta = at<int32_t>(ws, L.meta);
    r.slot_gate = at<float>(ws, L.slot_gate);
    r.slot_tok = at<int32_t>(ws, L.slot_tok);
    r.perm_scratch = at<int32_t>(ws, L.perm);
  }
  return launch_route(r, stream) == hipSuccess ? MOE_FP4_OK : MOE_FP4_EHIP;
}

int moe_fp4_forward(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                    const moe_fp4_weights* w, float* y, int mode, int flags, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                      nullptr, nullptr);
}

int moe_fp4_forward_routed(const moe_fp4_dims* dims, const uint16_t* x, const uint16_t* w_router,
                           const moe_fp4_weights* w, float* y, int mode, int flags, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!w_router) return MOE_FP4_EINVAL;
  return forward_impl(dims, x, nullptr, w_router, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                      nullptr, nullptr);
}

int moe_fp4_forward_residual(const moe_fp4_dims* dims, float* x, const float* logits,
                             const moe_fp4_weights* w, int mode, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  if (!x) return MOE_FP4_EINVAL;
  return forward_impl(dims, nullptr, logits, nullptr, w, nullptr, mode, 0, ws, ws_bytes, stream,
                      nullptr, nullptr, nullptr, nullptr, x);
}

int moe_fp4_forward_saliency(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                             const moe_fp4_weights* w, float* y, float* saliency, int mode,
                             int flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!saliency) return MOE_FP4_EINVAL;
  return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                      nullptr, nullptr, saliency);
}

int moe_fp4_shared_expert(const moe_fp4_dims* dims, const uint16_t* x,
                          const moe_fp4_shared_weights* sw, float* y, int flags, uint16_t* h,
                          hipStream_t stream) {
  if (!dims || !h) return MOE_FP4_EINVAL;
  const int rc = shared_check(*dims, x, sw, y);
  if (rc != MOE_FP4_OK) return rc;
  if (flags & ~MOE_FP4_ACCUMULATE) return MOE_FP4_EUNSUPPORTED;
  if (!aligned(h, 16)) return MOE_FP4_EALIGN;
  const uint8_t* t[6];
  return launch_shared(x, shared_tensors(sw, t), dims->T, dims->H, sw->I, y,
                       (flags & MOE_FP4_ACCUMULATE) ? 1 : 0, h, stream) == hipSuccess
             ? MOE_FP4_OK
             : MOE_FP4_EHIP;
}

int moe_fp4_forward_shared(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                           const moe_fp4_weights* w, const moe_fp4_shared_weights* sw, float* y,
                           int mode, int flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dims) return MOE_FP4_EINVAL;
  int rc = shared_check(*dims, x, sw, y);
  if (rc != MOE_FP4_OK) return rc;
  // the shared expert's h reuses the routed h section once the routed path is done
  if (sw->I > dims->k * dims->I) return MOE_FP4_EUNSUPPORTED;
  const int rmode = resolve_mode(*dims, mode);
  const moe_fp4_dims& d = *dims;
  if (rmode == MOE_FP4_MODE_DECODE && d.T == 1 && decode_one_token(d.T, d.H, d.I, d.k) &&
      sw->I <= d.H && ws && ws_bytes >= layout(d, rmode).total) {
    // One token: the shared w1/w3 rows run in the routed w1/w3 launch, their
    // h in the pre-norm input's section (unused without a residual), and the
    // shared w2 rows in the routed w2 launch, added to the routed y.  The
    // shared expert's own row arithmetic and the order of the two calls: the
    // same bits.
    SharedArgs s13{};
    s13.act = x;
    s13.w[0] = sw->w1; s13.s[0] = sw->s1; s13.w[1] = sw->w3; s13.s[1] = sw->s3;
    s13.N = sw->I; s13.K = d.H; s13.T = 1;
    s13.h = at<uint16_t>(ws, layout(d, rmode).u);
    SharedArgs s2{};
    s2.act = s13.h;
    s2.w[0] = sw->w2; s2.s[0] = sw->s2;
    s2.N = d.H; s2.K = sw->I; s2.T = 1; s2.accumulate = 1;
    return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                        nullptr, nullptr, nullptr, nullptr, &s13, &s2);
  }
  rc = forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                    nullptr, nullptr);
  if (rc != MOE_FP4_OK) return rc;
  uint16_t* const h = at<uint16_t>(ws, layout(*dims, rmode).h);
  const uint8_t* t[6];
  return launch_shared(x, shared_tensors(sw, t), dims->T, dims->H, sw->I, y, 1, h, stream) ==
                 hipSuccess
             ? MOE_FP4_OK
             : MOE_FP4_EHIP;
}

int moe_fp4_router_logits(const moe_fp4_dims* dims, const uint16_t* x, const uint16_t* w_router,
                          float* logits, hipStream_t stream) {
  if (!dims || !x || !w_router || !logits) return MOE_FP4_EINVAL;
  const moe_fp4_dims d = *dims;
  if (d.T < 1 || d.H < 1 || d.E < 1) return MOE_FP4_EINVAL;
  if (d.T > 65535 || d.E > kMaxExperts || d.H < 32 || d.H > 16384 || d.H % 32)
    return MOE_FP4_EUNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(logits, 4)) return MOE_FP4_EALIGN;
  return launch_router_logits(x, w_router, logits, d.T, d.H, d.E, stream) == hipSuccess
             ? MOE_FP4_OK
             : MOE_FP4_EHIP;
}

int moe_fp4_forward_profiled(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                             const moe_fp4_weights* w, float* y, int mode, int flags, void* ws,
                             size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                             int n_events) {
  if (!events || n_events < 2 * kStages) return MOE_FP4_EINVAL;
  for (int i = 0; i < 2 * kStages; ++i)
    if (!events[i]) return MOE_FP4_EINVAL;
  return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, nullptr,
                      nullptr, events);
}

int moe_fp4_forward_debug(const moe_fp4_dims* dims, const uint16_t* x, const float* logits,
                          const moe_fp4_weights* w, float* y, int mode, int flags, void* ws,
                          size_t ws_bytes, hipStream_t stream, uint16_t* h_out,
                          moe_fp4_route_out* route_out) {
  return forward_impl(dims, x, logits, nullptr, w, y, mode, flags, ws, ws_bytes, stream, h_out,
                      route_out, nullptr);
}

int moe_fp4_prenorm_bf16(const float* x, uint16_t* u, int32_t T, int32_t H, float eps,
                         hipStream_t stream) {
  if (!x || !u || T < 1 || H < 1) return MOE_FP4_EINVAL;
  if (H % 32 || H > 16384) return MOE_FP4_EUNSUPPORTED;
  if (!aligned(x, 16) || !aligned(u, 16)) return MOE_FP4_EALIGN;
  return launch_prenorm(x, u, T, H, eps, stream) == hipSuccess ? MOE_FP4_OK : MOE_FP4_EHIP;
}

int moe_fp4_quant_mxfp8(const uint16_t* src, int32_t rows, int32_t K, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream) {
  if (!src || !codes || !scales || rows < 1 || K < 1) return MOE_FP4_EINVAL;
  if (K % 32) return MOE_FP4_EUNSUPPORTED;
  if (!aligned(src, 16) || !aligned(codes, 8)) return MOE_FP4_EALIGN;
  return launch_quant_mx8(src, rows, K, codes, scales, stream) == hipSuccess ? MOE_FP4_OK
                                                                              : MOE_FP4_EHIP;
}

const char* moe_fp4_status_string(int status) {
  switch (status) {
    case MOE_FP4_OK: return "ok";
    case MOE_FP4_EINVAL: return "invalid argument (null pointer or inconsistent size)";
    case MOE_FP4_EUNSUPPORTED: return "unsupported sizes, mode or flags";
    case MOE_FP4_EALIGN: return "misaligned pointer or stride";
    case MOE_FP4_EWORKSPACE: return "workspace missing or too small";
    case MOE_FP4_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
