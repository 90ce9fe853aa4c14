#!/usr/bin/env python3
"""Benchmark of one routed-expert FP4 MoE layer on one MI355X.

Workload (timed steps): decode, T = 1 token per step, 384 experts resident in
HBM (7.22 GB of FP4 E2M1 codes + UE8M0 scales, 18,800,640 bytes per expert),
top-6 routing, H = 5120, I = 2304.  Each step is one whole layer call -- router,
permutation, w1/w3 GEMV with SiLU gating, w2 GEMV with the gate-weighted
combine -- on a fresh token (x ~ N(0,1) in bf16, logits ~ N(0,1) plus a
per-expert Zipf(1.1) bias).  Inputs are resident in HBM before timing starts.
The value is the cold figure: L2 and the MALL are flushed before every step.

Also measured, in the same JSON line: the same steps warm (graph replay),
per-kernel durations (roofline of the dominant decode kernel), the 2048-token
prefill chunk (TFLOP/s) in both activation modes, a streaming read of the
decode kernels' footprints (achievable bandwidth), the router, shared-expert,
verify and stack figures, and the CPU oracle timed on bounded samples of the
same units of work.

    python bench.py [--gpus 1] [--steps 256] [--warmup 16]
"""
from __future__ import annotations

import argparse
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 MoE layer: decode µs/token (HBM GB/s) & 2048-tok prefill TFLOP/s"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA (the FP4 x FP8 scaled MFMA is priced at it)
SPIN_CYCLES = 200_000_000       # head start for the host to enqueue profiled steps
# the one-token decode kernels (w1/w3 with the routing inside; w2 with the combine inside)
DECODE_KERNELS = {"w13": "gemv13_one_kernel", "w2": "gemv2_one_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(H, I):
    return 2 * (I * H // 2 + I * H // 32) + (H * I // 2 + H * I // 32)


def topk_sets(logits, k):
    return np.argsort(-logits, axis=1, kind="stable")[:, :k]


def decode_bytes(wl, idx):
    """Algorithmic HBM bytes of one decode step, per kernel."""
    H, I, T, k = wl.H, wl.I, wl.T, wl.k
    D = len(np.unique(idx))
    P = T * k
    broute = T * wl.E * 4 + P * 4 * 4
    b13 = D * 2 * (I * H // 2 + I * H // 32) + T * H * 2 + P * I * 2
    b2 = D * (H * I // 2 + H * I // 32) + P * I * 2 + T * H * 4
    if T == 1:  # the routing runs inside the w1/w3 kernel
        b13, broute = b13 + broute, 0
    return {"route": broute, "w13": b13, "w2": b2, "D": D}


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "moe_layer_decode_T1_prefill_T2048_hbm_traffic.md")


# The sources the decode kernels are compiled from (decode.hip and the headers
# it includes): the traffic record of a decode kernel holds while they do.
DECODE_SOURCES = ("decode.hip", "device_common.h", "kernels.h", "shared_gemv.h", "topk.h")


def decode_sources_hash():
    import hashlib
    csrc = os.path.join(ROOT, "mxfp4_routed_expert_router_amd", "csrc")
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel):
    """HBM bytes (read + written) per launch of the decode kernel `kernel` from
    the committed rocprofv3 PMC summary (FETCH_SIZE / WRITE_SIZE scaled by a
    device-copy calibration), or None when the decode kernels' sources differ
    from the ones the counters were taken with."""
    try:
        line = next(l for l in open(TRAFFIC_PROFILE) if l.startswith("traffic_json: "))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line[len("traffic_json: "):])
    if decode_sources_hash() != rec.get("decode_sources_sha256_16") or kernel not in rec["kernels"]:
        return None
    k = rec["kernels"][kernel]
    return float(k["read_bytes"] + k["write_bytes"])


TRACE_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                             "moe_layer_decode_T1_prefill_T2048_kernel_trace.md")


def library_sources_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "mxfp4_routed_expert_router_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traced_mean_us(kernel):
    """Mean duration of `kernel` (the row whose name starts with it) in the
    committed rocprofv3 kernel trace, or None when the library's sources differ
    from the ones the trace was taken with."""
    try:
        text = open(TRACE_PROFILE).read()
    except OSError:
        return None
    m = re.search(r"sha256 prefix `([0-9a-f]+)`", text)
    if not m or m.group(1) != library_sources_hash():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.split("|")]
        if len(cells) > 4 and cells[1].strip("`").startswith(kernel):
            return float(cells[3])
    return None


def run_extras(args, moe, synth, torch, dev, w, wl, x_d, lg_d, y_d, ws, n_gen, graph_us):
    """Decode with the router step and with the shared expert, the
    speculative-verify batches and the pruned 40-layer stack."""
    # ---------------------------------------------------------------- decode from the router step
    # The same steps with the logits computed on the GPU from x and a bf16
    # router weight [E, H] (moe_fp4_forward_routed), and the router kernel
    # alone; both as graph replays.
    wr_d = torch.from_numpy(synth.gen_router(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    lg_out = torch.empty((1, wl.E), dtype=torch.float32, device=dev)

    def step_routed(i):
        j = i % n_gen
        moe.moe_fp4_forward_routed(x_d[j:j + 1], wr_d, w, wl.k, y=y_d[j:j + 1], workspace=ws)

    def step_router(i):
        j = i % n_gen
        moe.moe_fp4_router_logits(x_d[j:j + 1], wr_d, out=lg_out)

    us_routed = graph_us(step_routed)
    us_router = graph_us(step_router)
    router_bytes = wl.E * wl.H * 2 + wl.H * 2 + wl.E * 4
    routed = {"us_per_token": us_routed, "router_us": us_router,
              "router_bytes": router_bytes, "router_GBps": router_bytes / (us_router * 1e-6) / 1e9,
              "note": "x -> router logits (bf16 router weight [384, 5120], 3.9 MB) -> the same "
                      "layer; graph replay; router_us: the router kernel alone, one call per "
                      "step in a graph"}
    log(f"decode with the router step: {us_routed:.2f} us/token; router kernel alone "
        f"{us_router:.2f} us ({routed['router_GBps']:.0f} GB/s)")

    # ---------------------------------------------------------------- decode with the shared expert
    # The routed layer plus the FP8 shared expert (moe_fp4_forward_shared),
    # and the shared expert alone; graph replays.
    sw_np = synth.gen_shared(wl)
    sw_d = moe.SharedWeights.from_dict({n: torch.from_numpy(a).to(dev) for n, a in sw_np.items()})
    h_s = torch.empty((1, wl.I), dtype=torch.bfloat16, device=dev)
    y_s = torch.empty((1, wl.H), dtype=torch.float32, device=dev)

    def step_shared(i):
        j = i % n_gen
        moe.moe_fp4_forward_shared(x_d[j:j + 1], lg_d[j:j + 1], w, sw_d, wl.k, y=y_d[j:j + 1],
                                   workspace=ws)

    def step_shared_only(i):
        j = i % n_gen
        moe.moe_fp4_shared_expert(x_d[j:j + 1], sw_d, y=y_s, h=h_s)

    def step_router_shared(i):  # the whole decode step: router, routed layer, shared expert
        j = i % n_gen
        moe.moe_fp4_router_logits(x_d[j:j + 1], wr_d, out=lg_out)
        moe.moe_fp4_forward_shared(x_d[j:j + 1], lg_out, w, sw_d, wl.k, y=y_d[j:j + 1],
                                   workspace=ws)

    us_shared = graph_us(step_shared)
    us_shared_only = graph_us(step_shared_only)
    us_router_shared = graph_us(step_router_shared)
    shared_bytes = sum(a.nbytes for a in sw_np.values()) + wl.H * 2 + wl.H * 4
    shared = {"us_per_token": us_shared, "shared_expert_us": us_shared_only,
              "us_per_token_with_router": us_router_shared,
              "shared_bytes": shared_bytes,
              "shared_GBps": shared_bytes / (us_shared_only * 1e-6) / 1e9,
              "note": "routed layer + shared expert (FP8 E4M3, 32x32 UE8M0 block scales, "
                      "I = 2304; 35.4 MB); graph replay; shared_expert_us: the shared expert "
                      "alone (two kernels), one call per step in a graph; "
                      "us_per_token_with_router: router logits, then the routed layer with "
                      "the shared expert (four kernels a step)"}
    log(f"decode with the shared expert: {us_shared:.2f} us/token; shared expert alone "
        f"{us_shared_only:.2f} us ({shared['shared_GBps']:.0f} GB/s); router + layer + shared "
        f"expert {us_router_shared:.2f} us/token")
    del sw_d

    # ---------------------------------------------------------------- speculative-verify batches
    # T = 6 and T = 32 tokens per step on the same 384 resident experts.
    from synth.configs import VERIFY6, VERIFY32, STACK1, STACK6
    verify = {}
    for vw in (VERIFY6, VERIFY32):
        n_v = min(vw.steps, 64)
        xv = torch.from_numpy(np.stack([synth.gen_x(vw, s) for s in range(n_v)]).view(np.int16)).to(
            dev).view(torch.bfloat16)
        lv_np = np.stack([synth.gen_logits(vw, s) for s in range(n_v)])
        lv = torch.from_numpy(lv_np).to(dev)
        yv = torch.empty((vw.T, vw.H), dtype=torch.float32, device=dev)
        wsv = torch.empty(moe.moe_fp4_workspace_size(vw.T, vw.H, vw.I, vw.E, vw.k), dtype=torch.uint8,
                          device=dev)

        def step_v(i, xv=xv, lv=lv, yv=yv, wsv=wsv, vw=vw, n_v=n_v):
            j = i % n_v
            moe.moe_fp4_forward(xv[j], lv[j], w, vw.k, y=yv, workspace=wsv)

        us_v = graph_us(step_v)
        timed = [(args.warmup + i) % n_v for i in range(args.steps)]   # the steps graph_us times
        d_v = [len(np.unique(topk_sets(lv_np[s], vw.k))) for s in timed]
        b_v = float(np.mean(d_v)) * expert_bytes(vw.H, vw.I)
        verify[vw.name] = {"T": vw.T, "us_per_step": us_v, "us_per_token": us_v / vw.T,
                           "distinct_experts": float(np.mean(d_v)), "bytes_per_step": b_v,
                           "GBps": b_v / (us_v * 1e-6) / 1e9}
        log(f"verify T={vw.T}: {us_v:.2f} us/step ({us_v / vw.T:.2f} us/token), "
            f"{np.mean(d_v):.1f} distinct experts, {b_v / (us_v * 1e-6) / 1e9:.0f} GB/s")
        del xv, lv, yv, wsv

    # ---------------------------------------------------------------- pruned resident stack
    # 40 layers x 138 experts (103.8 GB in HBM), x_{l+1} = x_l + moe_l(prenorm(x_l)),
    # every layer of every token in one graph.
    stack = {}
    t0 = time.time()
    layers = [moe.ExpertWeights.from_dict(synth.layer_device(STACK1, layer=l, device=dev))
              for l in range(STACK1.layers)]
    torch.cuda.synchronize()
    log(f"stack: {STACK1.layers} x {STACK1.E} experts generated in HBM in {time.time() - t0:.1f} s")
    for sw_ in (STACK1, STACK6):
        n_s = min(sw_.steps, 16)
        xs0 = torch.from_numpy(np.stack([synth.gen_x_f32(sw_, s) for s in range(n_s)])).to(dev)
        lgs_np = [[synth.gen_logits(sw_, s, l) for l in range(sw_.layers)] for s in range(n_s)]
        lgs_s = [[torch.from_numpy(a).to(dev) for a in row] for row in lgs_np]
        xst = xs0.clone()
        wss = torch.empty(moe.moe_fp4_workspace_size(sw_.T, sw_.H, sw_.I, sw_.E, sw_.k),
                          dtype=torch.uint8, device=dev)

        def step_s(i, xst=xst, wss=wss, lgs_s=lgs_s, sw_=sw_, n_s=n_s):
            j = i % n_s
            for l in range(sw_.layers):  # x += moe_l(prenorm(x)), one call per layer
                moe.moe_fp4_forward_residual(xst[j], lgs_s[j][l], layers[l], sw_.k, workspace=wss)

        # a few steps per graph (each step is 40 layer calls)
        saved = (args.warmup, args.steps)
        args.warmup, args.steps = 2, n_s
        us_step = graph_us(step_s)
        args.warmup, args.steps = saved
        timed = [(2 + i) % n_s for i in range(n_s)]   # the steps graph_us times (2 warm-up)
        d_s = [sum(len(np.unique(topk_sets(lgs_np[s][l], sw_.k))) for l in range(sw_.layers))
               for s in timed]
        b_s = float(np.mean(d_s)) * expert_bytes(sw_.H, sw_.I)
        stack[sw_.name] = {"T": sw_.T, "layers": sw_.layers, "E": sw_.E,
                           "us_per_step": us_step, "tokens_per_s": sw_.T / (us_step * 1e-6),
                           "bytes_per_step": b_s, "GBps": b_s / (us_step * 1e-6) / 1e9}
        log(f"stack T={sw_.T}: {us_step / 1e3:.3f} ms per pass of {sw_.layers} layers, "
            f"{sw_.T / (us_step * 1e-6):.0f} tokens/s, {b_s / (us_step * 1e-6) / 1e9:.0f} GB/s")
        del xs0, xst, wss, lgs_s
    del layers
    torch.cuda.empty_cache()

    return routed, shared, verify, stack


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(args, synth, wl, xs, lgs, idx_all):
    """The oracle (test infrastructure: plain double loops, OpenMP) on the same
    units of work as the GPU, on bounded samples, all host threads and one."""
    import oracle
    from synth.configs import VERIFY6, VERIFY32, PREFILL as pf, STACK1
    o = oracle.get()
    threads = o.threads()
    cache = {}

    def experts_of(w_, layer, ids):
        out = {}
        for e in np.unique(ids):
            key = (w_.weight_seed, layer, int(e))
            if key not in cache:
                cache[key] = synth.expert_host(w_, layer, int(e))
            out[int(e)] = cache[key]
        return out

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    res = {}
    # decode tokens, all threads, until the time budget is spent
    spent, n = 0.0, 0
    while spent < args.cpu_seconds and n < len(xs):
        ex = experts_of(wl, 0, idx_all[n])
        spent += timed(lambda: o.forward(wl.H, wl.I, wl.E, wl.k, xs[n:n + 1], lgs[n:n + 1], ex))
        n += 1
    res["decode_us_per_token"] = spent / n * 1e6
    res["decode_tokens"] = n
    # one thread, two decode tokens
    o.set_threads(1)
    t1 = [timed(lambda i=i: o.forward(wl.H, wl.I, wl.E, wl.k, xs[i:i + 1], lgs[i:i + 1],
                                      experts_of(wl, 0, idx_all[i])))
          for i in range(2)]
    o.set_threads(threads)
    res["decode_us_per_token_1_thread"] = float(np.mean(t1)) * 1e6
    # verify steps (one step each)
    for vw in (VERIFY6, VERIFY32):
        x, lg = synth.gen_x(vw, 0), synth.gen_logits(vw, 0)
        ex = experts_of(vw, 0, topk_sets(lg, vw.k))
        res[f"verify_T{vw.T}_us_per_step"] = timed(
            lambda: o.forward(vw.H, vw.I, vw.E, vw.k, x, lg, ex)) * 1e6
    # the prefill chunk: the first 256 of its 2048 tokens, scaled by 8 (the
    # oracle's work is proportional to the tokens it computes)
    x, lg = synth.gen_x(pf, 0), synth.gen_logits(pf, 0)
    n_s = 256
    toks = np.arange(n_s)
    ex = experts_of(pf, 0, topk_sets(lg[:n_s], pf.k))
    t = timed(lambda: o.forward(pf.H, pf.I, pf.E, pf.k, x, lg, ex, tokens=toks))
    res["prefill_ms_per_chunk"] = t * (pf.T / n_s) * 1e3
    # one token of the pruned 40-layer stack (40 layer calls)
    xf = synth.gen_x_f32(STACK1, 0)
    lgs_s = [synth.gen_logits(STACK1, 0, l) for l in range(STACK1.layers)]

    def stack_token():
        xx = xf
        for l in range(STACK1.layers):
            xx = o.stack_layer(STACK1.I, STACK1.E, STACK1.k, xx, lgs_s[l],
                               experts_of(STACK1, l, topk_sets(lgs_s[l], STACK1.k)))

    for l in range(STACK1.layers):     # weight generation stays outside the timing
        experts_of(STACK1, l, topk_sets(lgs_s[l], STACK1.k))
    res["stack_ms_per_token"] = timed(stack_token) * 1e3
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cpu = {"value": res["decode_us_per_token"], "unit": "us/token", "cores": threads,
           "kind": "oracle", "nproc": aff, "cpu_model": cpu_model(),
           "sample": (f"decode: {n} tokens of the timed workload on {threads} threads, and 2 on one "
                      f"thread; verify: one T=6 and one T=32 step; prefill: the first 256 tokens of "
                      f"the 2048-token chunk, scaled by 8; stack: one token through the 40 pruned "
                      f"layers.  Weight generation excluded."),
           "configs": {k: (round(v, 1) if isinstance(v, float) else v) for k, v in res.items()}}
    log(f"cpu oracle: {cpu['value']:.0f} us/token on {threads} threads "
        f"({res['decode_us_per_token_1_thread']:.0f} on one), verify T=6 "
        f"{res['verify_T6_us_per_step'] / 1e3:.0f} ms, T=32 {res['verify_T32_us_per_step'] / 1e3:.0f} ms, "
        f"prefill chunk {res['prefill_ms_per_chunk'] / 1e3:.1f} s, stack token "
        f"{res['stack_ms_per_token']:.0f} ms")
    return cpu


def run_stream(torch, dev, reps=6):
    """Achievable read bandwidth of one kernel reading the decode kernels'
    footprints and a long stream, caches cold (the windows rotate over 6 GiB)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_routed_expert_router_amd", "libmoe_fp4_measure.so"))
    lib.moe_fp4_measure_stream_read.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    total = 6 << 30
    buf = torch.full((total,), 3, dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1 << 21, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, nb in (("w13_75MB", 75202560 + 10240), ("w2_38MB", 37601280 + 10240),
                     ("step_113MB", 112803840), ("long_4GB", 4 << 30)):
        best = None
        for threads, per_cu, unroll in ((512, 2, 8), (256, 4, 8), (1024, 1, 8), (512, 2, 16)):
            ts = []
            for r in range(reps):
                flush.sum()
                span = (total - nb) // (1 << 24)
                off = ((r * 7 + 3) % max(span, 1)) * (1 << 24)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                b.record()
                rc = lib.moe_fp4_measure_stream_read(
                    ctypes.c_void_p(buf.data_ptr() + off), ctypes.c_size_t(nb), cus * per_cu, threads,
                    unroll, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(a.cuda_event),
                    ctypes.c_void_p(b.cuda_event), ctypes.c_void_p(stream.cuda_stream))
                assert rc == 0, rc
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3)
            us = float(np.median(ts[1:]))
            if best is None or us < best["us"]:
                best = {"bytes": nb, "us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                        "threads": threads, "workgroups": cus * per_cu, "loads_in_flight": unroll}
        out[name] = best
        log(f"stream read {name}: {best['us']:.2f} us, {best['GBps']:.0f} GB/s cold")
    del buf, flush, sink
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm (graph replay) decode figures: every decode launch is then cold")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read measurement")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip one GPU's share of the layer on eight (decode TP-8, prefill EP-8)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the router, shared-expert, verify and stack figures (profiling runs)")
    ap.add_argument("--eager", action="store_true",
                    help="no graph capture: the cold value is the mean span of eager steps, from "
                         "the first kernel's start to the last one's end (counter-collection runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X and this build has "
              "no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import mxfp4_routed_expert_router_amd as moe
    from synth.configs import DECODE as wl, PREFILL as pf

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"device: {torch.cuda.get_device_name(dev)}")

    # ---------------------------------------------------------------- set-up
    t0 = time.time()
    w = moe.ExpertWeights.from_dict(synth.layer_device(wl, layer=0, device=dev))
    torch.cuda.synchronize()
    log(f"weights: {wl.E} experts x {expert_bytes(wl.H, wl.I)} B generated in HBM "
        f"in {time.time() - t0:.1f} s")
    n_gen = args.warmup + max(args.steps, 1)   # one distinct token per step
    xs = np.stack([synth.gen_x(wl, s)[0] for s in range(n_gen)])
    lgs = np.stack([synth.gen_logits(wl, s)[0] for s in range(n_gen)])
    x_d = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
    lg_d = torch.from_numpy(lgs).to(dev)
    y_d = torch.empty((n_gen, wl.H), dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_fp4_workspace_size(1, wl.H, wl.I, wl.E, wl.k), dtype=torch.uint8,
                     device=dev)
    idx_all = topk_sets(lgs, wl.k)
    timed_ids = [args.warmup + i for i in range(args.steps)]

    def step(i, events=None):
        j = i % n_gen
        xi, li, yi = x_d[j:j + 1], lg_d[j:j + 1], y_d[j:j + 1]
        if events is None:
            moe.moe_fp4_forward(xi, li, w, wl.k, y=yi, workspace=ws)
        else:
            moe.moe_fp4_forward_profiled(xi, li, w, wl.k, events, y=yi, workspace=ws)

    by = [decode_bytes(wl, idx_all[i][None]) for i in timed_ids]
    k_bytes = {n: float(np.mean([b[n] for b in by])) for n in ("route", "w13", "w2")}
    step_bytes = k_bytes["route"] + k_bytes["w13"] + k_bytes["w2"]

    # ---------------------------------------------------------------- decode, cold (the value)
    # Every step runs with L2 and the MALL cold: a read-only sweep of 1 GiB
    # (libmoe_fp4_measure's streaming read) before each step, which leaves no
    # dirty lines to write back during the step.  The K timed steps, each after
    # its sweep, are one HIP graph; a second graph holds the K sweeps alone.
    # Both are replayed (wall clock between synchronisations, median of reps)
    # and the cold step is the difference over K: every launch gap between the
    # layer's kernels is inside it, the sweeps are not.
    import ctypes
    mlib = ctypes.CDLL(os.path.join(ROOT, "mxfp4_routed_expert_router_amd", "libmoe_fp4_measure.so"))
    mlib.moe_fp4_measure_stream_read.restype = ctypes.c_int
    fbuf = torch.full((1 << 30,), 1, dtype=torch.uint8, device=dev)
    fsink = torch.empty(1 << 21, dtype=torch.int32, device=dev)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count

    def sweep():
        rc = mlib.moe_fp4_measure_stream_read(
            ctypes.c_void_p(fbuf.data_ptr()), ctypes.c_size_t(1 << 30), 2 * n_cu, 512, 8,
            ctypes.c_void_p(fsink.data_ptr()), None, None,
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        assert rc == 0, rc

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        return g

    def replay_us(g, reps=5):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)) * 1e6

    for i in range(args.warmup):
        sweep()
        step(i)
    torch.cuda.synchronize()

    def cold_step(n):
        sweep()
        step(args.warmup + n)

    if not args.eager:
        g_cold = graph_of(cold_step, args.steps)
        g_sweep = graph_of(lambda n: sweep(), args.steps)
        t_cold, t_sweep = replay_us(g_cold), replay_us(g_sweep)
        us_tok = (t_cold - t_sweep) / args.steps / wl.T
        del g_cold, g_sweep
    # kernel durations for the roofline: the same cold steps run eagerly, each
    # kernel's dispatch recording its own start and end events
    # (moe_fp4_forward_profiled); warm-up steps are cold too, so every launch of
    # the decode kernels in a --no-warm run is a cold one
    # (the W warm-up steps run again first, inside the host's head start: the
    # first launches after the spin are slower while the clocks come back)
    evc = [moe.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    for i in range(args.warmup):
        sweep()
        step(i)
    for n, i in enumerate(timed_ids):
        sweep()
        step(i, evc[n])
    torch.cuda.synchronize()
    # One GPU's share of the layer on eight, decode in tensor parallel: the same
    # tokens and routing, 288 of the 2304 intermediate rows of every expert
    # (its y is the partial sum an all-reduce of 20 KB a token would complete),
    # caches cold as above.
    tp8 = None
    if not args.no_shards and not args.eager:
        from synth.configs import DECODE_TP8 as wt
        w_tp = moe.ExpertWeights.from_dict(synth.layer_device(wt, layer=0, device=dev))
        ws_tp = torch.empty(moe.moe_fp4_workspace_size(1, wt.H, wt.I, wt.E, wt.k), dtype=torch.uint8,
                            device=dev)

        def step_tp(i):
            j = i % n_gen
            moe.moe_fp4_forward(x_d[j:j + 1], lg_d[j:j + 1], w_tp, wt.k, y=y_d[j:j + 1], workspace=ws_tp)

        for i in range(args.warmup):
            sweep()
            step_tp(i)
        g_c = graph_of(lambda n: (sweep(), step_tp(args.warmup + n)), args.steps)
        g_s = graph_of(lambda n: sweep(), args.steps)
        us_tp = (replay_us(g_c) - replay_us(g_s)) / args.steps
        del g_c, g_s
        b_tp = float(np.mean([sum(v for n, v in decode_bytes(wt, idx_all[i][None]).items() if n != "D")
                              for i in timed_ids]))
        tp8 = {"workload": "decode T=1, E=384, top-6, H=5120, I=288 (one GPU's 1/8 of every expert's "
                           "intermediate rows), the decode workload's tokens, L2 and MALL cold",
               "us_per_token": us_tp, "bytes_per_step": b_tp,
               "GBps": b_tp / (us_tp * 1e-6) / 1e9, "hbm_frac": b_tp / (us_tp * 1e-6) / 1e9 / HBM_PEAK_GBPS,
               "note": "one GPU's share only: its y is a partial sum; the all-reduce of T x 5120 fp32 "
                       "that completes it on eight GPUs is not run (one GPU)"}
        log(f"decode TP-8 shard (I=288): {us_tp:.2f} us/token cold, {tp8['GBps']:.0f} GB/s")
        del w_tp, ws_tp
    del fbuf, fsink
    if args.eager:
        ev = [e.events for e in evc]
        span = np.array([e[2].elapsed_time(e[5]) for e in ev]) * 1e3   # w1/w3 start -> w2 end
        us_tok = float(span.mean()) / wl.T
        t_cold, t_sweep = us_tok * wl.T * args.steps, 0.0
    st = np.array([e.stage_ms() for e in evc]) * 1e3                   # [steps, 4] us
    # with one token the routing runs inside the w1/w3 kernel: no launch of its own
    k_us = {"route": float(st[:, 0].mean()) if wl.T > 1 else None, "w13": float(st[:, 1].mean()),
            "w2": float(st[:, 2].mean())}
    dom = max(("w13", "w2"), key=lambda n: k_us[n])
    achieved = k_bytes[dom] / (k_us[dom] * 1e-6) / 1e9
    log(f"decode cold: {us_tok:.2f} us/token (graph of {args.steps} swept steps {t_cold / args.steps:.1f} "
        f"us each, sweeps alone {t_sweep / args.steps:.1f}), {step_bytes / (us_tok * 1e-6) / 1e9:.0f} "
        f"GB/s; kernels w1/w3 {k_us['w13']:.2f} us, w2 {k_us['w2']:.2f} us")

    # ---------------------------------------------------------------- decode, warm
    # The same steps captured into one HIP graph and replayed (caches warm:
    # consecutive tokens share experts, and the MALL holds part of the layer).
    def graph_us(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                fn(args.warmup + i)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / args.steps

    warm = None
    routed = shared = None
    verify, stack = {}, {}
    if not args.no_warm and not args.eager:
        us_warm = graph_us(step)
        evs = [moe.StageEvents() for _ in range(args.steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        for i in range(args.warmup):
            step(i)
        for n, i in enumerate(timed_ids):
            step(i, evs[n])
        torch.cuda.synchronize()
        stw = np.array([e.stage_ms() for e in evs]) * 1e3
        eager_t0 = time.perf_counter()
        for i in timed_ids:
            step(i)
        torch.cuda.synchronize()
        us_eager = (time.perf_counter() - eager_t0) * 1e6 / args.steps
        warm = {"us_per_token": us_warm, "GBps": step_bytes / (us_warm * 1e-6) / 1e9,
                "w13_us": float(stw[:, 1].mean()), "w2_us": float(stw[:, 2].mean()),
                "us_per_token_eager": us_eager,
                "note": "the timed steps captured in one HIP graph, replayed once (wall clock); "
                        "kernel times from dispatch events, steps back to back; eager: one "
                        "Python call per step"}
        log(f"decode warm: {us_warm:.2f} us/token graph replay; kernels w1/w3 "
            f"{warm['w13_us']:.2f} us, w2 {warm['w2_us']:.2f} us; eager {us_eager:.2f} us/token")
        if not args.no_extras:
            routed, shared, verify, stack = run_extras(args, moe, synth, torch, dev, w, wl, x_d, lg_d,
                                                       y_d, ws, n_gen, graph_us)

    # ---------------------------------------------------------------- prefill chunk
    prefill = prefill_mx = None
    if args.prefill_reps > 0:
        xp = torch.from_numpy(synth.gen_x(pf, 0).view(np.int16)).to(dev).view(torch.bfloat16)
        lp_np = synth.gen_logits(pf, 0)
        lp = torch.from_numpy(lp_np).to(dev)
        yp = torch.empty((pf.T, pf.H), dtype=torch.float32, device=dev)
        pairs = pf.T * pf.k
        flops = pairs * (2 * 2 * pf.H * pf.I + 2 * pf.I * pf.H)
        Dp = len(np.unique(topk_sets(lp_np, pf.k)))
        p_bytes = Dp * expert_bytes(pf.H, pf.I) + pf.T * pf.H * 2 + pf.T * pf.H * 4

        def run_prefill(mode, label, mfma_peak):
            wsp = torch.empty(moe.moe_fp4_workspace_size(pf.T, pf.H, pf.I, pf.E, pf.k, mode),
                              dtype=torch.uint8, device=dev)
            for _ in range(2):
                moe.moe_fp4_forward(xp, lp, w, pf.k, y=yp, mode=mode, workspace=wsp)
            torch.cuda.synchronize()

            def chunk_ms(call):
                # median over the reps of plain calls back to back, each between
                # two events on the stream (markers between the calls, not per
                # dispatch)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.prefill_reps)]
                for e0, e1 in evs:
                    e0.record()
                    call()
                    e1.record()
                torch.cuda.synchronize()
                return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))

            # the stage split: the same calls with per-dispatch events, which
            # themselves cost a few percent of the chunk; run first, they also
            # bring the GPU out of the decode phase's memory-bound state
            evp = [moe.StageEvents() for _ in range(args.prefill_reps)]
            for i in range(args.prefill_reps):
                moe.moe_fp4_forward_profiled(xp, lp, w, pf.k, evp[i], y=yp, mode=mode, workspace=wsp)
            torch.cuda.synchronize()
            pst = np.array([e.stage_ms() for e in evp])
            p_ms = chunk_ms(lambda: moe.moe_fp4_forward(xp, lp, w, pf.k, y=yp, mode=mode, workspace=wsp))
            out = {
                "workload": "prefill chunk T=2048, E=384, top-6, H=5120, I=2304, Zipf(0.3) logit bias",
                "activations": label,
                "ms_per_chunk": p_ms, "tflops": flops / (p_ms * 1e-3) / 1e12, "gflop": flops / 1e9,
                "distinct_experts": Dp, "weight_GB": Dp * expert_bytes(pf.H, pf.I) / 1e9,
                "hbm_frac": p_bytes / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "mfma_frac": flops / (p_ms * 1e-3) / 1e12 / mfma_peak, "mfma_peak_tflops": mfma_peak,
                "kernel_ms": {"route": float(pst[:, 0].mean()), "w13": float(pst[:, 1].mean()),
                              "w2": float(pst[:, 2].mean()), "combine": float(pst[:, 3].mean())},
            }
            out["roofline_frac"] = max(out["hbm_frac"], out["mfma_frac"])
            # the same chunk with the saliency side output (moe_fp4_forward_saliency)
            sal = torch.zeros(pf.E, dtype=torch.float32, device=dev)
            moe.moe_fp4_forward_saliency(xp, lp, w, pf.k, saliency=sal, y=yp, mode=mode, workspace=wsp)
            torch.cuda.synchronize()
            out["ms_per_chunk_with_saliency"] = chunk_ms(lambda: moe.moe_fp4_forward_saliency(
                xp, lp, w, pf.k, saliency=sal, y=yp, mode=mode, workspace=wsp))
            log(f"prefill ({label}): {p_ms:.3f} ms/chunk, {out['tflops']:.1f} TFLOP/s, HBM frac "
                f"{out['hbm_frac']:.2f}, kernels {out['kernel_ms']}; with saliency "
                f"{out['ms_per_chunk_with_saliency']:.3f} ms")
            del wsp, sal
            return out

        prefill = run_prefill(moe.MODE_PREFILL, "bf16 (MFMA 16x16x32 bf16, FP4 staged in LDS and "
                                                "decoded to bf16 in registers)", BF16_PEAK_TFLOPS)
        prefill_mx = run_prefill(moe.MODE_PREFILL_MXFP8,
                                 "MXFP8 (x and h quantised; FP4 x FP8 scaled MFMA 16x16x128)",
                                 FP8_PEAK_TFLOPS)

    # One GPU's share of the 2048-token chunk on eight, expert parallel: 48
    # experts and the 1,536 pairs routed to them (32 an expert, as in the chunk)
    ep8 = None
    if args.prefill_reps > 0 and not args.no_shards:
        from synth.configs import PREFILL_EP8 as we
        w_ep = moe.ExpertWeights.from_dict(synth.layer_device(we, layer=0, device=dev))
        xe = torch.from_numpy(synth.gen_x(we, 0).view(np.int16)).to(dev).view(torch.bfloat16)
        le_np = synth.gen_logits(we, 0)
        le = torch.from_numpy(le_np).to(dev)
        ye = torch.empty((we.T, we.H), dtype=torch.float32, device=dev)
        De = len(np.unique(topk_sets(le_np, we.k)))
        e_bytes = De * expert_bytes(we.H, we.I) + we.T * we.H * 2 + we.T * we.H * 4
        ep8 = {"workload": "48 experts (one GPU's 1/8 of 384), 256 tokens top-6 over them: 1,536 pairs, "
                           "32 an expert, H=5120, I=2304, Zipf(0.3) logit bias",
               "distinct_experts": De, "bytes": e_bytes}
        for mode, name in ((moe.MODE_PREFILL, "bf16"), (moe.MODE_PREFILL_MXFP8, "mxfp8")):
            wse = torch.empty(moe.moe_fp4_workspace_size(we.T, we.H, we.I, we.E, we.k, mode),
                              dtype=torch.uint8, device=dev)
            for _ in range(2):
                moe.moe_fp4_forward(xe, le, w_ep, we.k, y=ye, mode=mode, workspace=wse)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.prefill_reps)]
            for e0, e1 in evs:
                e0.record()
                moe.moe_fp4_forward(xe, le, w_ep, we.k, y=ye, mode=mode, workspace=wse)
                e1.record()
            torch.cuda.synchronize()
            ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
            full = (prefill if mode == moe.MODE_PREFILL else prefill_mx)["ms_per_chunk"]
            ep8[name] = {"ms": ms, "GBps": e_bytes / (ms * 1e-3) / 1e9,
                         "hbm_frac": e_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "full_chunk_ms_over_8": full / 8}
            log(f"prefill EP-8 shard ({name}): {ms:.3f} ms, {ep8[name]['GBps']:.0f} GB/s "
                f"(full chunk / 8: {full / 8:.3f} ms)")
            del wse
        ep8["note"] = ("one GPU's share only: the all-to-all that brings each GPU its pairs' x rows "
                       "and the one that returns their outputs are not run (one GPU)")
        del w_ep
    del w
    torch.cuda.empty_cache()
    stream = None if args.no_stream else run_stream(torch, dev)
    cpu = None if args.no_cpu else run_cpu_baseline(args, synth, wl, xs, lgs, idx_all)

    res = {
        "metric": METRIC,
        "value": round(us_tok, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_tok * wl.T / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode T=1, E=384 resident (7.22 GB FP4 E2M1 + UE8M0), top-6, "
                               f"H=5120, I=2304, Zipf(1.1) logit bias, {n_gen} distinct tokens "
                               f"({args.warmup} warm-up, {args.steps} timed), L2 and MALL cold",
                   "T": wl.T, "E": wl.E, "k": wl.k, "H": wl.H, "I": wl.I},
        "tokens_per_s": 1e6 / us_tok,
        "hbm_GBps": step_bytes / (us_tok * 1e-6) / 1e9,
        "step_bytes": step_bytes,
        "step_frac": step_bytes / (us_tok * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": DECODE_KERNELS[dom],
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic(DECODE_KERNELS[dom]), "traffic_unit": "bytes/launch",
                     "bytes_per_launch": k_bytes[dom], "avg_us": k_us[dom],
                     "trace_avg_us": traced_mean_us(DECODE_KERNELS[dom]),
                     "note": "cold launches (L2 and MALL flushed before each step)"},
        "kernels_us": {n: (round(v, 3) if v is not None else None) for n, v in k_us.items()},
        "timing": ("value (--eager): mean span from the start of each cold step's first kernel to "
                   "the end of its last (per-dispatch events), each step after a 1 GiB read-only "
                   "sweep" if args.eager else
                   "value: the timed steps, each on a fresh token after a 1 GiB read-only sweep that "
                  "leaves L2 and the MALL cold, captured in one HIP graph and replayed; minus the "
                  "same graph of sweeps alone; divided by the steps.  Kernel durations (roofline): "
                  "the same cold steps run eagerly with start/end events recorded by each kernel's "
                  "own dispatch.  The one-token routing runs inside the w1/w3 kernel and its bytes "
                  "(the logits) are counted there"),
        "warm": warm,
        "stream_read": stream,
        "decode_routed": routed,
        "decode_shared": shared,
        "verify": verify,
        "stack": stack,
        "prefill": prefill,
        "prefill_mxfp8": prefill_mx,
        "shards": {"decode_tp8": tp8, "prefill_ep8": ep8},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
