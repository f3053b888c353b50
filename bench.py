#!/usr/bin/env python3
"""Benchmark: MoE-layer decode tokens/s and achieved HBM GB/s of the 4-bit
affine GEMV path on one MI355X.

Workload: one MoE layer decode step, batch 1 token -- hidden 2816, 128
experts, top-8 softmax routing with renormalisation, expert intermediate 704,
shared-expert intermediate 2112; 8-bit affine router, 4-bit affine (group
64) experts; bf16 activations ~N(0,1), fp32 accumulation; seeded synthetic
weights (the pages publish no dataset or checkpoint for this step).

One step = one token through the whole hot path of one layer (router GEMV,
softmax top-8, shared and 8 routed expert FFNs, weighted combine) in a single
launch of the library.  To measure HBM and not the 256 MB Infinity Cache,
the layer's weights are held in 32 separate copies (~14 GB) and consecutive
steps cycle through them, each with its own input token.

The 128-token prefill chunk (router with the Zipf prior, then the grouped
MFMA prefill) is timed as a second, reported-only leg on the same weights;
the standalone 4-bit GEMV on a large matrix of the decode width, the
30-layer stack and (with --streaming) the expert pool are further
reported-only legs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-prefill] [--no-gemv] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0
COPIES = 32
SAMPLE = 8  # launches per group bracketed by one pair of kernel-timing events
N_TOKENS = 64
PF_TOKENS = 128
COPY_BYTES = 1 << 30
# HBM traffic of the decode kernel from rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, scaled by the same counters on a plain copy of known size);
# valid only for the kernel sources it was measured on.
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_moe_step_layer_decode_pmc.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_quantized_gemv_amd", "csrc", f)
                  for f in ("qmoe_decode.hip", "qmoe_common.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """(bytes per launch, note) from the committed counter summary, or
    (None, reason) when it is missing or the kernel changed since."""
    if not os.path.exists(PMC_SUMMARY):
        return None, "no counter summary"
    kv = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None, "kernel changed since the counters were taken"
    try:
        return int(kv["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-scaled"
    except (KeyError, ValueError):
        return None, "counter summary incomplete"


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(lw, X, seconds_hint: float = 15.0):
    """The fp64 oracle (as it stands) over a bounded sample of tokens of the
    same layer, threaded over tokens on the host cores."""
    import oracle

    L = oracle.OracleLayer(lw)
    cores = host_threads()
    t0 = time.perf_counter()
    L.forward(X[0])
    one = time.perf_counter() - t0
    n = int(max(cores, min(4 * cores, seconds_hint * cores / max(one, 1e-3))))
    n = min(n, X.shape[0])
    threads = min(cores, n)
    t0 = time.perf_counter()
    oracle.forward_many(L, X[:n], threads=threads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} decode tokens of one layer (same shapes and weights), fp64 scalar C, "
                      f"{threads} threads over tokens"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-gemv", action="store_true", help="skip the standalone GEMV leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the 30-layer stack leg")
    ap.add_argument("--streaming", action="store_true",
                    help="only the expert-streaming leg (30 layers, pinned host experts, "
                         "16 device slots per layer); prints its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--phased", action="store_true",
                    help="time the three-launch variant instead of the single launch")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the MoE step runs on one GPU: --gpus must be 1 (the "
                          "library has no multi-GPU path)"}))
        sys.exit(2)

    import torch

    import bit_quantized_gemv_amd as q
    import synth
    import synth.device as sd

    if args.streaming:
        print(json.dumps(streaming_leg(torch, q, synth, sd)), flush=True)
        return

    wl = synth.WORKLOADS["layer_decode"]
    log("generating layer weights")
    lw = synth.make_layer(wl, 0)
    algo_bytes = lw.algorithmic_bytes_decode()
    X = synth.make_tokens(wl, N_TOKENS, stream=1)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"uploading {COPIES} copies of {lw.blobs.nbytes / 1e6:.0f} MB expert blobs")
    base = sd.DeviceLayer(lw)
    layers = [base]
    for i in range(1, COPIES):
        blobs = torch.empty_like(base.blobs)
        blobs.copy_(base.blobs)
        # router and shared expert are uploaded again per copy (own addresses)
        layers.append(sd.DeviceLayer(lw, blobs=blobs))
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    outs = torch.empty(N_TOKENS, wl.hidden, dtype=torch.int16, device=dev)
    idx = torch.empty(wl.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(wl.top_k, dtype=torch.float32, device=dev)
    ws = layers[0].layer.new_workspace(1)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i, e0=None, e1=None):
        L = layers[i % COPIES].layer
        t = i % N_TOKENS
        if e0 is not None and not args.phased:
            q.qmoe_moe_decode_timed(L, Xd[t], None, False, outs[t], idx, w, ws,
                                    e0.cuda_event, e1.cuda_event, stream=sptr)
        else:
            q.qmoe_moe_decode(L, Xd[t], None, False, outs[t], idx, w, ws, stream=sptr,
                              phased=args.phased)

    # The timed loop calls the C entry point with its arguments marshalled
    # beforehand (layer structs and device addresses), so that host-side
    # Python work does not throttle the launches.
    import ctypes

    lib = q.lib()
    timed_fn = lib.qmoe_moe_decode_timed
    cstructs = [ctypes.byref(dl.layer.c()) for dl in layers]
    xs = [Xd[t].data_ptr() for t in range(N_TOKENS)]
    os_ = [outs[t].data_ptr() for t in range(N_TOKENS)]
    ws_args = (idx.data_ptr(), w.data_ptr(), ws.data_ptr(), ws.numel())

    plain_fn = lib.qmoe_moe_decode

    def timed_step(i, e0, e1):
        t = i % N_TOKENS
        rc = timed_fn(cstructs[i % COPIES], xs[t], None, 0, os_[t], ws_args[0], ws_args[1],
                      ws_args[2], ws_args[3], sptr, e0, e1)
        if rc:
            raise q.QmoeError("qmoe_moe_decode_timed", rc)

    def plain_step(i):
        t = i % N_TOKENS
        rc = plain_fn(cstructs[i % COPIES], xs[t], None, 0, os_[t], ws_args[0], ws_args[1],
                      ws_args[2], ws_args[3], sptr)
        if rc:
            raise q.QmoeError("qmoe_moe_decode", rc)

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if q.qmoe_workspace_status(ws) != 0:
        raise SystemExit("device wait failure during warmup")

    # timed region: K steps in groups of SAMPLE consecutive launches.  The
    # first launch of a group records a HIP event at its kernel's start and
    # the last one at its kernel's end (the dispatches' own timestamps, on
    # the launch stream); the launches in between are plain.  A group's span
    # over SAMPLE is the average launch duration with the kernels running
    # back to back, as a caller's would.  (A launch that records events
    # costs the host about 29 us, more than the kernel takes: with events on
    # every launch the loop would be host-bound.)  The three-launch variant
    # is bracketed by event records every step.
    sample = 1 if args.phased else SAMPLE
    K = max(sample, args.steps - args.steps % sample)
    groups = K // sample
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * groups)]
    for e in ev:  # create the underlying hipEvents before the timed region
        e.record(stream)
    evh = [e.cuda_event for e in ev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.phased:
        for i in range(K):
            ev[2 * i].record(stream)
            step(args.warmup + i)
            ev[2 * i + 1].record(stream)
    else:
        for i in range(K):
            n, r = divmod(i, sample)
            e0 = evh[2 * n] if r == 0 else None
            e1 = evh[2 * n + 1] if r == sample - 1 else None
            if e0 or e1:
                timed_step(args.warmup + i, e0, e1)
            else:
                plain_step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code = q.qmoe_workspace_status(ws)
    if code != 0:
        raise SystemExit(f"device wait failure (code {code})")
    kern_ms = np.array([ev[2 * n].elapsed_time(ev[2 * n + 1]) / sample for n in range(groups)])
    kern_us = float(np.mean(kern_ms) * 1e3)
    kern_med_us = float(np.median(kern_ms) * 1e3)
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    tok_s = K / elapsed
    achieved = algo_bytes / (kern_us * 1e-6) / 1e9
    traffic, traffic_note = measured_traffic()
    log(f"step {ms_per_step * 1e3:.2f} us, kernel mean {kern_us:.2f} us median {kern_med_us:.2f} us, "
        f"{achieved:.0f} GB/s algorithmic")

    res = {
        "metric": "MoE-layer decode tokens/s + achieved HBM GB/s vs peak (4-bit affine GEMV)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; 4-bit/8-bit affine g64 weights, bf16 N(0,1) tokens)",
        "config": {"workload": "MoE layer decode, batch 1: hidden 2816, 128 experts, top-8, "
                               "expert inter 704, shared inter 2112, 8-bit router",
                   "launch": "phased (3 launches)" if args.phased else "single launch",
                   "weight_copies": COPIES, "algorithmic_bytes_per_step": algo_bytes,
                   "codes": "u4 experts / u8 router, affine g64, fp16 scale+bias",
                   "activations": "bf16 in, f32 accumulation, bf16 out"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_source": traffic_note,
                     "kernel": "k_moe_step (whole decode step)" if not args.phased else
                               "k_moe_step (three role launches)",
                     "kernel_us_mean": kern_us, "kernel_us_median": kern_med_us,
                     "launch_us_basis": f"HIP events spanning {sample} consecutive launches, "
                                        f"{groups} groups",},
    }
    if not args.no_prefill:
        res["prefill"] = prefill_leg(torch, q, synth, sd, lw, layers, wl, sptr)
    if not args.no_gemv:
        res["gemv"] = gemv_leg(torch, q, sptr)
    if not args.no_stack:
        del layers
        torch.cuda.empty_cache()
        res["stack"] = stack_leg(torch, q, synth, sd, sptr)
    if args.copy_calibration:
        copy_calibration(torch)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(lw, X)
    print(json.dumps(res), flush=True)


def prefill_leg(torch, q, synth, sd, lw, layers, wl, sptr, iters: int = 64):
    """Time one 128-token chunk (router top-8 with the Zipf log-prior, then
    the grouped prefill) per iteration, cycling through the weight copies."""
    pw = synth.WORKLOADS["prefill128"]
    prior = synth.zipf_prior(pw, 0)
    bias = torch.from_numpy(prior.astype(np.float32)).cuda()
    Xp = torch.from_numpy(synth.make_tokens(pw, PF_TOKENS, stream=2).view(np.int16)).cuda()
    T, E, K = PF_TOKENS, wl.n_experts, wl.top_k
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    out = torch.empty(T, wl.hidden, dtype=torch.int16, device="cuda")
    rws = torch.zeros(q.qmoe_router_workspace_bytes(E, T), dtype=torch.uint8, device="cuda")
    ws = layers[0].layer.new_workspace(T)
    saved = [dl.layer.logit_bias for dl in layers]
    for dl in layers:
        dl.layer.logit_bias = bias
        dl.layer._c = None

    def chunk(i):
        L = layers[i % COPIES].layer
        q.qmoe_router_topk(L.router, bias, Xp, T, K, idx, w, None, rws, stream=sptr)
        q.qmoe_prefill_grouped(L, Xp, T, idx, w, None, out, ws, stream=sptr)

    for i in range(8):
        chunk(i)
    torch.cuda.synchronize()
    distinct = int(torch.unique(idx).numel())
    hottest = int(torch.bincount(idx.flatten().long(), minlength=E).max())
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * iters)]
    for i in range(iters):
        ev[2 * i].record(stream)
        chunk(8 + i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(iters)]) * 1e3)
    for dl, b in zip(layers, saved):
        dl.layer.logit_bias = b
        dl.layer._c = None
    g, u, d = lw.expert(0)
    blob = sum(m.q.nbytes + m.s.nbytes + m.b.nbytes for m in (g, u, d))
    shared = sum(m.q.nbytes + m.s.nbytes + m.b.nbytes for m in (lw.sh_gate, lw.sh_up, lw.sh_down))
    router = lw.router.q.nbytes + lw.router.s.nbytes + lw.router.b.nbytes
    nbytes = router + shared + distinct * blob + 2 * 2 * T * wl.hidden
    H, I, Is = wl.hidden, wl.inter, wl.shared_inter
    flops = 2.0 * T * K * 3 * H * I + 2.0 * T * 3 * H * Is
    log(f"prefill chunk {us:.1f} us: {distinct} experts, hottest {hottest} rows")
    return {"workload": "128-token prefill chunk, Zipf(1.1) log-prior on the router logits, "
                        "weights of the decode layer",
            "tokens_per_s": T / (us * 1e-6), "us_per_chunk": us,
            "distinct_experts": distinct, "hottest_expert_rows": hottest,
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (us * 1e-6) / 1e9,
            "flops": flops, "achieved_TFLOPs": flops / (us * 1e-6) / 1e12,
            "mfma_f16_peak_TFLOPs": MFMA_F16_PEAK_TFS}


def stack_leg(torch, q, synth, sd, sptr, tokens: int = 256, warmup: int = 8):
    """The 30-layer decode stack (RMSNorm -> router top-8 -> shared + routed
    FFN -> residual per layer, independent seeded layers, all resident).
    Two ways: qmoe_stack_decode (one launch per token: every layer in one
    kernel), and 30 one-layer launches per token (for every SAMPLE-th token
    events record the first kernel's start and the last kernel's end)."""
    import ctypes

    st = synth.WORKLOADS["stack30_decode"]
    log(f"generating {st.layers} stack layers")
    dls, nbytes = [], 0
    for l in range(st.layers):
        lw = synth.make_layer(st, l)
        nbytes += lw.algorithmic_bytes_decode() + lw.gamma.nbytes
        dl = sd.DeviceLayer(lw)
        dl.lw = None  # keep only the device copy
        dls.append(dl)
    X = torch.from_numpy(synth.make_tokens(st, tokens, stream=3).view(np.int16)).cuda()
    H, K = st.hidden, st.top_k
    n = st.layers
    stream = torch.cuda.current_stream()

    # one launch per token
    stk = q.Stack([dl.layer for dl in dls])
    out = torch.empty(H, dtype=torch.int16, device="cuda")
    fs = q.lib().qmoe_stack_decode
    shape = ctypes.byref(stk.shape.c())
    targs = (stk.table.data_ptr(), n)
    wsa = (stk.ws.data_ptr(), stk.ws.numel())

    def token1(t):
        rc = fs(shape, targs[0], targs[1], X[t].data_ptr(), out.data_ptr(), None, None, None,
                wsa[0], wsa[1], sptr)
        if rc:
            raise q.QmoeError("qmoe_stack_decode", rc)

    for t in range(warmup):
        token1(t)
    torch.cuda.synchronize()
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(2 * tokens)]
    t0 = time.perf_counter()
    for t in range(tokens):
        ev1[2 * t].record(stream)
        token1(t)
        ev1[2 * t + 1].record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter() - t0
    if q.qmoe_workspace_status(stk.ws) != 0:
        raise SystemExit("device wait failure in the one-launch stack")
    k1 = np.array([ev1[2 * i].elapsed_time(ev1[2 * i + 1]) for i in range(tokens)]) * 1e3
    log(f"stack, one launch per token: {tokens / wall1:.0f} tokens/s, "
        f"{k1.mean():.1f} us per token ({k1.mean() / n:.2f} us per layer)")

    # one launch per layer
    buf = [torch.empty(H, dtype=torch.int16, device="cuda") for _ in range(2)]
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    ws = dls[0].layer.new_workspace(1)
    fn = q.lib().qmoe_moe_decode_timed
    cl = [ctypes.byref(dl.layer.c()) for dl in dls]
    bp = [b.data_ptr() for b in buf]
    wsa = (idx.data_ptr(), w.data_ptr(), ws.data_ptr(), ws.numel())
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * tokens)]
    for e in ev:
        e.record(stream)
    evh = [e.cuda_event for e in ev]

    def token(t, timed):
        src = X[t].data_ptr()
        for l in range(n):
            dst = bp[l & 1]
            e0 = evh[2 * t] if timed and l == 0 else None
            e1 = evh[2 * t + 1] if timed and l == n - 1 else None
            rc = fn(cl[l], src, None, 1, dst, wsa[0], wsa[1], wsa[2], wsa[3], sptr, e0, e1)
            if rc:
                raise q.QmoeError("qmoe_moe_decode_timed", rc)
            src = dst

    for t in range(warmup):
        token(t, False)
    torch.cuda.synchronize()
    # every SAMPLE-th token's launches are bracketed by timing events, the
    # first layer's start and the last layer's end (a launch with events
    # costs the host more than the kernel takes)
    t0 = time.perf_counter()
    for t in range(tokens):
        token(t, t % SAMPLE == 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if q.qmoe_workspace_status(ws) != 0:
        raise SystemExit("device wait failure in the stack leg")
    kern_tok = np.array([ev[2 * t].elapsed_time(ev[2 * t + 1])
                         for t in range(0, tokens, SAMPLE)]) * 1e3
    kern_token_us = float(kern_tok.mean())
    kern = kern_tok / n
    log(f"stack, one launch per layer: {tokens / wall:.0f} tokens/s, "
        f"{kern.mean():.2f} us per layer (events over each sampled token)")
    return {"workload": "30-layer MoE decode stack, batch 1, RMSNorm + residual per layer, "
                        "independent seeded layers, all experts resident",
            "algorithmic_bytes_per_token": nbytes,
            "one_launch": {
                "entry": "qmoe_stack_decode", "tokens_per_s": tokens / wall1,
                "us_per_token": wall1 * 1e6 / tokens, "event_us_per_token": float(k1.mean()),
                "event_us_per_token_median": float(np.median(k1)),
                "achieved_GBps": nbytes / (k1.mean() * 1e-6) / 1e9,
                "frac_of_hbm_peak": nbytes / (k1.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "launch_per_layer": {
                "entry": "qmoe_moe_decode_timed", "tokens_per_s": tokens / wall,
                "us_per_token": wall * 1e6 / tokens,
                "event_us_per_token": kern_token_us, "event_us_per_layer": float(kern.mean()),
                "achieved_GBps": nbytes / (kern_token_us * 1e-6) / 1e9,
                "frac_of_hbm_peak": nbytes / (kern_token_us * 1e-6) / 1e9 / HBM_PEAK_GBS}}


def streaming_leg(torch, q, synth, sd, steps: int = 512):
    """Expert-streaming decode: the 30-layer stack with every routed expert
    in pinned host memory and 16 device slots per layer.  Per layer:
    RMSNorm, router, routing to the host, shared gate/up while the pool
    copies the missing experts on a side stream, then the routed part."""
    st = synth.WORKLOADS["streaming_decode"]
    L, E, K, H, S = st.layers, st.n_experts, st.top_k, st.hidden, st.slots
    log(f"generating {L} layers into pinned host memory")
    lws = []
    host = None
    for l in range(L):
        lw = synth.make_layer(st, l)
        if host is None:
            blob = lw.layout.nbytes
            host = torch.empty((L * E, blob), dtype=torch.uint8, pin_memory=True)
        host[l * E:(l + 1) * E].copy_(torch.from_numpy(lw.blobs))
        lw.blobs = lw.blobs[:1]  # the host copy now lives in pinned memory
        lws.append(lw)
    arenas = [torch.zeros((S, blob), dtype=torch.uint8, device="cuda") for _ in range(L)]
    dls = [sd.DeviceLayer(lw, blobs=arenas[l]) for l, lw in enumerate(lws)]
    pool = q.Pool(L, E, S, blob, [host[i].data_ptr() for i in range(L * E)],
                  [a.data_ptr() for a in arenas])
    maps = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in range(L)]
    X = torch.from_numpy(synth.make_tokens(st, steps, stream=5).view(np.int16)).cuda()
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ws = dls[0].layer.new_workspace(1)
    rws = torch.zeros(q.qmoe_router_workspace_bytes(E, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    idx_h = torch.empty(K, dtype=torch.int32, pin_memory=True)
    h = torch.empty(H, dtype=torch.int16, device="cuda")
    buf = [torch.empty(H, dtype=torch.int16, device="cuda") for _ in range(2)]
    ev_idx = torch.cuda.Event()
    ready = torch.cuda.Event()
    ready.record(copy)

    def token(t):
        x = X[t]
        for l, dl in enumerate(dls):
            Ly = dl.layer
            q.qmoe_rmsnorm(x, dl.gamma, 1e-6, 1, H, h)
            q.qmoe_router_topk(Ly.router, dl.logit_bias, h, 1, K, idx, w, None, rws)
            idx_h.copy_(idx, non_blocking=True)
            ev_idx.record(compute)
            q.qmoe_expert_ffn_shared(Ly, h, ws)
            ev_idx.synchronize()
            s = pool.acquire(l, idx_h.data_ptr(), K, maps[l], copy, ready.cuda_event)
            compute.wait_event(ready)
            out = buf[l & 1]
            q.qmoe_expert_ffn_routed(Ly, h, idx, w, maps[l], x, out, ws)
            x = out
        return s

    t0 = time.perf_counter()
    last = None
    for t in range(steps):
        s = token(t)
        if t == steps // 2:
            torch.cuda.synchronize()
            last = (time.perf_counter(), s.hits, s.misses, s.h2d_bytes)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    s = pool.stats()
    hits, misses = s.hits, s.misses
    wh = (s.hits - last[1]) / max(1, (s.hits - last[1]) + (s.misses - last[2]))
    warm_s = t1 - last[0]
    warm_tokens = steps - steps // 2 - 1
    res = {"metric": "expert-streaming stack decode tokens/s (pinned host experts, 16-slot LFU)",
           "value": steps / (t1 - t0), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
           "higher_is_better": True, "dtype": "f32", "data": "synthetic (seeded)",
           "config": {"workload": "30-layer MoE decode stack, batch 1, hidden 2816, 128 experts "
                                  "per layer in pinned host memory, 16 device slots per layer, "
                                  "Zipf(1.1) log-prior on the router logits"},
           "hit_rate": hits / (hits + misses), "hit_rate_second_half": wh,
           "h2d_bytes": s.h2d_bytes,
           "h2d_GBps": s.h2d_bytes / (t1 - t0) / 1e9,
           "tokens_per_s_second_half": warm_tokens / warm_s,
           "h2d_GBps_second_half": (s.h2d_bytes - last[3]) / warm_s / 1e9}
    pool.close()
    log(f"streaming: {res['value']:.1f} tokens/s, hit rate {res['hit_rate']:.3f}, "
        f"H2D {res['h2d_GBps']:.1f} GB/s")
    return res


def gemv_leg(torch, q, sptr, rows: int = 65536, cols: int = 2816, copies: int = 8,
             iters: int = 400):
    """The standalone 4-bit affine GEMV (qmoe_gemv_affine4) on a large matrix
    of the decode width (rows x cols, seeded codes, scales ~U(0.005, 0.02),
    biases -8*scale), cycling through copies that together exceed the 256 MB
    MALL.  Three untimed rounds of `iters` back-to-back launches, then HIP
    events around each of three such rounds (the median is reported); algorithmic bytes
    = codes + fp16 scales and biases + x + y.  Also a plain 512 MiB device
    copy, for context (bytes read + written per second)."""
    import ctypes

    g = torch.Generator(device="cuda")
    g.manual_seed(20260)
    mats = []
    for _ in range(copies):
        qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows, cols // 8), dtype=torch.int32,
                           device="cuda", generator=g)
        sc = (torch.rand(rows, cols // 64, device="cuda", generator=g) * 0.015 + 0.005).half()
        bi = (-8.0 * sc.float()).half()
        mats.append(q.QTensor(qw, sc.view(torch.int16), bi.view(torch.int16), rows, cols, 4))
    x = torch.randn(cols, device="cuda", generator=g).bfloat16().view(torch.int16)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    nbytes = rows * cols // 2 + rows * (cols // 64) * 4 + cols * 2 + rows * 4
    fn = q.lib().qmoe_gemv_affine4
    cts = [ctypes.byref(m.c()) for m in mats]
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launches():
        for i in range(iters):
            rc = fn(cts[i % copies], x.data_ptr(), y.data_ptr(), sptr)
            if rc:
                raise q.QmoeError("qmoe_gemv_affine4", rc)

    # the first few hundred launches over freshly allocated copies run up to
    # ~12% slower: three untimed rounds, then three timed rounds (median
    # reported)
    for _ in range(3):
        launches()
    reps = []
    for _ in range(3):
        torch.cuda.synchronize()
        e0.record(stream)
        launches()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e3 / iters)
    us = sorted(reps)[1]
    del mats
    src = torch.ones(COPY_BYTES // 8, dtype=torch.int32, device="cuda")  # 512 MiB: beyond the MALL
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"gemv {rows}x{cols}: {us:.2f} us, {gbs:.0f} GB/s; device copy {copy_gbs:.0f} GB/s")
    return {"workload": f"4-bit affine g64 GEMV, {rows} x {cols} (decode width), "
                        f"{copies} copies cycled",
            "entry": "qmoe_gemv_affine4", "us_per_gemv": us,
            "us_per_gemv_rounds": [round(r, 3) for r in reps], "algorithmic_bytes": nbytes,
            "achieved_GBps": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "device_copy_GBps_read_plus_write": copy_gbs}


def copy_calibration(torch, reps: int = 3):
    """A plain device copy of COPY_BYTES, for scaling the byte counters."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} x {COPY_BYTES} bytes read and written")


if __name__ == "__main__":
    main()
