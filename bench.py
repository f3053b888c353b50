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
the standalone 4-bit GEMV on a large matrix of the decode width (MLX and
repacked tiled layouts), token sampling, decode attention over the FP16
cache of 30 layers, the 30-layer stack, the expert pool (streaming from
pinned host memory) and the file-backed expert tier are further
reported-only legs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-prefill] [--no-gemv] [--no-sampling] [--no-attention]
                    [--no-stack] [--no-streaming] [--no-file-tier]
                    [--copy-calibration]
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
                  for f in ("qmoe_decode.hip", "qmoe_common.h", "qmoe_topk.h")]


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
    """Threads the oracle may use: every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lw, X, Xp=None, prior=None):
    """The fp64 oracle (as it stands) on a bounded sample of tokens of the
    same layer: one thread over a few tokens, then every host core (one
    token per thread) over a larger sample; with Xp, also one whole prefill
    chunk (the chunk's tokens through the layer with the Zipf log-prior on
    the router logits, one token per thread)."""
    import oracle

    L = oracle.OracleLayer(lw)
    cores = host_threads()
    n1 = 6
    t0 = time.perf_counter()
    for t in range(n1):
        L.forward(X[t])
    one = n1 / (time.perf_counter() - t0)
    n = min(X.shape[0], max(2 * cores, 32))
    n = max(cores, n - n % cores) if n >= cores else n
    threads = min(cores, n)
    t0 = time.perf_counter()
    oracle.forward_many(L, X[:n], threads=threads)
    dt = time.perf_counter() - t0
    res = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "value_1thread": one, "cpu_model": cpu_model(), "host_cores": cores,
           "sample": f"{n} decode tokens of one layer (same shapes and weights) on {threads} "
                     f"threads, one token per thread; 1-thread figure over {n1} tokens; "
                     f"fp64 scalar C oracle"}
    if Xp is not None:
        P = oracle.OracleLayer(lw, logit_bias=prior)
        t0 = time.perf_counter()
        oracle.forward_many(P, Xp, threads=cores)
        dt = time.perf_counter() - t0
        res["prefill"] = {"tokens_per_s": Xp.shape[0] / dt, "us_per_chunk": dt * 1e6,
                          "cores": min(cores, Xp.shape[0]),
                          "sample": f"one {Xp.shape[0]}-token prefill chunk (the prefill leg's "
                                    f"tokens and Zipf(1.1) log-prior) on {min(cores, Xp.shape[0])} "
                                    f"threads, one token per thread"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-gemv", action="store_true", help="skip the standalone GEMV leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the 30-layer stack leg")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the expert-streaming leg (30 layers, pinned host experts, "
                         "16 device slots per layer)")
    ap.add_argument("--no-sampling", action="store_true", help="skip the token sampling leg")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the decode attention leg (30 layers at a 4,096-token context)")
    ap.add_argument("--no-file-tier", action="store_true",
                    help="skip the file-backed expert tier leg (8 layers read from a file)")
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

    # One untimed pass over every weight copy and every token, whatever
    # --warmup says (the first launches on freshly allocated copies run
    # slower), then the requested warmup steps.
    log("warm pass over every weight copy and token, then warmup")
    n_warm = max(COPIES, N_TOKENS) + args.warmup
    for i in range(n_warm):
        step(i)
    torch.cuda.synchronize()
    if q.qmoe_workspace_status(ws) != 0:
        raise SystemExit("device wait failure during warmup")

    # timed region: exactly K steps, in groups of up to SAMPLE consecutive
    # launches.  The first launch of a group records a HIP event at its
    # kernel's start and the last one at its kernel's end (the dispatches'
    # own timestamps, on the launch stream); the launches in between are
    # plain.  Sum of group spans over K is the average launch duration with
    # the kernels running back to back, as a caller's would.  (A launch that
    # records events costs the host about 29 us, more than the kernel takes:
    # with events on every launch the loop would be host-bound.)  The
    # three-launch variant is bracketed by event records every step.
    sample = 1 if args.phased else SAMPLE
    K = max(1, args.steps)
    groups = [(g0, min(sample, K - g0)) for g0 in range(0, K, sample)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(groups))]
    for e in ev:  # create the underlying hipEvents before the timed region
        e.record(stream)
    evh = [e.cuda_event for e in ev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.phased:
        for i in range(K):
            ev[2 * i].record(stream)
            step(n_warm + i)
            ev[2 * i + 1].record(stream)
    else:
        for n, (g0, gs) in enumerate(groups):
            for r in range(gs):
                e0 = evh[2 * n] if r == 0 else None
                e1 = evh[2 * n + 1] if r == gs - 1 else None
                if e0 or e1:
                    timed_step(n_warm + g0 + r, e0, e1)
                else:
                    plain_step(n_warm + g0 + r)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code = q.qmoe_workspace_status(ws)
    if code != 0:
        raise SystemExit(f"device wait failure (code {code})")
    spans = np.array([ev[2 * n].elapsed_time(ev[2 * n + 1]) for n in range(len(groups))])
    sizes = np.array([gs for _, gs in groups], dtype=np.float64)
    kern_us = float(spans.sum() / sizes.sum() * 1e3)
    kern_med_us = float(np.median(spans / sizes) * 1e3)
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
                     "launch_us_basis": f"HIP events spanning up to {sample} consecutive "
                                        f"launches, {len(groups)} groups over the {K} timed "
                                        f"steps, after {n_warm} untimed steps",},
    }
    if not args.no_prefill:
        res["prefill"] = prefill_leg(torch, q, synth, sd, lw, layers, wl, sptr)
    if not args.no_gemv:
        res["gemv"] = gemv_leg(torch, q, sptr)
    if not args.no_sampling:
        res["sampling"] = sampling_leg(torch, q, sptr)
    del layers, cstructs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_stack:
        res["stack"] = stack_leg(torch, q, synth, sd, sptr)
    if not args.no_streaming:
        res["streaming"] = streaming_leg(torch, q, synth, sd)
    if not args.no_file_tier:
        # reported only, and it depends on the host's storage: a failure is
        # recorded in its entry instead of ending the run
        try:
            res["file_tier"] = file_tier_leg(torch, q, synth, sd)
        except Exception as exc:  # noqa: BLE001
            log(f"file tier leg failed: {exc!r}")
            res["file_tier"] = {"error": repr(exc)}
    if not args.no_attention:
        # after the stack legs: run before them, its HIP graphs and side
        # streams left the cooperative one-launch stack 13% slower (measured)
        res["attention"] = attention_leg(torch, q, synth, sptr)
    if args.copy_calibration:
        copy_calibration(torch)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        pw = synth.WORKLOADS["prefill128"]
        res["cpu_baseline"] = cpu_baseline(lw, X, synth.make_tokens(pw, PF_TOKENS, stream=2),
                                           synth.zipf_prior(pw, 0))
    torch.cuda.synchronize()
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
    # release the stack's device objects (table, workspaces, events) before
    # the next leg and before the interpreter exits
    del stk, ev, ev1, evh, cl, dls, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
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
    copies the missing experts on a side stream, then the routed part.

    Run three ways over the same tokens: all experts resident (no copies),
    streamed with the copies overlapping the shared expert, and streamed
    with every layer's copies finished before its shared expert starts (a
    fresh pool: the same LFU decisions).  The overlap achieved is the part
    of the copy time the overlapped run hides:
    (t_serial - t_overlap) / (t_serial - t_resident)."""
    st = synth.WORKLOADS["streaming_decode"]
    L, E, K, H, S = st.layers, st.n_experts, st.top_k, st.hidden, st.slots
    log(f"streaming: generating {L} layers into pinned host memory")
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
    X = torch.from_numpy(synth.make_tokens(st, steps, stream=5).view(np.int16)).cuda()
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    rws = torch.zeros(q.qmoe_router_workspace_bytes(E, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    idx_h = torch.empty(K, dtype=torch.int32, pin_memory=True)
    h = torch.empty(H, dtype=torch.int16, device="cuda")
    buf = [torch.empty(H, dtype=torch.int16, device="cuda") for _ in range(2)]
    ev_idx = torch.cuda.Event()
    ready = torch.cuda.Event()
    ready.record(copy)

    def run(dls, pool, serial):
        ws = dls[0].layer.new_workspace(1)
        maps = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in range(L)]
        half = None

        def token(t):
            x = X[t]
            for l, dl in enumerate(dls):
                Ly = dl.layer
                q.qmoe_rmsnorm(x, dl.gamma, 1e-6, 1, H, h)
                q.qmoe_router_topk(Ly.router, dl.logit_bias, h, 1, K, idx, w, None, rws)
                smap = None
                if pool is not None:
                    idx_h.copy_(idx, non_blocking=True)
                    ev_idx.record(compute)
                    if serial:
                        ev_idx.synchronize()
                        pool.acquire(l, idx_h.data_ptr(), K, maps[l], copy, ready.cuda_event)
                        compute.wait_event(ready)
                q.qmoe_expert_ffn_shared(Ly, h, ws)
                if pool is not None:
                    if not serial:
                        ev_idx.synchronize()
                        pool.acquire(l, idx_h.data_ptr(), K, maps[l], copy, ready.cuda_event)
                        compute.wait_event(ready)
                    smap = maps[l]
                out = buf[l & 1]
                q.qmoe_expert_ffn_routed(Ly, h, idx, w, smap, x, out, ws)
                x = out

        t0 = time.perf_counter()
        for t in range(steps):
            token(t)
            if t == steps // 2 - 1:
                torch.cuda.synchronize()
                s = pool.stats() if pool is not None else None
                half = (time.perf_counter(), s)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if q.qmoe_workspace_status(ws) != 0:
            raise SystemExit("device wait failure in the streaming leg")
        return t0, half, t1

    # resident: every expert of every layer on the device
    res_dls = []
    for l, lw in enumerate(lws):
        blobs = host[l * E:(l + 1) * E].to("cuda")
        res_dls.append(sd.DeviceLayer(lw, blobs=blobs))
    t0, _, t1 = run(res_dls, None, False)
    t_res = t1 - t0
    del res_dls
    torch.cuda.empty_cache()

    arenas = [torch.zeros((S, blob), dtype=torch.uint8, device="cuda") for _ in range(L)]
    dls = [sd.DeviceLayer(lw, blobs=arenas[l]) for l, lw in enumerate(lws)]
    hp = [host[i].data_ptr() for i in range(L * E)]
    ap = [a.data_ptr() for a in arenas]
    out = {}
    for serial in (False, True):
        pool = q.Pool(L, E, S, blob, hp, ap)
        t0, (th, sh), t1 = run(dls, pool, serial)
        s = pool.stats()
        pool.close()
        out[serial] = (t0, th, sh, t1, s)
    t0, th, sh, t1, s = out[False]
    t_ovl = t1 - t0
    t_ser = out[True][3] - out[True][0]
    warm_tokens = steps - steps // 2
    warm_s = t1 - th
    whits, wmiss = s.hits - sh.hits, s.misses - sh.misses
    res = {"workload": "30-layer MoE decode stack, batch 1, hidden 2816, 128 experts per layer "
                       "in pinned host memory, 16 device slots per layer (LFU), Zipf(1.1) "
                       "log-prior on the router logits",
           "steps": steps, "tokens_per_s": steps / t_ovl,
           "tokens_per_s_warm": warm_tokens / warm_s,
           "hit_rate": s.hits / (s.hits + s.misses),
           "hit_rate_warm": whits / max(1, whits + wmiss),
           "h2d_bytes": s.h2d_bytes,
           "h2d_GBps": s.h2d_bytes / t_ovl / 1e9,
           "h2d_GBps_warm": (s.h2d_bytes - sh.h2d_bytes) / warm_s / 1e9,
           "tokens_per_s_resident": steps / t_res,
           "tokens_per_s_serialized_copies": steps / t_ser,
           "overlap_achieved": (t_ser - t_ovl) / max(1e-9, t_ser - t_res),
           "warm": f"second half of the run ({warm_tokens} tokens)",
           "overlap_basis": "(t_serialized - t_overlapped) / (t_serialized - t_resident), "
                            "same tokens and LFU decisions"}
    res["h2d_ceiling_GBps"] = h2d_ceiling(torch, host.view(-1), blob)
    log(f"streaming: {res['tokens_per_s']:.1f} tokens/s, hit rate {res['hit_rate']:.3f} "
        f"(warm {res['hit_rate_warm']:.3f}), H2D {res['h2d_GBps']:.1f} GB/s, overlap "
        f"{res['overlap_achieved']:.2f} (resident {res['tokens_per_s_resident']:.0f}, "
        f"serialized {res['tokens_per_s_serialized_copies']:.0f} tokens/s); pinned-copy "
        f"ceiling {res['h2d_ceiling_GBps']}")
    del dls, arenas, host
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def h2d_ceiling(torch, host, blob: int, n: int = 96, reps: int = 3):
    """Practical host -> device ceiling: pinned copies of one expert blob
    (the pool's unit), on one stream and as two halves on two streams (as
    the pool issues them), and 64 MB copies; best of `reps` rounds of n
    copies, wall clock."""
    big = 64 << 20
    dev = torch.empty(max(n * blob, 8 * big), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(2)]

    def rate(size, count, lanes):
        best = 0.0
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(count):
                o = i * size
                if lanes == 1:
                    with torch.cuda.stream(streams[0]):
                        dev[o:o + size].copy_(host[o:o + size], non_blocking=True)
                else:
                    h = size // 2
                    for k, (a, b) in enumerate(((o, o + h), (o + h, o + size))):
                        with torch.cuda.stream(streams[k]):
                            dev[a:b].copy_(host[a:b], non_blocking=True)
            torch.cuda.synchronize()
            best = max(best, count * size / (time.perf_counter() - t0) / 1e9)
        return round(best, 1)

    out = {"blob_one_stream": rate(blob, n, 1), "blob_halves_two_streams": rate(blob, n, 2),
           "64MB_one_stream": rate(big, 8, 1)}
    del dev
    return out


def gemv_leg(torch, q, sptr, rows: int = 65536, cols: int = 2816, copies: int = 8,
             iters: int = 400):
    """The standalone 4-bit affine GEMV on a large matrix of the decode width
    (rows x cols, seeded codes, scales ~U(0.005, 0.02), biases -8*scale),
    cycling through copies that together exceed the 256 MB MALL: first on the
    MLX layout (qmoe_gemv_affine4), then on the same matrices repacked
    offline into the tiled layout (qmoe_repack_tiled4 on the host, then
    qmoe_gemv_tiled4), which is the leg's headline.  Each: three untimed
    rounds of `iters` back-to-back launches, then HIP events around each of
    three such rounds (the median is reported); algorithmic bytes = codes +
    fp16 scales and biases + x + y (the same for both layouts).  Also a plain
    512 MiB device copy, for context (bytes read + written per second)."""
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
    # the same matrices repacked offline into the tiled layout
    # (qmoe_repack_tiled4 on the host), same timing
    tiled = []
    for m in mats:
        qh = m.q.cpu().numpy().view(np.uint8)
        t = q.qmoe_repack_tiled4(qh, m.scales.cpu().numpy().view(np.uint16),
                                 m.biases.cpu().numpy().view(np.uint16), rows, cols)
        tiled.append(torch.from_numpy(t).cuda())
    del mats
    fnt = q.lib().qmoe_gemv_tiled4

    def launches_tiled():
        for i in range(iters):
            rc = fnt(tiled[i % copies].data_ptr(), rows, cols, x.data_ptr(), y.data_ptr(), 0, sptr)
            if rc:
                raise q.QmoeError("qmoe_gemv_tiled4", rc)

    for _ in range(3):
        launches_tiled()
    reps_t = []
    for _ in range(3):
        torch.cuda.synchronize()
        e0.record(stream)
        launches_tiled()
        e1.record(stream)
        torch.cuda.synchronize()
        reps_t.append(e0.elapsed_time(e1) * 1e3 / iters)
    us_t = sorted(reps_t)[1]
    del tiled
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
    gbs_t = nbytes / (us_t * 1e-6) / 1e9
    log(f"gemv {rows}x{cols}: {us:.2f} us, {gbs:.0f} GB/s; tiled layout {us_t:.2f} us, "
        f"{gbs_t:.0f} GB/s; device copy {copy_gbs:.0f} GB/s")
    return {"workload": f"4-bit affine g64 GEMV, {rows} x {cols} (decode width), "
                        f"{copies} copies cycled",
            "entry": "qmoe_gemv_tiled4 (matrices repacked offline by qmoe_repack_tiled4: "
                     "the same bytes, 1 KiB per wave load; output bit-identical to "
                     "qmoe_gemv_affine4)",
            "us_per_gemv": us_t, "us_per_gemv_rounds": [round(r, 3) for r in reps_t],
            "algorithmic_bytes": nbytes, "achieved_GBps": gbs_t,
            "frac_of_hbm_peak": gbs_t / HBM_PEAK_GBS,
            "mlx_layout": {"entry": "qmoe_gemv_affine4", "us_per_gemv": us,
                           "us_per_gemv_rounds": [round(r, 3) for r in reps],
                           "achieved_GBps": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS},
            "device_copy_GBps_read_plus_write": copy_gbs}


def sampling_leg(torch, q, sptr, V: int = 262144, K: int = 64, T: float = 0.2, P: float = 0.95,
                 n_logits: int = 64, iters: int = 2000):
    """Token sampling (qmoe_sample) with the pages' defaults (temperature 0.2,
    top-K 64, top-P 0.95) over a vocabulary of V logits (a reading: the
    pages give no vocabulary size), n_logits seeded N(0, 2) logit vectors
    resident on the GPU, seeded uniform draws.  HIP events around `iters`
    back-to-back calls (two launches each), after as many untimed ones."""
    import ctypes

    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    lg = torch.randn(n_logits, V, device="cuda", generator=g) * 2.0
    us_draw = np.random.default_rng(78).random(iters)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(q.qmoe_sample_workspace_bytes(V, K), dtype=torch.uint8, device="cuda")
    fn = q.lib().qmoe_sample
    wsb = ws.numel()

    def calls():
        for i in range(iters):
            rc = fn(lg[i % n_logits].data_ptr(), V, ctypes.c_float(T), K, ctypes.c_float(P),
                    ctypes.c_float(float(us_draw[i])), tok.data_ptr(), None, ws.data_ptr(), wsb,
                    sptr)
            if rc:
                raise q.QmoeError("qmoe_sample", rc)

    calls()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    calls()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    log(f"sampling V={V}: {us:.2f} us per token")
    return {"workload": f"token sampling, vocabulary {V} (fp32 logits), temperature {T}, "
                        f"top-K {K}, top-P {P}",
            "entry": "qmoe_sample (two launches)", "us_per_token": us,
            "tokens_per_s": 1e6 / us, "logit_bytes": V * 4,
            "achieved_GBps": V * 4 / (us * 1e-6) / 1e9}


def attention_leg(torch, q, synth, sptr, iters: int = 50):
    """Decode attention (qmoe_attn_decode) of a 30-layer stack at a full
    4,096-token context: 25 sliding-window layers (1,024-slot circular
    stores) and 5 full-attention layers (4,096-slot linear stores, every
    sixth layer), 16 query heads over 8 key/value heads of width 256 (the
    pages give the layer split, the FP16 cache and the context; the head
    shapes are a stated reading).  One step is the token at position 4,095
    through the 30 layers, each with its own seeded cache resident in HBM
    (378 MB together, more than the 256 MB Infinity Cache).

    A call is one short launch, shorter than the host takes to issue it, so the calls are captured into HIP graphs and the graphs
    replayed between HIP events: the 30-layer token, and for the per-layer
    figures 12 distinct full layers (402 MB) and 48 distinct sliding layers
    (403 MB), so that no replay finds its cache rows in the Infinity Cache."""
    import ctypes

    aw = synth.ATTN_WORKLOADS["attn30_decode"]
    Hq, Hkv, D = aw.n_heads, aw.n_kv_heads, aw.head_dim
    pos = aw.context - 1
    fn = q.lib().qmoe_attn_decode
    out = torch.empty(Hq, D, dtype=torch.int16, device="cuda")

    def make(full, layer):
        S = aw.context if full else aw.window
        qv, kv, vv, kc, vc = synth.attn_inputs(aw, S, layer=layer)
        shape = q.AttnShape(Hq, Hkv, D, S, 0 if full else 1, aw.rope_base, 1.0 / np.sqrt(D))
        t = [torch.from_numpy(a).cuda() for a in (qv, kv, vv)]
        t += [torch.from_numpy(a.view(np.int16)).cuda() for a in (kc, vc)]
        ws = torch.zeros(q.qmoe_attn_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
        return (shape, t, ws)

    def argv(layer):
        shape, t, ws = layer
        return (ctypes.byref(shape), t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), pos,
                t[3].data_ptr(), t[4].data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel())

    def graph_us(layers):
        argl = [argv(L) for L in layers]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sp = side.cuda_stream
            for a in argl:  # eager warm-up on the capture stream
                rc = fn(*a, sp)
                if rc:
                    raise q.QmoeError("qmoe_attn_decode", rc)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            sp = torch.cuda.current_stream().cuda_stream
            for a in argl:
                rc = fn(*a, sp)
                if rc:
                    raise q.QmoeError("qmoe_attn_decode", rc)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(iters):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / iters

    log("attention: 30 layers, 12 full and 48 sliding caches")
    stack = [make(l % 6 == 5, l) for l in range(aw.sliding_layers + aw.full_layers)]
    us_token = graph_us(stack)
    del stack
    fulls = [make(True, 100 + i) for i in range(12)]
    us_full = graph_us(fulls) / len(fulls)
    del fulls
    slides = [make(False, 200 + i) for i in range(48)]
    us_slide = graph_us(slides) / len(slides)
    del slides
    torch.cuda.empty_cache()
    slot_bytes = Hkv * D * 2 * 2  # one token's key and value, fp16

    def algo(S):  # cache rows read, the new row written, q/k/v in, out
        return ((min(pos + 1, S) - 1) * slot_bytes + slot_bytes + (Hq + 2 * Hkv) * D * 4 +
                Hq * D * 2)

    gbs_full = algo(aw.context) / (us_full * 1e-6) / 1e9
    gbs_slide = algo(aw.window) / (us_slide * 1e-6) / 1e9
    log(f"attention: {us_token:.1f} us per token over 30 layers; full layer {us_full:.2f} us "
        f"({gbs_full:.0f} GB/s), sliding layer {us_slide:.2f} us ({gbs_slide:.0f} GB/s)")
    return {"workload": f"decode attention at position {pos} (a {aw.context}-token context), "
                        f"{aw.sliding_layers} sliding-window layers ({aw.window} slots, circular) + "
                        f"{aw.full_layers} full layers ({aw.context} slots, linear); Hq {Hq}, "
                        f"Hkv {Hkv}, D {D}, FP16 cache, RoPE base {aw.rope_base:g}",
            "entry": "qmoe_attn_decode (one launch per call), captured in HIP graphs",
            "us_per_token": us_token, "tokens_per_s": 1e6 / us_token,
            "us_full_layer": us_full, "us_sliding_layer": us_slide,
            "algorithmic_bytes_full_layer": algo(aw.context),
            "algorithmic_bytes_sliding_layer": algo(aw.window),
            "roofline_full_layer": {"bound": "hbm", "achieved": gbs_full, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": gbs_full / HBM_PEAK_GBS,
                                    "basis": "graph replays of 12 distinct full layers"},
            "achieved_GBps_sliding_layer": gbs_slide}


def file_tier_leg(torch, q, synth, sd, n_layers: int = 8, steps: int = 256, threads: int = 8):
    """The file-backed expert tier: the first n_layers layers of the
    streaming workload (hidden 2816, 128 experts, top-8, 16 device slots per
    layer, Zipf(1.1) prior), every routed expert in an expert-major file
    (4 KiB-aligned strides), read on a miss by `threads` workers into pinned
    staging, then copied to the layer's slots on a side stream while the
    shared expert runs.  O_DIRECT when the file system takes it; otherwise
    buffered reads after the file's pages are dropped from the page cache
    (posix_fadvise DONTNEED after fsync).  Storage GB/s = bytes read / time
    in reads; effective = bytes read / run time."""
    import tempfile

    st = synth.WORKLOADS["streaming_decode"]
    L, E, K, H, S = n_layers, st.n_experts, st.top_k, st.hidden, st.slots
    log(f"file tier: generating {L} layers")
    lws = [synth.make_layer(st, l) for l in range(L)]
    blob = lws[0].layout.nbytes
    stride = -(-blob // 4096) * 4096
    tmpdir = tempfile.mkdtemp(prefix="qmoe_ft_", dir=os.environ.get("TMPDIR") or "/tmp")
    path = os.path.join(tmpdir, "experts.bin")
    pad = np.zeros(stride - blob, dtype=np.uint8)
    with open(path, "wb") as f:
        for lw in lws:
            for e in range(E):
                f.write(lw.blobs[e].tobytes())
                f.write(pad.tobytes())
            lw.blobs = lw.blobs[:1]  # the file now holds the experts
        f.flush()
        os.fsync(f.fileno())
    fd = os.open(path, os.O_RDONLY)
    os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
    os.close(fd)
    direct = True
    try:
        tier = q.FileTier(path, L, E, blob, stride, threads=threads, direct=True)
    except q.QmoeError:
        direct = False
        tier = q.FileTier(path, L, E, blob, stride, threads=threads, direct=False)
    arenas = [torch.zeros((S, blob), dtype=torch.uint8, device="cuda") for _ in range(L)]
    dls = [sd.DeviceLayer(lw, blobs=arenas[l]) for l, lw in enumerate(lws)]
    pool = q.Pool(L, E, S, blob, None, [a.data_ptr() for a in arenas])
    maps = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in range(L)]
    X = torch.from_numpy(synth.make_tokens(st, steps, stream=6).view(np.int16)).cuda()
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    rws = torch.zeros(q.qmoe_router_workspace_bytes(E, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    idx_h = torch.empty(K, dtype=torch.int32, pin_memory=True)
    h = torch.empty(H, dtype=torch.int16, device="cuda")
    buf = [torch.empty(H, dtype=torch.int16, device="cuda") for _ in range(2)]
    ev_idx = torch.cuda.Event()
    ready = torch.cuda.Event()
    ready.record(copy)
    ws = dls[0].layer.new_workspace(1)
    half = None
    t0 = time.perf_counter()
    for t in range(steps):
        x = X[t]
        for l, dl in enumerate(dls):
            Ly = dl.layer
            q.qmoe_rmsnorm(x, dl.gamma, 1e-6, 1, H, h)
            q.qmoe_router_topk(Ly.router, dl.logit_bias, h, 1, K, idx, w, None, rws)
            idx_h.copy_(idx, non_blocking=True)
            ev_idx.record(compute)
            q.qmoe_expert_ffn_shared(Ly, h, ws)
            ev_idx.synchronize()
            pool.acquire_file(tier, l, idx_h.data_ptr(), K, maps[l], copy, ready.cuda_event)
            compute.wait_event(ready)
            out = buf[l & 1]
            q.qmoe_expert_ffn_routed(Ly, h, idx, w, maps[l], x, out, ws)
            x = out
        if t == steps // 2 - 1:
            torch.cuda.synchronize()
            half = (time.perf_counter(), pool.stats(), tier.stats())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if q.qmoe_workspace_status(ws) != 0:
        raise SystemExit("device wait failure in the file tier leg")
    ps, fs = pool.stats(), tier.stats()
    th, ph, fh = half
    whits, wmiss = ps.hits - ph.hits, ps.misses - ph.misses
    res = {"workload": f"first {L} layers of the streaming workload (hidden 2816, 128 experts, "
                       f"top-8, 16 device slots per layer, Zipf(1.1) prior), routed experts in "
                       f"an expert-major file of {L * E * stride / 1e9:.2f} GB",
           "steps": steps, "reader_threads": threads,
           "io": "O_DIRECT" if direct else "buffered, page cache dropped after writing",
           "tokens_per_s": steps / (t1 - t0), "layer_steps_per_s": steps * L / (t1 - t0),
           "hit_rate": ps.hits / (ps.hits + ps.misses),
           "hit_rate_warm": whits / max(1, whits + wmiss),
           "reads": fs.reads, "read_bytes": fs.read_bytes,
           "storage_GBps_in_reads": fs.read_bytes / max(1, fs.read_ns),
           "storage_GBps_in_reads_warm": (fs.read_bytes - fh.read_bytes) /
                                         max(1, fs.read_ns - fh.read_ns),
           "read_share_of_run": fs.read_ns * 1e-9 / (t1 - t0),
           "effective_GBps": fs.read_bytes / (t1 - t0) / 1e9}
    log(f"file tier ({res['io']}): {res['tokens_per_s']:.1f} tokens/s over {L} layers, hit rate "
        f"{res['hit_rate']:.3f}, {res['storage_GBps_in_reads']:.2f} GB/s in reads, reads "
        f"{100 * res['read_share_of_run']:.0f}% of the run")
    tier.close()
    pool.close()
    del dls, arenas
    os.remove(path)
    os.rmdir(tmpdir)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


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
