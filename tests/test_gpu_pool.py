"""GPU check of the host-resident expert pool: a stack streamed through
16 device slots per layer (pinned host blobs, copies on a side stream
overlapping the shared expert) gives bit-identical outputs to the same
kernels on resident weights; the pool's trace equals the oracle's LFU
replay; outputs match the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import (bf16_to_f64, log, rel_l2, routing_bound, routing_certified,
                           to_u16)

pytestmark = pytest.mark.gpu


def _flow(torch, q, WL, dls, X, pool=None, slot_maps=None, trace=None, tier=None):
    """RMSNorm -> router -> shared gate/up -> (pool acquire, from the file
    tier if one is given) -> routed part, layer after layer, token after
    token.  Returns every layer's output."""
    H, K = WL.hidden, WL.top_k
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ws = dls[0].layer.new_workspace(1)
    rws = torch.zeros(q.qmoe_router_workspace_bytes(WL.n_experts, 1), dtype=torch.uint8,
                      device="cuda")
    idx_d = torch.empty(K, dtype=torch.int32, device="cuda")
    w_d = torch.empty(K, dtype=torch.float32, device="cuda")
    idx_h = torch.empty(K, dtype=torch.int32, pin_memory=True)
    ev_idx = torch.cuda.Event()
    ready = torch.cuda.Event()
    ready.record(copy)  # create the event before handing it to the library
    outs = []
    for t in range(X.shape[0]):
        x = torch.from_numpy(np.ascontiguousarray(X[t]).view(np.int16)).cuda()
        per = []
        for l, dl in enumerate(dls):
            L = dl.layer
            h = torch.empty(H, dtype=torch.int16, device="cuda")
            q.qmoe_rmsnorm(x, dl.gamma, 1e-6, 1, H, h)
            q.qmoe_router_topk(L.router, dl.logit_bias, h, 1, K, idx_d, w_d, None, rws)
            smap = None
            if pool is not None:
                idx_h.copy_(idx_d, non_blocking=True)
                ev_idx.record(compute)
            q.qmoe_expert_ffn_shared(L, h, ws)
            if pool is not None:
                ev_idx.synchronize()
                smap = slot_maps[l]
                if tier is None:
                    st = pool.acquire(l, idx_h.data_ptr(), K, smap, copy, ready.cuda_event)
                else:
                    st = pool.acquire_file(tier, l, idx_h.data_ptr(), K, smap, copy,
                                           ready.cuda_event)
                compute.wait_event(ready)
            out = torch.empty(H, dtype=torch.int16, device="cuda")
            q.qmoe_expert_ffn_routed(L, h, idx_d, w_d, smap, x, out, ws)
            if trace is not None:
                torch.cuda.synchronize()
                trace.append((l, idx_d.cpu().numpy().copy(), w_d.cpu().numpy().copy(),
                              None if smap is None else smap.cpu().numpy().copy(),
                              None if pool is None else (st.last_hits, st.last_misses)))
            per.append(to_u16(out))
            x = out
        outs.append(per)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name", ["tiny_streaming_decode", "streaming_decode_3l"])
def test_pool_streaming_equals_resident_and_oracle(name):
    """Small shapes (3 layers, 12 steps) and the streaming workload's own
    shapes (its first 3 layers, 16 steps, hidden 2816, 128 experts)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import bit_quantized_gemv_amd as q

    assert torch.cuda.is_available()
    WL = synth.WORKLOADS[name]
    log(f"{name}: drawing {WL.layers} layers")
    layers = [synth.make_layer(WL, l) for l in range(WL.layers)]

    E, K, S = WL.n_experts, WL.top_k, WL.slots
    blob = layers[0].layout.nbytes
    X = synth.make_tokens(WL, WL.tokens, stream=91)
    prior = [synth.zipf_prior(WL, l) for l in range(WL.layers)]

    # resident: every expert on the device
    res_dls = [synth.device.DeviceLayer(lw, logit_bias=prior[l]) for l, lw in enumerate(layers)]
    res_trace = []
    ref = _flow(torch, q, WL, res_dls, X, trace=res_trace)

    # streamed: pinned host blobs, 16 device slots per layer
    host = torch.empty((WL.layers * E, blob), dtype=torch.uint8, pin_memory=True)
    for l, lw in enumerate(layers):
        host[l * E:(l + 1) * E].copy_(torch.from_numpy(lw.blobs))
    arenas = [torch.zeros((S, blob), dtype=torch.uint8, device="cuda") for _ in layers]
    pool = q.Pool(WL.layers, E, S, blob,
                  [host[i].data_ptr() for i in range(WL.layers * E)],
                  [a.data_ptr() for a in arenas])
    slot_maps = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in layers]
    str_dls = [synth.device.DeviceLayer(lw, logit_bias=prior[l], blobs=arenas[l])
               for l, lw in enumerate(layers)]
    trace = []
    got = _flow(torch, q, WL, str_dls, X, pool=pool, slot_maps=slot_maps, trace=trace)

    # 1. bit-identical to the resident run (same kernels, other addresses)
    for t in range(len(X)):
        for l in range(WL.layers):
            assert np.array_equal(got[t][l], ref[t][l]), (t, l)

    # 2. the pool's trace equals the oracle's LFU replay of the same needs
    st = pool.stats()
    total_hits = 0
    for l in range(WL.layers):
        rows = [tr for tr in trace if tr[0] == l]
        need = np.stack([r[1] for r in rows])
        rep = oracle.lfu_replay(need, E, S)
        for step, r in enumerate(rows):
            _, idx, _, smap, (hits, misses) = r
            assert hits == int(rep["hit"][step].sum()), (l, step)
            assert list(smap[idx]) == list(rep["slot"][step]), (l, step)
        total_hits += rep["hits"]
    assert st.hits == total_hits and st.hits + st.misses == WL.tokens * WL.layers * K
    assert st.h2d_bytes == st.misses * blob
    log(f"  pool hit rate {st.hits / (st.hits + st.misses):.3f}, "
        f"{st.h2d_bytes / 1e6:.1f} MB host->device")

    # 3. every layer against the oracle on the device's own layer input
    orcs = [oracle.OracleLayer(lw, logit_bias=prior[l]) for l, lw in enumerate(layers)]

    def one(job):
        t, l = job
        lw, ol = layers[l], orcs[l]
        xin = X[t] if l == 0 else got[t][l - 1]
        r = ol.forward(xin, residual=True)
        _, gidx, gw, _, _ = trace[t * WL.layers + l]
        flip = list(gidx) != list(r["idx"])
        if flip:
            lg = r["logits"]
            B = routing_bound(lw.router, xin, lg, gamma=lw.gamma)
            assert routing_certified(B, lg, gidx), (t, l, "routing flip not certified")
            r = ol.forward(xin, residual=True, force_idx=gidx, force_w=gw.astype(np.float64))
        return rel_l2(bf16_to_f64(got[t][l]), bf16_to_f64(r["out"])), flip

    jobs = [(t, l) for t in range(len(X)) for l in range(WL.layers)]
    with ThreadPoolExecutor(max_workers=16) as ex:
        res = list(ex.map(one, jobs))
    worst = max(e for e, _ in res)
    log(f"  worst layer relL2 vs oracle {worst:.2e}, certified near-tie flips "
        f"{sum(f for _, f in res)}")
    assert worst <= 2e-3
    pool.close()


def test_file_tier_streaming_equals_resident(tmp_path):
    """The routed experts read from an expert-major file (4 KiB-aligned
    strides, 8 reader threads) into the 16-slot pool: bit-identical to the
    resident run, one read per miss, and the same hits and misses as the
    pinned-host pool's LFU.  O_DIRECT when the file system takes it."""
    import torch

    import bit_quantized_gemv_amd as q

    WL = synth.WORKLOADS["tiny_streaming_decode"]
    layers = [synth.make_layer(WL, l) for l in range(WL.layers)]
    E, K, S = WL.n_experts, WL.top_k, WL.slots
    blob = layers[0].layout.nbytes
    stride = -(-blob // 4096) * 4096
    path = tmp_path / "experts.bin"
    with open(path, "wb") as f:
        for lw in layers:
            for e in range(E):
                f.write(lw.blobs[e].tobytes())
                f.write(b"\0" * (stride - blob))
    X = synth.make_tokens(WL, WL.tokens, stream=93)
    prior = [synth.zipf_prior(WL, l) for l in range(WL.layers)]
    res_dls = [synth.device.DeviceLayer(lw, logit_bias=prior[l]) for l, lw in enumerate(layers)]
    ref = _flow(torch, q, WL, res_dls, X)
    arenas = [torch.zeros((S, blob), dtype=torch.uint8, device="cuda") for _ in layers]
    dls = [synth.device.DeviceLayer(lw, logit_bias=prior[l], blobs=arenas[l])
           for l, lw in enumerate(layers)]
    for direct in (True, False):
        try:
            tier = q.FileTier(str(path), WL.layers, E, blob, stride, threads=8, direct=direct)
        except q.QmoeError:
            assert direct, "buffered open must work"
            log("file system refuses O_DIRECT: buffered reads only")
            continue
        pool = q.Pool(WL.layers, E, S, blob, None, [a.data_ptr() for a in arenas])
        maps = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in layers]
        try:
            got = _flow(torch, q, WL, dls, X, pool=pool, slot_maps=maps, tier=tier)
        except q.QmoeError:
            raise AssertionError(f"read failed, errno {tier.stats().last_errno}")
        for t in range(len(X)):
            for l in range(WL.layers):
                assert np.array_equal(got[t][l], ref[t][l]), (direct, t, l)
        ps, fs = pool.stats(), tier.stats()
        assert fs.reads == ps.misses and fs.read_bytes == ps.misses * stride
        assert ps.hits + ps.misses == len(X) * WL.layers * K
        log(f"file tier (direct={direct}): {ps.misses} reads, "
            f"{fs.read_bytes / max(1, fs.read_ns) :.2f} GB/s in reads")
        tier.close()
        pool.close()
