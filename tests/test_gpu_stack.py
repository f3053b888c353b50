"""GPU parity of the 30-layer decode stack (RMSNorm -> router top-8 ->
shared + routed FFN -> residual per layer, independent seeded layers)
against the fp64 oracle: teacher-forced per layer, then free-running.  The
one-launch stack decode must reproduce the one-layer launches bit for bit."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import bf16_to_f64, log, rel_l2, to_u16

pytestmark = pytest.mark.gpu

STACK = synth.WORKLOADS["stack30_decode"]
N_TOKENS = 3


@pytest.fixture(scope="module")
def stack():
    import torch

    assert torch.cuda.is_available()
    layers = []
    for l in range(STACK.layers):
        lw = synth.make_layer(STACK, l)
        layers.append((lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)))
    log(f"stack of {len(layers)} layers on the device")
    return layers


@pytest.fixture(scope="module")
def stack_kernel(stack):
    import bit_quantized_gemv_amd as q

    return q.Stack([dl.layer for _, _, dl in stack])


def _near_tie(lg, a, b):
    gap = max(abs(lg[i] - lg[j]) for i, j in zip(a, b))
    return gap <= 1e-3 * max(1.0, abs(lg).max())


def _run_gpu(torch, q, layers, x):
    """Layer by layer on the device; returns every layer's input and routing."""
    L0 = layers[0][2].layer
    ws = L0.new_workspace(1)
    cur = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    xs, idxs = [x], []
    for lw, ol, dl in layers:
        out = torch.empty(STACK.hidden, dtype=torch.int16, device="cuda")
        idx = torch.empty(STACK.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(STACK.top_k, dtype=torch.float32, device="cuda")
        q.qmoe_moe_decode(dl.layer, cur, None, True, out, idx, w, ws)
        cur = out
        xs.append(to_u16(out))
        idxs.append((idx.cpu().numpy(), w.cpu().numpy()))
    assert q.qmoe_workspace_status(ws) == 0
    return xs, idxs


def _run_stack_kernel(torch, stk, x):
    """The same token through the one-launch stack decode."""
    n, H, K = STACK.layers, STACK.hidden, STACK.top_k
    lo = torch.empty(n, H, dtype=torch.int16, device="cuda")
    idx = torch.empty(n, K, dtype=torch.int32, device="cuda")
    w = torch.empty(n, K, dtype=torch.float32, device="cuda")
    out = torch.empty(H, dtype=torch.int16, device="cuda")
    stk.decode(torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda(), out, lo, idx, w)
    torch.cuda.synchronize()
    return to_u16(lo), idx.cpu().numpy(), w.cpu().numpy(), to_u16(out)


def test_stack_teacher_forced_and_free_running(stack, stack_kernel):
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import bit_quantized_gemv_amd as q

    X = synth.make_tokens(STACK, N_TOKENS, stream=81)
    runs = []
    for t in range(N_TOKENS):
        log(f"stack token {t}: 30 layers on the device")
        runs.append(_run_gpu(torch, q, stack, X[t]))
        log(f"stack token {t}: one-launch stack decode")
        lo, idx, w, out = _run_stack_kernel(torch, stack_kernel, X[t])
        xs, routing = runs[-1]
        for l in range(STACK.layers):
            assert np.array_equal(lo[l], xs[l + 1]), (t, l, "layer output differs")
            assert np.array_equal(idx[l], routing[l][0]), (t, l)
            assert np.array_equal(w[l].view(np.uint32), routing[l][1].view(np.uint32)), (t, l)
        assert np.array_equal(out, xs[-1])
    assert q.qmoe_workspace_status(stack_kernel.ws) == 0

    # teacher-forced: the oracle's layer l on the device's input to layer l
    flips = 0
    worst = 0.0
    with ThreadPoolExecutor(max_workers=8) as ex:
        for l, (lw, ol, dl) in enumerate(stack):
            res = list(ex.map(lambda t: ol.forward(runs[t][0][l], residual=True), range(N_TOKENS)))
            for t in range(N_TOKENS):
                gidx, gw = runs[t][1][l]
                r = res[t]
                if list(gidx) != list(r["idx"]):
                    assert _near_tie(r["logits"], gidx, r["idx"]), (l, t, "routing flip not a near-tie")
                    flips += 1
                    r = ol.forward(runs[t][0][l], residual=True, force_idx=gidx,
                                   force_w=gw.astype(np.float64))
                e = rel_l2(bf16_to_f64(runs[t][0][l + 1]), bf16_to_f64(r["out"]))
                worst = max(worst, e)
                assert e <= 2e-3, (l, t, e)
    log(f"  teacher-forced: worst layer relL2 {worst:.2e}, certified near-tie flips {flips}")

    # free-running: the device's 30-layer trajectory against the oracle's own.
    # Rounding differences compound through the residual layers (the FFN
    # output dominates the stream), so the bar is the oracle's own
    # divergence under per-layer perturbations at least as large as the
    # device's largest per-layer difference: the lowest bf16 bit of 3% of
    # the elements flipped after every layer (seeded).
    def free(t, flip_frac, seed):
        rng = np.random.default_rng(seed)
        x, xs, step = X[t], [], []
        for lw, ol, dl in stack:
            y = ol.forward(x, residual=True)["out"].copy()
            if flip_frac:
                m = rng.random(y.shape) < flip_frac
                z = y.copy()
                z[m] ^= 1
                step.append(rel_l2(bf16_to_f64(z), bf16_to_f64(y)))
                y = z
            xs.append(y)
            x = y
        return xs, step

    jobs = [(t, 0.0, 0) for t in range(N_TOKENS)] + [(t, 0.03, 100 + t) for t in range(N_TOKENS)]
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        res = list(ex.map(lambda j: free(*j), jobs))
    for t in range(N_TOKENS):
        clean, _ = res[t]
        pert, steps = res[N_TOKENS + t]
        assert min(steps) >= worst, "perturbation smaller than the device's per-layer error"
        for l in (9, 19, 29):
            e = rel_l2(bf16_to_f64(runs[t][0][l + 1]), bf16_to_f64(clean[l]))
            d = rel_l2(bf16_to_f64(pert[l]), bf16_to_f64(clean[l]))
            log(f"  token {t} after layer {l + 1}: device vs oracle {e:.2e}, "
                f"oracle vs perturbed oracle {d:.2e}")
            if flips == 0:
                assert e <= max(2e-3, 2 * d), (t, l, e, d)


def test_stack_residual_stream_grows_and_stays_finite(stack):
    """Every layer adds its FFN output to the residual stream: the device's
    layer outputs are finite and differ from their inputs."""
    import torch

    import bit_quantized_gemv_amd as q

    x = synth.make_tokens(STACK, 1, stream=82)[0]
    xs, _ = _run_gpu(torch, q, stack, x)
    for l in range(STACK.layers):
        a, b = bf16_to_f64(xs[l]), bf16_to_f64(xs[l + 1])
        assert np.all(np.isfinite(b))
        assert not np.array_equal(a, b)
