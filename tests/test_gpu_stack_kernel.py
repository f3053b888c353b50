"""GPU parity of the one-launch stack decode (qmoe_stack_decode) through the
C ABI: every layer's output and routing equal, bit for bit, those of the
same layers run as ordered one-layer qmoe_moe_decode calls, and every
layer's output is within the relL2 bar of the fp64 oracle's layer on the
same input (teacher-forced; routing differences must be certified near
ties).  Small shapes, shapes without a compile-time specialisation,
repeated and interleaved calls on one workspace, partial stacks, errors."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import (bf16_to_f64, log, rel_l2, routing_bound, routing_certified,
                           to_u16, weights_consistent)

pytestmark = pytest.mark.gpu


def _build(name):
    import torch

    import bit_quantized_gemv_amd as q

    assert torch.cuda.is_available()
    wl = synth.WORKLOADS[name]
    layers = []
    for l in range(wl.layers):
        lw = synth.make_layer(wl, l)
        layers.append((lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)))
    stk = q.Stack([dl.layer for _, _, dl in layers])
    log(f"{name}: {wl.layers} layers, table {stk.table.numel()} B, workspace {stk.ws.numel()} B")
    return wl, layers, stk


@pytest.fixture(scope="module")
def tiny():
    return _build("tiny_stack_decode")


@pytest.fixture(scope="module")
def odd():
    return _build("odd_stack_decode")


def _u16_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _layered(torch, q, wl, layers, x, n, ws):
    """n layers as ordered one-layer launches: outputs, idx, w per layer."""
    cur = _u16_dev(torch, x)
    outs, idxs, ws_ = [], [], []
    for lw, ol, dl in layers[:n]:
        out = torch.empty(wl.hidden, dtype=torch.int16, device="cuda")
        idx = torch.empty(wl.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.top_k, dtype=torch.float32, device="cuda")
        q.qmoe_moe_decode(dl.layer, cur, None, True, out, idx, w, ws)
        cur = out
        outs.append(to_u16(out))
        idxs.append(idx.cpu().numpy())
        ws_.append(w.cpu().numpy())
    return np.stack(outs), np.stack(idxs), np.stack(ws_)


def _stacked(torch, q, wl, stk, x, n):
    lo = torch.empty(n, wl.hidden, dtype=torch.int16, device="cuda")
    idx = torch.empty(n, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(n, wl.top_k, dtype=torch.float32, device="cuda")
    out = torch.empty(wl.hidden, dtype=torch.int16, device="cuda")
    stk.decode(_u16_dev(torch, x), out, lo, idx, w, n_layers=n)
    torch.cuda.synchronize()
    lo, out = to_u16(lo), to_u16(out)
    assert np.array_equal(lo[n - 1], out), "out is the last layer's output"
    return lo, idx.cpu().numpy(), w.cpu().numpy()


def _same(a, b):
    la, ia, wa = a
    lb, ib, wb = b
    assert np.array_equal(ia, ib)
    assert np.array_equal(wa.view(np.uint32), wb.view(np.uint32))
    assert np.array_equal(la, lb)


def _teacher_forced(wl, layers, x, lo, idx, w):
    """Layer l of the oracle on the device's input to layer l."""
    from concurrent.futures import ThreadPoolExecutor

    ins = [x] + [lo[l] for l in range(len(lo) - 1)]

    def one(l):
        ol = layers[l][1]
        r = ol.forward(ins[l], residual=True)
        flip = list(idx[l]) != list(r["idx"])
        lw = layers[l][0]
        B = routing_bound(lw.router, ins[l], r["logits"], gamma=lw.gamma)
        assert weights_consistent(B, r["logits"], idx[l], w[l]), (l, "combine weights")
        if flip:
            assert routing_certified(B, r["logits"], idx[l]), (l, "routing flip not certified")
            r = ol.forward(ins[l], residual=True, force_idx=idx[l],
                           force_w=w[l].astype(np.float64))
        return rel_l2(bf16_to_f64(lo[l]), bf16_to_f64(r["out"])), flip

    with ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, range(len(lo))))
    worst = max(e for e, _ in res)
    log(f"  teacher-forced worst layer relL2 {worst:.2e}, near-tie flips "
        f"{sum(f for _, f in res)}")
    assert worst <= 2e-3


@pytest.mark.parametrize("which", ["tiny", "odd"])
def test_stack_equals_layer_calls_and_oracle(which, request):
    import torch

    import bit_quantized_gemv_amd as q

    wl, layers, stk = request.getfixturevalue(which)
    X = synth.make_tokens(wl, wl.tokens, stream=91)
    ws1 = layers[0][2].layer.new_workspace(1)
    for t in range(wl.tokens):
        log(f"{wl.name} token {t}: stack launch and {wl.layers} one-layer launches")
        a = _stacked(torch, q, wl, stk, X[t], wl.layers)
        b = _layered(torch, q, wl, layers, X[t], wl.layers, ws1)
        _same(a, b)
        _teacher_forced(wl, layers, X[t], *a)
    assert q.qmoe_workspace_status(stk.ws) == 0
    assert q.qmoe_workspace_status(ws1) == 0


def test_stack_repeated_interleaved_and_partial_calls(tiny):
    """One workspace: stack calls of 5, 1 and 2 layers, with one-layer calls
    of the same layers on the same workspace in between; every call's
    results equal those of one-layer calls on a fresh workspace."""
    import torch

    import bit_quantized_gemv_amd as q

    wl, layers, stk = tiny
    X = synth.make_tokens(wl, 6, stream=92)
    ref_ws = layers[0][2].layer.new_workspace(1)
    plan = [(0, 5), (1, 1), (2, 2), (3, 5), (4, 5), (5, 3)]
    for step, (t, n) in enumerate(plan):
        log(f"call {step}: token {t}, {n} layers")
        got = _stacked(torch, q, wl, stk, X[t], n)
        _same(got, _layered(torch, q, wl, layers, X[t], n, ref_ws))
        if step % 2 == 0:
            # one-layer launches sharing the stack's workspace
            _same(_layered(torch, q, wl, layers, X[t], 2, stk.ws),
                  _layered(torch, q, wl, layers, X[t], 2, ref_ws))
    assert q.qmoe_workspace_status(stk.ws) == 0


def test_stack_zero_input_is_zero(tiny):
    """x = 0: RMSNorm gives 0, every GEMV is 0 up to its biases' terms times
    zero sums, so every layer's output is exactly zero."""
    import torch

    import bit_quantized_gemv_amd as q

    wl, layers, stk = tiny
    lo, idx, w = _stacked(torch, q, wl, stk, np.zeros(wl.hidden, np.uint16), wl.layers)
    assert np.all(lo == 0)
    # all logits equal (zero input, no bias): ties go to the lower index
    assert np.array_equal(idx, np.tile(np.arange(wl.top_k, dtype=np.int32), (wl.layers, 1)))
    assert np.allclose(w, 1.0 / wl.top_k)


def test_stack_rejects_bad_arguments(tiny):
    import torch

    import bit_quantized_gemv_amd as q

    wl, layers, stk = tiny
    x = torch.zeros(wl.hidden, dtype=torch.int16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(q.QmoeError):
        q.qmoe_stack_decode(stk.shape, stk.table, 0, x, out, None, None, None, stk.ws)
    with pytest.raises(q.QmoeError):
        q.qmoe_stack_decode(stk.shape, stk.table, 2, x, x, None, None, None, stk.ws)
    with pytest.raises(q.QmoeError):
        q.qmoe_stack_decode(stk.shape, stk.table, 2, x, out, None, None, None, stk.ws[:4096])
    odd_layer = synth.device.DeviceLayer(synth.make_layer(synth.WORKLOADS["odd_stack_decode"], 0))
    with pytest.raises(q.QmoeError):
        q.Stack([layers[0][2].layer, odd_layer.layer])
