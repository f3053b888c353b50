"""GPU regression tests of the workspace's tag counter: every decode call on
a workspace matches its cross-block flags and tags against values no earlier
call wrote, whatever ran in between (other kernels, other modes, other layer
shapes, the counter's restart).  Each call's results must equal those of the
same call on a fresh workspace, bit for bit, and the oracle's."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import bf16_to_f64, log, rel_l2, to_u16

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_layer_decode"]
ODD = synth.WORKLOADS["odd_experts_decode"]
RESTART = 0xFFFFFF00  # the counter restarts before reaching this value


@pytest.fixture(scope="module")
def env():
    import torch

    import bit_quantized_gemv_amd as q

    assert torch.cuda.is_available()
    out = {}
    for wl in (TINY, ODD):
        lw = synth.make_layer(wl, 0)
        out[wl.name] = (lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw))
    return torch, q, out


def _u16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _shared_ws(torch, q, layers):
    """One zero-filled workspace large enough for every layer given."""
    n = max(max(q.qmoe_workspace_bytes(dl.layer, 1), q.qmoe_stack_workspace_bytes(dl.layer))
            for _, _, dl in layers)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _decode(torch, q, dl, x, ws, mode="fused"):
    L = dl.layer
    out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
    idx = torch.empty(L.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(L.top_k, dtype=torch.float32, device="cuda")
    q.qmoe_moe_decode(L, _u16(torch, x), None, True, out, idx, w, ws, phased=mode == "phased")
    torch.cuda.synchronize()
    return to_u16(out), idx.cpu().numpy(), w.cpu().numpy()


def _split(torch, q, dl, h, idx, w, ws):
    L = dl.layer
    out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
    hd = _u16(torch, h)
    q.qmoe_expert_ffn_shared(L, hd, ws)
    q.qmoe_expert_ffn_routed(L, hd, torch.from_numpy(np.asarray(idx, np.int32)).cuda(),
                             torch.from_numpy(np.asarray(w, np.float32)).cuda(), None, None, out,
                             ws)
    torch.cuda.synchronize()
    return to_u16(out)


def _fresh(torch, q, dl, x, mode="fused"):
    ws = dl.layer.new_workspace(1)
    r = _decode(torch, q, dl, x, ws, mode)
    assert q.qmoe_workspace_status(ws) == 0
    return r


def _same(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def _oracle_ok(ol, x, got):
    r = ol.forward(x, residual=True)
    assert list(got[1]) == list(r["idx"])
    assert rel_l2(bf16_to_f64(got[0]), bf16_to_f64(r["out"])) <= 2e-3


def test_tag_counter_advances_by_the_tags_each_call_uses(env):
    torch, q, L = env
    lw, ol, dl = L[TINY.name]
    ws = dl.layer.new_workspace(1)
    X = synth.make_tokens(TINY, 4, stream=201)
    assert q.qmoe_workspace_tag_counter(ws) == 0
    _decode(torch, q, dl, X[0], ws)
    assert q.qmoe_workspace_tag_counter(ws) == 1
    _decode(torch, q, dl, X[1], ws, mode="phased")
    assert q.qmoe_workspace_tag_counter(ws) == 2
    idx, w = synth.dirichlet_routing(TINY, 1, stream=3)
    _split(torch, q, dl, X[2], idx[0], w[0], ws)
    assert q.qmoe_workspace_tag_counter(ws) == 4   # shared-only, then routed
    stk = q.Stack([dl.layer] * 5)
    out = torch.empty(TINY.hidden, dtype=torch.int16, device="cuda")
    q.qmoe_workspace_raise_tag_counter(stk.ws, 7)
    stk.decode(_u16(torch, X[3]), out)
    assert q.qmoe_workspace_tag_counter(stk.ws) == 12
    assert q.qmoe_workspace_status(ws) == 0 and q.qmoe_workspace_status(stk.ws) == 0


def test_calls_separated_by_many_other_launches(env):
    """Two calls on one workspace with thousands of unrelated kernel launches
    between them (enough to wrap any dispatch queue): both equal fresh-
    workspace calls and the oracle."""
    torch, q, L = env
    lw, ol, dl = L[TINY.name]
    X = synth.make_tokens(TINY, 2, stream=202)
    ws = dl.layer.new_workspace(1)
    a = _decode(torch, q, dl, X[0], ws)
    filler = torch.zeros(64, device="cuda")
    for i in range(6000):
        filler.add_(1.0)
    torch.cuda.synchronize()
    b = _decode(torch, q, dl, X[1], ws)
    assert q.qmoe_workspace_status(ws) == 0
    assert float(filler[0]) == 6000.0
    _same(a, _fresh(torch, q, dl, X[0]))
    _same(b, _fresh(torch, q, dl, X[1]))
    _oracle_ok(ol, X[0], a)
    _oracle_ok(ol, X[1], b)


def test_mixed_modes_and_shapes_on_one_workspace(env):
    """One workspace serves, in turn: fused, phased and split calls of one
    layer, a layer of another shape, and stack calls; each result equals the
    same call on a fresh workspace."""
    torch, q, L = env
    tiny, odd = L[TINY.name], L[ODD.name]
    ws = _shared_ws(torch, q, [tiny, odd])
    Xt = synth.make_tokens(TINY, 6, stream=203)
    Xo = synth.make_tokens(ODD, 3, stream=204)
    idx, w = synth.dirichlet_routing(TINY, 2, stream=4)
    stk = q.Stack([tiny[2].layer] * 3)
    stk_out = torch.empty(TINY.hidden, dtype=torch.int16, device="cuda")
    ref_stack = []
    for i in range(2):
        ws1 = stk.ws.clone().zero_()
        stk.ws, keep = ws1, stk.ws
        stk.decode(_u16(torch, Xt[4 + i]), stk_out)
        torch.cuda.synchronize()
        ref_stack.append(to_u16(stk_out))
        stk.ws = keep
    for rep in range(3):
        log(f"round {rep}")
        _same(_decode(torch, q, tiny[2], Xt[0], ws), _fresh(torch, q, tiny[2], Xt[0]))
        _same(_decode(torch, q, odd[2], Xo[rep], ws), _fresh(torch, q, odd[2], Xo[rep]))
        _same(_decode(torch, q, tiny[2], Xt[1], ws, mode="phased"),
              _fresh(torch, q, tiny[2], Xt[1]))
        ref = _split(torch, q, tiny[2], Xt[2], idx[0], w[0], tiny[2].layer.new_workspace(1))
        assert np.array_equal(_split(torch, q, tiny[2], Xt[2], idx[0], w[0], ws), ref)
        # the stack on the same workspace (its layer-input buffers lie past
        # the one-layer part, inside this larger workspace)
        q.qmoe_stack_decode(stk.shape, stk.table, 3, _u16(torch, Xt[4 + rep % 2]), stk_out,
                            None, None, None, ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_u16(stk_out), ref_stack[rep % 2])
        _same(_decode(torch, q, odd[2], Xo[rep], ws), _fresh(torch, q, odd[2], Xo[rep]))
    assert q.qmoe_workspace_status(ws) == 0


def test_tag_counter_restart(env):
    """Near the top of its range the counter restarts at 0 after clearing
    every flag and tag: calls across the restart keep their results."""
    torch, q, L = env
    lw, ol, dl = L[TINY.name]
    X = synth.make_tokens(TINY, 4, stream=205)
    ws = dl.layer.new_workspace(1)
    q.qmoe_workspace_raise_tag_counter(ws, RESTART - 2)
    a = _decode(torch, q, dl, X[0], ws)
    assert q.qmoe_workspace_tag_counter(ws) == RESTART - 1
    b = _decode(torch, q, dl, X[1], ws)            # uses RESTART - 0 ... restarts
    assert q.qmoe_workspace_tag_counter(ws) == 0
    c = _decode(torch, q, dl, X[2], ws)
    assert q.qmoe_workspace_tag_counter(ws) == 1
    for got, x in zip((a, b, c), X[:3]):
        _same(got, _fresh(torch, q, dl, x))
    # a stack call crossing the threshold
    stk = q.Stack([dl.layer] * 5)
    out = torch.empty(TINY.hidden, dtype=torch.int16, device="cuda")
    ref_ws = stk.ws.clone()
    stk.decode(_u16(torch, X[3]), out)
    ref = to_u16(out)
    stk.ws = ref_ws.zero_()
    q.qmoe_workspace_raise_tag_counter(stk.ws, RESTART - 3)
    stk.decode(_u16(torch, X[3]), out)
    assert np.array_equal(to_u16(out), ref)
    assert q.qmoe_workspace_tag_counter(stk.ws) == 0
    stk.decode(_u16(torch, X[3]), out)
    assert np.array_equal(to_u16(out), ref)
    assert q.qmoe_workspace_tag_counter(stk.ws) == 5
    assert q.qmoe_workspace_status(ws) == 0 and q.qmoe_workspace_status(stk.ws) == 0
