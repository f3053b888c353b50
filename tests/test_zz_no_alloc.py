"""GPU check of the allocation-free decode entry point (qmoe_moe_decode_noalloc,
workspace in the library's own per-GPU device array) against qmoe_moe_decode
on a fresh caller workspace: bitwise equal outputs, routing and weights, on
two calls in a row, the second on a smaller layer (and a third on the
first layer again)."""
import ctypes as C

import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import bf16_to_f64, log, rel_l2, to_u16

pytestmark = pytest.mark.gpu


def _both(torch, q, dl, x, residual):
    L = dl.layer
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    res = []
    for noalloc in (False, True):
        out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
        idx = torch.empty(L.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(L.top_k, dtype=torch.float32, device="cuda")
        if noalloc:
            rc = q.lib().qmoe_moe_decode_noalloc(C.byref(L.c()), xd.data_ptr(), None,
                                                 int(residual), out.data_ptr(), idx.data_ptr(),
                                                 w.data_ptr(), torch.cuda.current_stream().cuda_stream)
            assert rc == 0, q.qmoe_status_string(rc) if hasattr(q, "qmoe_status_string") else rc
        else:
            ws = L.new_workspace(1)
            q.qmoe_moe_decode(L, xd, None, residual, out, idx, w, ws)
            assert q.qmoe_workspace_status(ws) == 0
        torch.cuda.synchronize()
        res.append((to_u16(out), idx.cpu().numpy(), w.cpu().numpy()))
    return res


def test_noalloc_equals_workspace_call_big_then_small():
    import torch

    import bit_quantized_gemv_amd as q

    assert torch.cuda.is_available()
    big = synth.WORKLOADS["layer_decode"]
    small = synth.WORKLOADS["tiny_layer_decode"]
    calls = []
    for wl, stream in ((big, 301), (small, 302), (big, 303)):
        lw = synth.make_layer(wl, 0)
        dl = synth.device.DeviceLayer(lw)
        x = synth.make_tokens(wl, 1, stream=stream)[0]
        log(f"noalloc decode {wl.name}")
        (ref, ri, rw), (got, gi, gw) = _both(torch, q, dl, x, residual=wl is small)
        assert np.array_equal(got, ref)
        assert np.array_equal(gi, ri)
        assert np.array_equal(gw.view(np.uint32), rw.view(np.uint32))
        calls.append((lw, x, got, gi, wl is small))
    # and the oracle's bar for the first two calls
    for lw, x, got, gi, residual in calls[:2]:
        r = oracle.OracleLayer(lw).forward(x, residual=residual)
        assert list(gi) == list(r["idx"])
        assert rel_l2(bf16_to_f64(got), bf16_to_f64(r["out"])) <= 2e-3
