"""Upload synthetic host weights to the GPU as binding objects.

Plumbing only (host -> device copies and pointer bookkeeping); shared by the
GPU tests and the benchmark.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import LayerWeights, QMat


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def qtensor(m: QMat, device="cuda"):
    import bit_quantized_gemv_amd as q

    return q.QTensor(dev(m.q, device), dev(m.s, device), dev(m.b, device), m.rows, m.cols, m.bits)


class DeviceLayer:
    """Device copy of one LayerWeights plus its binding MoeLayer."""

    def __init__(self, lw: LayerWeights, device="cuda", use_prior: bool = True,
                 logit_bias: Optional[np.ndarray] = None, blobs: Optional[torch.Tensor] = None):
        import bit_quantized_gemv_amd as q

        wl = lw.wl
        self.lw = lw
        self.blobs = dev(lw.blobs, device) if blobs is None else blobs
        offs = {n: o for n, o, _ in lw.layout.offsets}
        gate, up, down = q.MoeLayer.stacked_experts(self.blobs, offs, wl.hidden, wl.inter)
        self.gamma = None if lw.gamma is None else dev(lw.gamma, device)
        bias = logit_bias
        if bias is None and use_prior and lw.prior is not None:
            bias = lw.prior
        self.logit_bias = None if bias is None else dev(np.asarray(bias, np.float32), device)
        self.layer = q.MoeLayer(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter,
                                qtensor(lw.router, device), gate, up, down,
                                qtensor(lw.sh_gate, device), qtensor(lw.sh_up, device),
                                qtensor(lw.sh_down, device), rms_gamma=self.gamma,
                                rms_eps=1e-6, logit_bias=self.logit_bias)
