"""Shared helpers of the test suite (numerics, error bounds, device plumbing)."""
from __future__ import annotations

import os
import sys

import numpy as np

U32 = 2.0**-24  # fp32 unit roundoff


def gamma_n(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32."""
    return n * U32 / (1 - n * U32)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (d if d > 0 else 1.0))


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_u16(t) -> np.ndarray:
    """torch tensor of 16-bit patterns (int16/bf16/fp16) -> numpy uint16."""
    import torch

    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.view(torch.int16)
    return t.numpy().view(np.uint16)


def codes_of(m) -> np.ndarray:
    """Codes of a QMat through a little-endian byte view (independent of
    both the oracle's and the kernels' unpacking)."""
    by = np.ascontiguousarray(m.q).view(np.uint8).reshape(m.rows, -1)
    if m.bits == 8:
        return by[:, :m.cols].astype(np.float64)
    out = np.empty((m.rows, by.shape[1] * 2), dtype=np.float64)
    out[:, 0::2] = by & 0xF
    out[:, 1::2] = by >> 4
    return out[:, :m.cols]


def gemv4_bound(m, x: np.ndarray) -> np.ndarray:
    """Per-row forward error bound of the 4-bit GEMV as the kernels compute
    it: per 32-column chunk D = sum q x on the dot2 unit (exact products),
    then acc += s D + b X with X the chunk sum of x; chunk partials are
    summed by each lane and across 8 lanes.  Every term passes through at
    most n = 64 + cols/32 roundings, so |err| <= gamma_n * M for any
    M >= sum_c (|s| q_c + |b|) |x_c|; the M used here,
    sum_c (16|s| + |s| q_c + |b - 16 s|) |x_c|, is larger (|b| <= |b - 16 s| + 16|s|)."""
    q = codes_of(m)
    s = np.repeat(m.s.view(np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(m.b.view(np.float16).astype(np.float64), 64, axis=1)
    M = ((16 * np.abs(s) + np.abs(s) * q + np.abs(b - 16 * s)) * np.abs(x)[None, :]).sum(1)
    return gamma_n(64 + m.cols // 32) * M


def gemv8_bound(m, x: np.ndarray) -> np.ndarray:
    """Same for the 8-bit router GEMV (acc += s * sum q x + b * sum x)."""
    q = codes_of(m)
    s = np.repeat(m.s.view(np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(m.b.view(np.float16).astype(np.float64), 64, axis=1)
    M = ((np.abs(s) * q + np.abs(b)) * np.abs(x)[None, :]).sum(1)
    return gamma_n(64 + m.cols // 16) * M


def _abs_dequant(m) -> np.ndarray:
    """|W| of a QMat as fp64 [rows][cols] (from the byte-view codes)."""
    q = codes_of(m)
    s = np.repeat(m.s.view(np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(m.b.view(np.float16).astype(np.float64), 64, axis=1)
    return np.abs(s * q + b)


def _bf16_step(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (the subnormal quantum below 2^-126)."""
    a = np.maximum(np.abs(v), 2.0**-126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def routing_bound(router, x_bits, logits64, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """Per-expert bound on |device logit - fp64 logit| for one token.

    The device computes the router GEMV in fp32 (bounded by gemv8_bound) and
    adds the logit bias with one more fp32 rounding (|l| * 2^-24; doubled for
    the fp32 representation of the fp64 reference).  With an RMSNorm in front
    (gamma given, x the layer input), the device's bf16 expert input may sit
    one bf16 step away from the oracle's wherever the exact value
    x * gamma / rms lies within 64 fp32 roundings of a bf16 rounding midpoint
    (the fp32 sum of squares, square root, division and two products); each
    such element can move logit e by |W_ec| times that step."""
    x = bf16_to_f64(x_bits)
    if gamma is None:
        h = x
    else:
        g = bf16_to_f64(gamma)
        hv = x * g / np.sqrt(np.mean(x * x) + eps)
        step = _bf16_step(hv)
        frac = np.abs(hv) / step
        dist = np.abs(frac - np.floor(frac) - 0.5) * step
        cand = dist <= 64 * U32 * np.abs(hv)
        # the expert input the oracle rounds to (round to nearest even of hv)
        import oracle

        h = bf16_to_f64(oracle.rmsnorm(x_bits, gamma, eps))
    B = gemv8_bound(router, h) + 2 * np.abs(np.asarray(logits64, np.float64)) * U32
    if gamma is not None and np.any(cand):
        # |W (h_dev - h)| plus the GEMV bound's growth from |h_dev| <= |h| + step
        moved = _abs_dequant(router)[:, cand] @ step[cand]
        B = B + (1 + gamma_n(64 + router.cols // 16)) * moved
    return B


def routing_certified(bound, logits64, gidx) -> bool:
    """True when the device's ranking gidx (top-k in rank order, every other
    expert below the last) is consistent with the fp64 logits moved by at
    most `bound` each: for every expert a the device ranks above b,
    l_b - l_a <= bound_a + bound_b."""
    lg = np.asarray(logits64, np.float64)
    B = np.asarray(bound, np.float64)
    sel = [int(e) for e in gidx]
    if len(set(sel)) != len(sel):
        return False
    rest = np.setdiff1d(np.arange(lg.size), sel)
    for j, a in enumerate(sel):
        below = np.concatenate([np.asarray(sel[j + 1:], dtype=np.int64), rest])
        if below.size and np.max(lg[below] - B[below]) > lg[a] + B[a]:
            return False
    return True


def weights_consistent(bound, logits64, gidx, gw) -> bool:
    """The device's combine weights gw for its routing gidx against the fp64
    softmax over the same experts: each logit may be off by its bound B, so
    log w_j may move by at most B_j + max_i B_i (i over the kept experts);
    plus 1e-5 relative for the fp32 softmax itself."""
    lg = np.asarray(logits64, np.float64)[np.asarray(gidx)]
    B = np.asarray(bound, np.float64)[np.asarray(gidx)]
    ref = np.exp(lg - lg.max())
    ref = ref / ref.sum()
    tol = np.expm1(B + B.max()) + 1e-5
    return bool(np.all(np.abs(np.asarray(gw, np.float64) - ref) <= tol * ref + 1e-30))


def have_gpu() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)
