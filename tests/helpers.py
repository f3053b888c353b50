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


def have_gpu() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)
