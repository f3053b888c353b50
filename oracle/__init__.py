"""fp64 scalar CPU oracle of the quantized MoE FFN step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package; the product path
(``bit_quantized_gemv_amd``) never does.  The arithmetic lives in
``oracle.c`` (plain C, fp64, no shared code with the HIP library); this file
only marshals numpy arrays into it.

Every oracle function has a pin in ``tests/test_oracle_pins.py``,
``tests/test_sample_pins.py`` (sampling) or ``tests/test_attn_pins.py``
(decode attention, RoPE, the fp16 encoder).  Parity is
unpinned for: the bit order of MLX codes inside a word (no trained MLX weights
are loaded; both sides read the same generator output) and the Zipf prior's
scale (a workload choice).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=gnu11",
                               "-Wall", "-Wno-unused-function", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _QMat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [("H", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("I", C.c_int32), ("Is", C.c_int32),
                ("router", _QMat), ("gate", C.c_void_p), ("up", C.c_void_p),
                ("down", C.c_void_p), ("sh_gate", _QMat), ("sh_up", _QMat),
                ("sh_down", _QMat), ("gamma", C.c_void_p), ("logit_bias", C.c_void_p)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=False)
            L = C.CDLL(_LIB)
            L.orc_half_to_double.restype = C.c_double
            L.orc_half_to_double.argtypes = [C.c_uint16]
            L.orc_bf16_to_double.restype = C.c_double
            L.orc_bf16_to_double.argtypes = [C.c_uint16]
            L.orc_double_to_bf16.restype = C.c_uint16
            L.orc_double_to_bf16.argtypes = [C.c_double]
            L.orc_gelu_tanh.restype = C.c_double
            L.orc_gelu_tanh.argtypes = [C.c_double]
            L.orc_unpack.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int, C.c_void_p]
            L.orc_dequant.argtypes = [C.c_void_p] * 3 + [C.c_int64, C.c_int64, C.c_int, C.c_void_p]
            L.orc_qgemv.argtypes = [C.c_void_p] * 3 + [C.c_int64, C.c_int64, C.c_int,
                                                       C.c_void_p, C.c_void_p]
            L.orc_rmsnorm.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_double, C.c_void_p]
            L.orc_topk_softmax.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
            L.orc_router_logits.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
            L.orc_expert_ffn.argtypes = [C.c_void_p] * 3 + [C.c_int32, C.c_int32,
                                                            C.c_void_p, C.c_void_p]
            L.orc_layer_forward.restype = C.c_int
            L.orc_layer_forward.argtypes = [C.c_void_p, C.c_void_p, C.c_int] + [C.c_void_p] * 8
            L.orc_dispatch.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_void_p, C.c_void_p, C.c_void_p]
            L.orc_lfu_replay.restype = C.c_int64
            L.orc_lfu_replay.argtypes = [C.c_int32] * 4 + [C.c_void_p] * 4
            L.orc_sample.restype = C.c_int32
            L.orc_sample.argtypes = [C.c_void_p, C.c_int32, C.c_double, C.c_int32, C.c_double,
                                     C.c_double, C.c_void_p, C.c_void_p, C.c_void_p]
            L.orc_double_to_half.restype = C.c_uint16
            L.orc_double_to_half.argtypes = [C.c_double]
            L.orc_rope.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_double, C.c_void_p]
            L.orc_attn_step.restype = C.c_int
            L.orc_attn_step.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_double,
                                        C.c_double, C.c_int64] + [C.c_void_p] * 6
            _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------ scalar helpers
def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def double_to_bf16(v: float) -> int:
    return lib().orc_double_to_bf16(float(v))


def bf16_vec_to_double(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([L.orc_bf16_to_double(int(b)) for b in flat]).reshape(np.shape(bits))


def gelu_tanh(z: float) -> float:
    return lib().orc_gelu_tanh(float(z))


# ------------------------------------------------------------ matrix helpers
def unpack(q: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    q = _c(q, np.uint32)
    out = np.zeros((rows, cols), dtype=np.uint8)
    lib().orc_unpack(_p(q), rows, cols, bits, _p(out))
    return out


def dequant(m) -> np.ndarray:
    q, s, b = _c(m.q, np.uint32), _c(m.s, np.uint16), _c(m.b, np.uint16)
    W = np.zeros((m.rows, m.cols), dtype=np.float64)
    lib().orc_dequant(_p(q), _p(s), _p(b), m.rows, m.cols, m.bits, _p(W))
    return W


def qgemv(m, x: np.ndarray) -> np.ndarray:
    q, s, b = _c(m.q, np.uint32), _c(m.s, np.uint16), _c(m.b, np.uint16)
    x = _c(x, np.float64)
    y = np.zeros(m.rows, dtype=np.float64)
    lib().orc_qgemv(_p(q), _p(s), _p(b), m.rows, m.cols, m.bits, _p(x), _p(y))
    return y


def rmsnorm(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x, g = _c(x_bits, np.uint16), _c(gamma_bits, np.uint16)
    h = np.zeros_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(h))
    return h


def topk_softmax(logits: np.ndarray, k: int):
    lg = _c(logits, np.float64)
    idx = np.zeros(k, dtype=np.int32)
    w = np.zeros(k, dtype=np.float64)
    lib().orc_topk_softmax(_p(lg), lg.size, k, _p(idx), _p(w))
    return idx, w


def expert_ffn(g, u, d, h_bits: np.ndarray) -> np.ndarray:
    keep = []
    mats = []
    for m in (g, u, d):
        q, s, b = _c(m.q, np.uint32), _c(m.s, np.uint16), _c(m.b, np.uint16)
        keep += [q, s, b]
        mats.append(_QMat(_p(q), _p(s), _p(b)))
    h = _c(h_bits, np.uint16)
    y = np.zeros(g.cols, dtype=np.float64)
    lib().orc_expert_ffn(C.byref(mats[0]), C.byref(mats[1]), C.byref(mats[2]),
                         g.cols, g.rows, _p(h), _p(y))
    return y


# ------------------------------------------------------------------ layers
class OracleLayer:
    """Holds the ctypes view of one synth.LayerWeights (arrays kept alive)."""

    def __init__(self, lw, logit_bias: Optional[np.ndarray] = None, use_prior: bool = True):
        self.lw = lw
        wl = lw.wl
        self._keep = []

        def qm(m):
            q, s, b = _c(m.q, np.uint32), _c(m.s, np.uint16), _c(m.b, np.uint16)
            self._keep += [q, s, b]
            return _QMat(_p(q), _p(s), _p(b))

        E = wl.n_experts
        self._gate = (_QMat * E)()
        self._up = (_QMat * E)()
        self._down = (_QMat * E)()
        for e in range(E):
            g, u, d = lw.expert(e)
            self._gate[e], self._up[e], self._down[e] = qm(g), qm(u), qm(d)
        bias = logit_bias
        if bias is None and use_prior and lw.prior is not None:
            bias = lw.prior
        self.logit_bias = None if bias is None else _c(bias, np.float32)
        gamma = None if lw.gamma is None else _c(lw.gamma, np.uint16)
        self._keep += [gamma, self.logit_bias]
        self.s = _Layer(wl.hidden, E, wl.top_k, wl.inter, wl.shared_inter,
                        qm(lw.router), C.addressof(self._gate), C.addressof(self._up),
                        C.addressof(self._down), qm(lw.sh_gate), qm(lw.sh_up),
                        qm(lw.sh_down), _p(gamma), _p(self.logit_bias))

    def forward(self, x_bits: np.ndarray, residual: bool = False,
                force_idx: Optional[Sequence[int]] = None,
                force_w: Optional[Sequence[float]] = None) -> Dict[str, np.ndarray]:
        wl = self.lw.wl
        H, E, K = wl.hidden, wl.n_experts, wl.top_k
        x = _c(x_bits, np.uint16)
        out = np.zeros(H, dtype=np.uint16)
        y = np.zeros(H, dtype=np.float64)
        h = np.zeros(H, dtype=np.uint16)
        logits = np.zeros(E, dtype=np.float64)
        idx = np.zeros(K, dtype=np.int32)
        w = np.zeros(K, dtype=np.float64)
        fi = None if force_idx is None else _c(force_idx, np.int32)
        fw = None if force_w is None else _c(force_w, np.float64)
        lib().orc_layer_forward(C.byref(self.s), _p(x), int(residual), _p(fi), _p(fw),
                                _p(out), _p(y), _p(h), _p(logits), _p(idx), _p(w))
        return {"out": out, "y": y, "h": h, "logits": logits, "idx": idx, "w": w}

    def router_logits(self, h_bits: np.ndarray) -> np.ndarray:
        h = _c(h_bits, np.uint16)
        logits = np.zeros(self.lw.wl.n_experts, dtype=np.float64)
        lib().orc_router_logits(C.byref(self.s), _p(h), _p(logits))
        return logits


def forward_many(layer: OracleLayer, X: np.ndarray, threads: int = 0, **kw):
    """Run ``layer.forward`` over the rows of X on a thread pool (the C code
    runs without the GIL).  Returns a list of result dicts."""
    from concurrent.futures import ThreadPoolExecutor

    n = X.shape[0]
    threads = threads or min(n, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda t: layer.forward(X[t], **kw), range(n)))


def dispatch(idx: np.ndarray, n_experts: int):
    idx = _c(idx, np.int32)
    T, K = idx.shape
    counts = np.zeros(n_experts, dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    perm = np.zeros(T * K, dtype=np.int32)
    lib().orc_dispatch(_p(idx), T, K, n_experts, _p(counts), _p(offsets), _p(perm))
    return counts, offsets, perm


def lfu_replay(need: np.ndarray, n_experts: int, slots: int):
    need = _c(need, np.int32)
    steps, K = need.shape
    hit = np.zeros_like(need)
    slot = np.zeros_like(need)
    victim = np.zeros_like(need)
    hits = lib().orc_lfu_replay(n_experts, slots, K, steps, _p(need), _p(hit), _p(slot),
                                _p(victim))
    if hits < 0:
        raise RuntimeError("LFU replay found no victim")
    return {"hits": int(hits), "hit": hit, "slot": slot, "victim": victim}


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float):
    """The sampled token id, the ranked top_k ids, their cumulative
    masses over the total (fp64) and the number of kept ranks."""
    logits = _c(logits, np.float32)
    ranked = np.zeros(top_k, dtype=np.int32)
    cum = np.zeros(top_k, dtype=np.float64)
    kept = np.zeros(1, dtype=np.int32)
    tok = lib().orc_sample(_p(logits), logits.size, float(temperature), int(top_k),
                           float(top_p), float(u), _p(ranked), _p(cum), _p(kept))
    return {"token": int(tok), "ranked": ranked, "cum": cum, "kept": int(kept[0])}


def double_to_half(v: float) -> int:
    return int(lib().orc_double_to_half(float(v)))


def rope(x: np.ndarray, pos: int, base: float) -> np.ndarray:
    """RoPE of one head vector (fp64), pairs (i, i + D/2)."""
    x = _c(x, np.float64)
    out = np.zeros_like(x)
    lib().orc_rope(_p(x), x.size, int(pos), float(base), _p(out))
    return out


def attn_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, khist: np.ndarray,
              vhist: np.ndarray, pos: int, window: int, scale: float, base: float) -> np.ndarray:
    """One decode attention step of the token at time ``pos``.

    q [Hq][D], k and v [Hkv][D] (fp32); khist and vhist [times][Hkv][D] fp16
    bits in time order, modified in place (time ``pos`` is written).  Returns
    the output [Hq][D] in fp64."""
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    Hq, D = q.shape
    Hkv = k.shape[0]
    assert khist.dtype == np.uint16 and khist.flags.c_contiguous and khist.shape[0] > pos
    assert vhist.dtype == np.uint16 and vhist.flags.c_contiguous and vhist.shape == khist.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    rc = lib().orc_attn_step(Hq, Hkv, D, int(window), float(scale), float(base), int(pos),
                             _p(q), _p(k), _p(v), _p(khist), _p(vhist), _p(out))
    if rc:
        raise ValueError("orc_attn_step: bad shape")
    return out
