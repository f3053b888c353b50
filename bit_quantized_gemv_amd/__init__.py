"""Python binding of libqmoe (include/qmoe.h): argument marshalling only.

Every step of the quantized MoE FFN runs in the gfx950 HIP kernels of
``libqmoe.so``; PyTorch only provides device memory and streams.  The
library is built in-tree by ``bit_quantized_gemv_amd.build``; importing this
package without it raises ImportError (there is no fallback path).

Names mirror the C entry points: ``qmoe_gemv_affine4``, ``qmoe_router_topk``,
``qmoe_expert_ffn``, ``qmoe_moe_decode``, ``qmoe_prefill_grouped``,
``qmoe_rmsnorm``, ``qmoe_workspace_bytes``, ``qmoe_workspace_status``,
``qmoe_stack_decode`` (with ``Stack``, a table and workspace holder).
Tensor arguments are torch tensors on the GPU; bf16/fp16 data may be given as
``torch.bfloat16`` / ``torch.float16`` or as 16-bit integer bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# QMOE_LIB may name another build of the same library (the trace build)
LIB_PATH = os.environ.get("QMOE_LIB") or os.path.join(_HERE, "libqmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m bit_quantized_gemv_amd.build` "
        "(the quantized MoE path has no CPU fallback)")

# One HIP runtime per process: torch's libtorch_hip asks for its bundled
# libamdhip64 by file name, so if this library (which names the runtime by
# its soname) were loaded first, torch would map a second runtime next to
# it, and device symbols set through one would be unknown to the other.
# Loading torch first makes this library bind to torch's runtime.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

# status codes
QMOE_OK = 0
STATUS_NAMES = {0: "QMOE_OK", 1: "QMOE_ERR_NULL_ARG", 2: "QMOE_ERR_BAD_SHAPE",
                3: "QMOE_ERR_UNSUPPORTED", 4: "QMOE_ERR_WORKSPACE", 5: "QMOE_ERR_ALIGN",
                6: "QMOE_ERR_HIP", 7: "QMOE_ERR_DEVICE"}


class QmoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        msg = _lib.qmoe_status_string(code).decode()
        super().__init__(f"{fn}: {STATUS_NAMES.get(code, code)} ({msg})")


class _QT(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("rows", C.c_int32), ("cols", C.c_int32), ("bits", C.c_int32),
                ("group", C.c_int32), ("expert_stride_bytes", C.c_int64)]


class _Layer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32),
                ("router", _QT), ("gate", _QT), ("up", _QT), ("down", _QT),
                ("sh_gate", _QT), ("sh_up", _QT), ("sh_down", _QT),
                ("rms_gamma", C.c_void_p), ("rms_eps", C.c_float), ("logit_bias", C.c_void_p)]


_vp = C.c_void_p
_lib.qmoe_status_string.restype = C.c_char_p
_lib.qmoe_status_string.argtypes = [C.c_int]
_lib.qmoe_gemv_affine4.argtypes = [C.POINTER(_QT), _vp, _vp, _vp]
_lib.qmoe_sample_workspace_bytes.restype = C.c_size_t
_lib.qmoe_sample_workspace_bytes.argtypes = [C.c_int32, C.c_int32]
_lib.qmoe_sample.argtypes = [_vp, C.c_int32, C.c_float, C.c_int32, C.c_float, C.c_float, _vp, _vp,
                             _vp, C.c_size_t, _vp]
_lib.qmoe_attn_workspace_bytes.restype = C.c_size_t
_lib.qmoe_attn_workspace_bytes.argtypes = [C.c_void_p]
_lib.qmoe_attn_decode.argtypes = [C.c_void_p, _vp, _vp, _vp, C.c_int32, _vp, _vp, _vp, _vp,
                                  C.c_size_t, _vp]
_lib.qmoe_attn_workspace_status.argtypes = [_vp, C.c_size_t, C.c_int32, C.POINTER(C.c_int32),
                                            _vp]
_lib.qmoe_tiled4_bytes.restype = C.c_size_t
_lib.qmoe_tiled4_bytes.argtypes = [C.c_int32, C.c_int32]
_lib.qmoe_repack_tiled4.argtypes = [_vp, _vp, _vp, C.c_int32, C.c_int32, _vp, C.c_size_t]
_lib.qmoe_gemv_tiled4.argtypes = [_vp, C.c_int32, C.c_int32, _vp, _vp, C.c_int32, _vp]
_lib.qmoe_router_topk.argtypes = [C.POINTER(_QT), _vp, _vp, C.c_int32, C.c_int32, _vp, _vp, _vp,
                                  _vp, C.c_size_t, _vp]
_lib.qmoe_expert_ffn.argtypes = [C.POINTER(_Layer), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 C.c_size_t, _vp]
_lib.qmoe_moe_decode.argtypes = [C.POINTER(_Layer), _vp, _vp, C.c_int32, _vp, _vp, _vp, _vp,
                                 C.c_size_t, _vp]
_lib.qmoe_moe_decode_phased.argtypes = _lib.qmoe_moe_decode.argtypes
_lib.qmoe_moe_decode_noalloc.argtypes = [C.POINTER(_Layer), _vp, _vp, C.c_int32, _vp, _vp, _vp,
                                         _vp]
_lib.qmoe_moe_decode_timed.argtypes = _lib.qmoe_moe_decode.argtypes + [_vp, _vp]
_lib.qmoe_prefill_grouped.argtypes = [C.POINTER(_Layer), _vp, C.c_int32, _vp, _vp, _vp, _vp, _vp,
                                      C.c_size_t, _vp]
_lib.qmoe_prefill_dispatch_offsets.argtypes = [C.POINTER(_Layer), C.c_int32,
                                               C.POINTER(C.c_size_t), C.POINTER(C.c_size_t),
                                               C.POINTER(C.c_size_t)]
_lib.qmoe_expert_ffn_shared.argtypes = [C.POINTER(_Layer), _vp, _vp, C.c_size_t, _vp]
_lib.qmoe_expert_ffn_routed.argtypes = _lib.qmoe_expert_ffn.argtypes


class PoolStats(C.Structure):
    _fields_ = [("hits", C.c_int64), ("misses", C.c_int64), ("h2d_bytes", C.c_int64),
                ("last_hits", C.c_int32), ("last_misses", C.c_int32)]


_lib.qmoe_pool_create.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_size_t, _vp, _vp,
                                  C.POINTER(_vp)]
_lib.qmoe_pool_plan.argtypes = [_vp, C.c_int32, _vp, C.c_int32, _vp, _vp, _vp]
_lib.qmoe_pool_acquire.argtypes = [_vp, C.c_int32, _vp, C.c_int32, _vp, _vp, _vp,
                                   C.POINTER(PoolStats)]
_lib.qmoe_pool_stats_get.argtypes = [_vp, C.POINTER(PoolStats)]
_lib.qmoe_pool_destroy.argtypes = [_vp]
_lib.qmoe_pool_destroy.restype = None


class FileTierStats(C.Structure):
    _fields_ = [("reads", C.c_int64), ("read_bytes", C.c_int64), ("read_ns", C.c_int64),
                ("last_errno", C.c_int32)]


_lib.qmoe_file_tier_open.argtypes = [C.c_char_p, C.c_int32, C.c_int32, C.c_size_t, C.c_size_t,
                                     C.c_int32, C.c_int32, C.c_int32, C.POINTER(_vp)]
_lib.qmoe_pool_acquire_file.argtypes = [_vp, _vp, C.c_int32, _vp, C.c_int32, _vp, _vp, _vp,
                                        C.POINTER(PoolStats)]
_lib.qmoe_file_tier_stats_get.argtypes = [_vp, C.POINTER(FileTierStats)]
_lib.qmoe_file_tier_close.argtypes = [_vp]
_lib.qmoe_file_tier_close.restype = None
_lib.qmoe_rmsnorm.argtypes = [_vp, _vp, C.c_float, C.c_int32, C.c_int32, _vp, _vp]
_lib.qmoe_workspace_bytes.restype = C.c_size_t
_lib.qmoe_workspace_bytes.argtypes = [C.POINTER(_Layer), C.c_int32]
_lib.qmoe_router_workspace_bytes.restype = C.c_size_t
_lib.qmoe_router_workspace_bytes.argtypes = [C.c_int32, C.c_int32]
_lib.qmoe_workspace_status.argtypes = [_vp, C.c_size_t, C.POINTER(C.c_int32), _vp]
_lib.qmoe_workspace_tag_counter.argtypes = [_vp, C.c_size_t, C.POINTER(C.c_uint32), _vp]
_lib.qmoe_workspace_raise_tag_counter.argtypes = [_vp, C.c_size_t, C.c_uint32, _vp]
_lib.qmoe_stack_table_bytes.restype = C.c_size_t
_lib.qmoe_stack_table_bytes.argtypes = [C.c_int32]
_lib.qmoe_stack_table_init.argtypes = [C.POINTER(_Layer), C.c_int32, _vp, C.c_size_t, _vp]
_lib.qmoe_stack_workspace_bytes.restype = C.c_size_t
_lib.qmoe_stack_workspace_bytes.argtypes = [C.POINTER(_Layer)]
_lib.qmoe_stack_decode.argtypes = [C.POINTER(_Layer), _vp, C.c_int32, _vp, _vp, _vp, _vp, _vp,
                                   _vp, C.c_size_t, _vp]
for _f in ("qmoe_gemv_affine4", "qmoe_router_topk", "qmoe_expert_ffn", "qmoe_moe_decode",
           "qmoe_moe_decode_phased", "qmoe_prefill_grouped", "qmoe_rmsnorm",
           "qmoe_workspace_status", "qmoe_prefill_dispatch_offsets", "qmoe_moe_decode_timed",
           "qmoe_expert_ffn_shared", "qmoe_expert_ffn_routed", "qmoe_pool_create",
           "qmoe_pool_plan", "qmoe_pool_acquire", "qmoe_pool_stats_get", "qmoe_file_tier_open",
           "qmoe_pool_acquire_file", "qmoe_file_tier_stats_get",
           "qmoe_stack_table_init", "qmoe_stack_decode", "qmoe_workspace_tag_counter",
           "qmoe_moe_decode_noalloc", "qmoe_repack_tiled4", "qmoe_gemv_tiled4", "qmoe_sample",
           "qmoe_workspace_raise_tag_counter"):
    getattr(_lib, _f).restype = C.c_int


def lib() -> C.CDLL:
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, code: int) -> None:
    if code != QMOE_OK:
        raise QmoeError(fn, code)


class QTensor:
    """One affine-quantized matrix on the GPU (or stacked experts)."""

    def __init__(self, q, scales, biases, rows: int, cols: int, bits: int,
                 expert_stride_bytes: int = 0, owner=None):
        self.q, self.scales, self.biases = q, scales, biases
        self.rows, self.cols, self.bits = rows, cols, bits
        self.expert_stride_bytes = expert_stride_bytes
        self._owner = owner  # keeps a backing tensor alive when q/s/b are raw addresses

    def c(self) -> _QT:
        return _QT(_ptr(self.q), _ptr(self.scales), _ptr(self.biases), self.rows, self.cols,
                   self.bits, 64, self.expert_stride_bytes)


class MoeLayer:
    """Device weights of one MoE layer, as the C struct qmoe_moe_layer."""

    def __init__(self, hidden: int, n_experts: int, top_k: int, inter: int, shared_inter: int,
                 router: QTensor, gate: QTensor, up: QTensor, down: QTensor, sh_gate: QTensor,
                 sh_up: QTensor, sh_down: QTensor, rms_gamma=None, rms_eps: float = 1e-6,
                 logit_bias=None):
        self.hidden, self.n_experts, self.top_k = hidden, n_experts, top_k
        self.inter, self.shared_inter = inter, shared_inter
        self.router, self.gate, self.up, self.down = router, gate, up, down
        self.sh_gate, self.sh_up, self.sh_down = sh_gate, sh_up, sh_down
        self.rms_gamma, self.rms_eps, self.logit_bias = rms_gamma, rms_eps, logit_bias
        self._c = None

    @staticmethod
    def stacked_experts(blobs, offsets: Dict[str, int], hidden: int, inter: int):
        """gate/up/down QTensors over a [E][blob_bytes] uint8 device tensor in
        which every expert blob holds its parts at the given byte offsets."""
        base = blobs.data_ptr()
        stride = blobs.stride(0) * blobs.element_size()

        def qt(name, rows, cols):
            return QTensor(base + offsets[name + ".q"], base + offsets[name + ".s"],
                           base + offsets[name + ".b"], rows, cols, 4, stride, owner=blobs)

        return (qt("gate", inter, hidden), qt("up", inter, hidden), qt("down", hidden, inter))

    def c(self) -> _Layer:
        if self._c is None:
            self._c = _Layer(self.hidden, self.n_experts, self.top_k, self.inter,
                             self.shared_inter, self.router.c(), self.gate.c(), self.up.c(),
                             self.down.c(), self.sh_gate.c(), self.sh_up.c(), self.sh_down.c(),
                             _ptr(self.rms_gamma), float(self.rms_eps), _ptr(self.logit_bias))
        return self._c

    def workspace_bytes(self, T: int = 1) -> int:
        return qmoe_workspace_bytes(self, T)

    def new_workspace(self, T: int = 1, device="cuda"):
        import torch

        n = self.workspace_bytes(T)
        if n == 0:
            raise QmoeError("qmoe_workspace_bytes", 2)
        return torch.zeros(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------- entry points
def qmoe_workspace_bytes(layer: MoeLayer, T: int = 1) -> int:
    return int(_lib.qmoe_workspace_bytes(C.byref(layer.c()), T))


def qmoe_router_workspace_bytes(n_experts: int, T: int) -> int:
    return int(_lib.qmoe_router_workspace_bytes(n_experts, T))


def qmoe_gemv_affine4(W: QTensor, x, y, stream=None) -> None:
    qt = W.c()
    _check("qmoe_gemv_affine4", _lib.qmoe_gemv_affine4(C.byref(qt), _ptr(x), _ptr(y),
                                                        _stream(stream)))


def qmoe_sample_workspace_bytes(V: int, top_k: int) -> int:
    return int(_lib.qmoe_sample_workspace_bytes(V, top_k))


def qmoe_sample(logits, V: int, temperature: float, top_k: int, top_p: float, u: float, token,
                ranked, ws, stream=None) -> None:
    _check("qmoe_sample", _lib.qmoe_sample(_ptr(logits), V, float(temperature), top_k,
                                            float(top_p), float(u), _ptr(token), _ptr(ranked),
                                            _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream)))


class AttnShape(C.Structure):
    """qmoe_attn_shape: head counts, head width, cache slots, circular or
    linear store, RoPE base and score scale."""
    _fields_ = [("n_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("slots", C.c_int32), ("circular", C.c_int32), ("rope_base", C.c_float),
                ("scale", C.c_float)]


def qmoe_attn_workspace_bytes(shape: AttnShape) -> int:
    return int(_lib.qmoe_attn_workspace_bytes(C.byref(shape)))


def qmoe_attn_decode(shape: AttnShape, q, k, v, pos: int, k_cache, v_cache, out, ws,
                     stream=None) -> None:
    _check("qmoe_attn_decode", _lib.qmoe_attn_decode(
        C.byref(shape), _ptr(q), _ptr(k), _ptr(v), int(pos), _ptr(k_cache), _ptr(v_cache),
        _ptr(out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def qmoe_attn_workspace_status(ws, n_kv_heads: int, stream=None) -> int:
    """The attention workspace's error word (0: every merge completed).  A
    nonzero word raises QmoeError after the workspace has been zeroed."""
    code = C.c_int32(0)
    _check("qmoe_attn_workspace_status", _lib.qmoe_attn_workspace_status(
        _ptr(ws), ws.numel() * ws.element_size(), int(n_kv_heads), C.byref(code),
        _stream(stream)))
    return int(code.value)


def qmoe_tiled4_bytes(rows: int, cols: int) -> int:
    return int(_lib.qmoe_tiled4_bytes(rows, cols))


def qmoe_repack_tiled4(q, scales, biases, rows: int, cols: int):
    """Host-side repack (numpy arrays in, a uint8 numpy array out): codes
    uint8 [rows][cols/2], scales and biases fp16 bits (uint16) [rows][cols/64]."""
    import numpy as np

    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    b = np.ascontiguousarray(biases, dtype=np.uint16)
    n = qmoe_tiled4_bytes(rows, cols)
    if n == 0:
        raise QmoeError("qmoe_tiled4_bytes", 2)
    out = np.empty(n, dtype=np.uint8)
    _check("qmoe_repack_tiled4", _lib.qmoe_repack_tiled4(
        q.ctypes.data, s.ctypes.data, b.ctypes.data, rows, cols, out.ctypes.data, n))
    return out


def qmoe_gemv_tiled4(tiled, rows: int, cols: int, x, y, row_blocks_per_wave: int = 0,
                     stream=None) -> None:
    _check("qmoe_gemv_tiled4", _lib.qmoe_gemv_tiled4(_ptr(tiled), rows, cols, _ptr(x), _ptr(y),
                                                      row_blocks_per_wave, _stream(stream)))


def qmoe_router_topk(Wr: QTensor, logit_bias, x, T: int, top_k: int, idx, w, logits, ws,
                     stream=None) -> None:
    qt = Wr.c()
    _check("qmoe_router_topk", _lib.qmoe_router_topk(
        C.byref(qt), _ptr(logit_bias), _ptr(x), T, top_k, _ptr(idx), _ptr(w), _ptr(logits),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def qmoe_expert_ffn(layer: MoeLayer, h, idx, w, expert_slot, residual, out, ws,
                    stream=None) -> None:
    _check("qmoe_expert_ffn", _lib.qmoe_expert_ffn(
        C.byref(layer.c()), _ptr(h), _ptr(idx), _ptr(w), _ptr(expert_slot), _ptr(residual),
        _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def qmoe_expert_ffn_shared(layer: MoeLayer, h, ws, stream=None) -> None:
    _check("qmoe_expert_ffn_shared", _lib.qmoe_expert_ffn_shared(
        C.byref(layer.c()), _ptr(h), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def qmoe_expert_ffn_routed(layer: MoeLayer, h, idx, w, expert_slot, residual, out, ws,
                           stream=None) -> None:
    _check("qmoe_expert_ffn_routed", _lib.qmoe_expert_ffn_routed(
        C.byref(layer.c()), _ptr(h), _ptr(idx), _ptr(w), _ptr(expert_slot), _ptr(residual),
        _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


class Pool:
    """The host-resident expert pool (qmoe_pool_*).  ``host_blobs``: one
    pinned host address per (layer, expert), layer-major; ``arenas``: one
    device address per layer (``slots`` blobs each).  Both None: a
    planning-only pool; ``arenas`` alone: a file-backed pool (filled by
    acquire_file)."""

    def __init__(self, layers: int, experts: int, slots: int, blob_bytes: int,
                 host_blobs=None, arenas=None):
        self.layers, self.experts, self.slots = layers, experts, slots
        hb = ar = None
        if host_blobs is not None:
            self._hb = (_vp * (layers * experts))(*host_blobs)
            hb = self._hb
        if arenas is not None:
            self._ar = (_vp * layers)(*arenas)
            ar = self._ar
        h = _vp()
        _check("qmoe_pool_create", _lib.qmoe_pool_create(layers, experts, slots, blob_bytes,
                                                          hb, ar, C.byref(h)))
        self._h = h

    def plan(self, layer: int, idx):
        import numpy as np

        idx = np.ascontiguousarray(idx, dtype=np.int32)
        k = idx.shape[0]
        slot = np.zeros(k, np.int32)
        hit = np.zeros(k, np.int32)
        victim = np.zeros(k, np.int32)
        _check("qmoe_pool_plan", _lib.qmoe_pool_plan(
            self._h, layer, idx.ctypes.data, k, slot.ctypes.data, hit.ctypes.data,
            victim.ctypes.data))
        return slot, hit, victim

    def acquire(self, layer: int, host_idx_ptr: int, k: int, dev_expert_slot, copy_stream,
                ready_event: int) -> PoolStats:
        st = PoolStats()
        _check("qmoe_pool_acquire", _lib.qmoe_pool_acquire(
            self._h, layer, host_idx_ptr, k, _ptr(dev_expert_slot), _stream(copy_stream),
            ready_event, C.byref(st)))
        return st

    def acquire_file(self, tier: "FileTier", layer: int, host_idx_ptr: int, k: int,
                     dev_expert_slot, copy_stream, ready_event: int) -> PoolStats:
        st = PoolStats()
        _check("qmoe_pool_acquire_file", _lib.qmoe_pool_acquire_file(
            self._h, tier._h, layer, host_idx_ptr, k, _ptr(dev_expert_slot),
            _stream(copy_stream), ready_event, C.byref(st)))
        return st

    def stats(self) -> PoolStats:
        st = PoolStats()
        _check("qmoe_pool_stats_get", _lib.qmoe_pool_stats_get(self._h, C.byref(st)))
        return st

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.qmoe_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


class FileTier:
    """The file-backed expert tier (qmoe_file_tier_*): blobs of an
    expert-major file, read by ``threads`` workers into pinned staging."""

    def __init__(self, path: str, layers: int, experts: int, blob_bytes: int, stride: int,
                 threads: int = 8, max_misses: int = 8, direct: bool = False):
        h = _vp()
        _check("qmoe_file_tier_open", _lib.qmoe_file_tier_open(
            path.encode(), layers, experts, blob_bytes, stride, threads, max_misses,
            1 if direct else 0, C.byref(h)))
        self._h = h

    def stats(self) -> FileTierStats:
        st = FileTierStats()
        _check("qmoe_file_tier_stats_get", _lib.qmoe_file_tier_stats_get(self._h, C.byref(st)))
        return st

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.qmoe_file_tier_close(self._h)
            self._h = None

    def __del__(self):
        self.close()


def qmoe_moe_decode(layer: MoeLayer, x, expert_slot, residual: bool, out, idx_out, w_out, ws,
                    stream=None, phased: bool = False) -> None:
    fn = _lib.qmoe_moe_decode_phased if phased else _lib.qmoe_moe_decode
    _check("qmoe_moe_decode", fn(
        C.byref(layer.c()), _ptr(x), _ptr(expert_slot), int(bool(residual)), _ptr(out),
        _ptr(idx_out), _ptr(w_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def qmoe_moe_decode_noalloc(layer: MoeLayer, x, expert_slot, residual: bool, out, idx_out,
                            w_out, stream=None) -> None:
    """qmoe_moe_decode with the library's own per-GPU workspace (no
    allocation; calls on one GPU must not overlap)."""
    _check("qmoe_moe_decode_noalloc", _lib.qmoe_moe_decode_noalloc(
        C.byref(layer.c()), _ptr(x), _ptr(expert_slot), int(bool(residual)), _ptr(out),
        _ptr(idx_out), _ptr(w_out), _stream(stream)))


def qmoe_moe_decode_timed(layer: MoeLayer, x, expert_slot, residual: bool, out, idx_out, w_out,
                          ws, ev_start, ev_stop, stream=None) -> None:
    """qmoe_moe_decode whose launch records two HIP events (raw handles, e.g.
    ``torch.cuda.Event.cuda_event``) at its kernel's start and end."""
    _check("qmoe_moe_decode_timed", _lib.qmoe_moe_decode_timed(
        C.byref(layer.c()), _ptr(x), _ptr(expert_slot), int(bool(residual)), _ptr(out),
        _ptr(idx_out), _ptr(w_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
        ev_start, ev_stop))


def qmoe_prefill_grouped(layer: MoeLayer, X, T: int, idx, w, residual, out, ws,
                         stream=None) -> None:
    _check("qmoe_prefill_grouped", _lib.qmoe_prefill_grouped(
        C.byref(layer.c()), _ptr(X), T, _ptr(idx), _ptr(w), _ptr(residual), _ptr(out),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def qmoe_prefill_dispatch_offsets(layer: MoeLayer, T: int):
    """Byte offsets (counts, offsets, perm) of the dispatch arrays that the last
    qmoe_prefill_grouped call for T tokens wrote into its workspace."""
    c, o, p = C.c_size_t(0), C.c_size_t(0), C.c_size_t(0)
    _check("qmoe_prefill_dispatch_offsets", _lib.qmoe_prefill_dispatch_offsets(
        C.byref(layer.c()), T, C.byref(c), C.byref(o), C.byref(p)))
    return int(c.value), int(o.value), int(p.value)


def qmoe_rmsnorm(x, gamma, eps: float, T: int, H: int, out, stream=None) -> None:
    _check("qmoe_rmsnorm", _lib.qmoe_rmsnorm(_ptr(x), _ptr(gamma), float(eps), T, H, _ptr(out),
                                             _stream(stream)))


def qmoe_stack_table_bytes(n_layers: int) -> int:
    return int(_lib.qmoe_stack_table_bytes(n_layers))


def qmoe_stack_table_init(layers, table, stream=None) -> None:
    """Device layer table of ``layers`` (MoeLayer list, one shape) into the
    uint8 device tensor ``table``; waits for the copy."""
    arr = (_Layer * len(layers))(*[l.c() for l in layers])
    _check("qmoe_stack_table_init", _lib.qmoe_stack_table_init(
        arr, len(layers), _ptr(table), table.numel() * table.element_size(), _stream(stream)))


def qmoe_stack_workspace_bytes(layer: MoeLayer) -> int:
    return int(_lib.qmoe_stack_workspace_bytes(C.byref(layer.c())))


def qmoe_stack_decode(shape: MoeLayer, table, n_layers: int, x, out, layer_out, idx_out, w_out,
                      ws, stream=None) -> None:
    _check("qmoe_stack_decode", _lib.qmoe_stack_decode(
        C.byref(shape.c()), _ptr(table), n_layers, _ptr(x), _ptr(out), _ptr(layer_out),
        _ptr(idx_out), _ptr(w_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


class Stack:
    """A decode stack on the device: the layers (kept alive), their device
    table and a workspace for qmoe_stack_decode."""

    def __init__(self, layers, device="cuda"):
        import torch

        self.layers = list(layers)
        self.shape = self.layers[0]
        n = qmoe_stack_table_bytes(len(self.layers))
        if n == 0:
            raise QmoeError("qmoe_stack_table_bytes", 2)
        self.table = torch.zeros(n, dtype=torch.uint8, device=device)
        qmoe_stack_table_init(self.layers, self.table)
        wsn = qmoe_stack_workspace_bytes(self.shape)
        if wsn == 0:
            raise QmoeError("qmoe_stack_workspace_bytes", 2)
        self.ws = torch.zeros(wsn, dtype=torch.uint8, device=device)

    def decode(self, x, out, layer_out=None, idx_out=None, w_out=None, n_layers=None,
               stream=None) -> None:
        qmoe_stack_decode(self.shape, self.table,
                          len(self.layers) if n_layers is None else n_layers, x, out,
                          layer_out, idx_out, w_out, self.ws, stream)


def qmoe_workspace_status(ws, stream=None) -> int:
    """Device error word of a workspace (0 = every in-kernel wait completed);
    synchronises the stream and clears the word."""
    code = C.c_int32(0)
    rc = _lib.qmoe_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), C.byref(code),
                                    _stream(stream))
    if rc not in (QMOE_OK, 7):
        _check("qmoe_workspace_status", rc)
    return int(code.value)


def qmoe_workspace_tag_counter(ws, stream=None) -> int:
    """The workspace's tag counter (synchronises the stream)."""
    v = C.c_uint32(0)
    _check("qmoe_workspace_tag_counter",
           _lib.qmoe_workspace_tag_counter(_ptr(ws), ws.numel() * ws.element_size(), C.byref(v),
                                           _stream(stream)))
    return int(v.value)


def qmoe_workspace_raise_tag_counter(ws, value: int, stream=None) -> None:
    """Test hook: raise the workspace's tag counter to `value`."""
    _check("qmoe_workspace_raise_tag_counter",
           _lib.qmoe_workspace_raise_tag_counter(_ptr(ws), ws.numel() * ws.element_size(),
                                                 int(value), _stream(stream)))


__all__ = [
    "QTensor", "MoeLayer", "QmoeError", "lib", "LIB_PATH",
    "qmoe_gemv_affine4", "qmoe_router_topk", "qmoe_expert_ffn", "qmoe_moe_decode",
    "qmoe_moe_decode_timed", "qmoe_moe_decode_noalloc", "qmoe_expert_ffn_shared", "qmoe_expert_ffn_routed", "Pool",
    "PoolStats", "qmoe_prefill_grouped", "qmoe_prefill_dispatch_offsets",
    "qmoe_rmsnorm",
    "qmoe_workspace_bytes",
    "qmoe_router_workspace_bytes", "qmoe_workspace_status", "qmoe_workspace_tag_counter",
    "qmoe_workspace_raise_tag_counter",
    "qmoe_stack_table_bytes", "qmoe_stack_table_init", "qmoe_stack_workspace_bytes",
    "qmoe_stack_decode", "Stack",
]
