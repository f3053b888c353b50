"""Seeded synthetic inputs for the quantized MoE FFN step.

This module is the one place both sides of every parity check draw their
inputs from: the HIP library (through ``bit_quantized_gemv_amd``) and the
fp64 CPU oracle (``oracle/``).  It holds none of the method's arithmetic:
no unpacking, no dequantization, no GEMV, no routing.  It only draws random
numbers, rounds them to the storage types (fp16 / bf16 through numpy and
torch conversions) and lays the bytes out in the storage format.

Storage format (MLX-style affine quantization, group size 64, as the pages
describe it: remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…",
section "L'affermazione dei 2 GB trasforma la larghezza di banda dell'SSD nel
nuovo vincolo"; elsolitario.org, section "Detalles técnicos y rendimiento"):

* a matrix ``W[rows][cols]`` is stored as codes ``q`` packed LSB-first along
  the column (input) axis into uint32 words -- 8 codes per word for 4-bit,
  4 for 8-bit -- rows contiguous, plus one fp16 scale and one fp16 bias per
  row and per group of 64 consecutive columns: ``s, bias: fp16[rows][cols/64]``.
* Because codes are uniform over ``0..2^b-1`` and packed without gaps, a
  uniformly random uint32 word *is* 8 (or 4) independent uniform codes, so
  the generator draws whole words and never packs anything.
* A routed expert is one contiguous blob (gate.q, up.q, down.q, then the six
  fp16 scale/bias arrays), each part at a 256-byte aligned offset, so that a
  single byte stride addresses expert ``e`` in every part.

Distributions (identical for every workload): codes uniform; scales
``U(0.005, 0.02)`` rounded to fp16; biases ``fp16(-8*scale + N(0, 1e-3))``;
activations ``N(0,1)`` rounded to bf16; RMSNorm weights ``N(1, 0.02)`` in
bf16.  The 8-bit router uses the same recipe with codes ``0..255``.

Seeds: ``1000*workload_id + 10*layer + tensor_id`` with numpy PCG64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

GROUP = 64
ALIGN = 256

# tensor ids inside one layer's seed space
_TID_ROUTER, _TID_SHARED, _TID_EXPERTS, _TID_GAMMA, _TID_PRIOR = 1, 2, 3, 4, 5
_TID_TOKENS = 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload."""

    wid: int                 # seed namespace
    name: str
    hidden: int              # H
    n_experts: int           # E
    top_k: int               # k
    inter: int               # I   (routed expert intermediate)
    shared_inter: int        # I_s (shared expert intermediate)
    layers: int = 1
    tokens: int = 1          # decode steps, or rows of a prefill chunk
    rmsnorm: bool = False    # RMSNorm + residual around the FFN
    zipf: bool = False       # Zipf(s=1.1) log-prior added to router logits
    slots: int = 0           # device expert-cache slots per layer (0: resident)


WORKLOADS: Dict[str, Workload] = {
    "tiny_layer_decode": Workload(1, "tiny_layer_decode", 512, 32, 8, 256, 512),
    "layer_decode": Workload(2, "layer_decode", 2816, 128, 8, 704, 2112),
    "stack30_decode": Workload(3, "stack30_decode", 2816, 128, 8, 704, 2112,
                               layers=30, tokens=256, rmsnorm=True),
    "prefill128": Workload(4, "prefill128", 2816, 128, 8, 704, 2112,
                           tokens=128, zipf=True),
    "streaming_decode": Workload(5, "streaming_decode", 2816, 128, 8, 704, 2112,
                                 layers=30, tokens=512, rmsnorm=True, zipf=True,
                                 slots=16),
    # the first 3 layers of the streaming stack (same seeds, full shapes),
    # 16 steps: pool parity at the real sizes
    "streaming_decode_3l": Workload(5, "streaming_decode_3l", 2816, 128, 8, 704, 2112,
                                    layers=3, tokens=16, rmsnorm=True, zipf=True, slots=16),
    # small-shape version of the streaming stack, for parity tests
    "tiny_streaming_decode": Workload(6, "tiny_streaming_decode", 512, 32, 8, 256, 512,
                                      layers=3, tokens=12, rmsnorm=True, zipf=True, slots=16),
    # small stacks for parity tests of the one-launch stack decode: the
    # small shapes, and shapes with no compile-time specialisation
    "tiny_stack_decode": Workload(7, "tiny_stack_decode", 512, 32, 8, 256, 512,
                                  layers=5, tokens=3, rmsnorm=True),
    "odd_stack_decode": Workload(8, "odd_stack_decode", 1024, 64, 4, 128, 256,
                                 layers=4, tokens=2, rmsnorm=True),
    # a prefill shape whose widths are not multiples of 128 (padded operand
    # rows) and whose counts are not powers of two
    "odd_prefill": Workload(9, "odd_prefill", 576, 24, 4, 192, 320, tokens=33),
    # a decode layer whose expert count is not a multiple of the router's 8
    # rows per block (its last router block has 5 rows), with odd widths
    "odd_experts_decode": Workload(10, "odd_experts_decode", 576, 21, 4, 192, 320, tokens=3,
                                   rmsnorm=True),
    # a prefill shape wider than the GEMMs' LDS scale tables (hidden and
    # shared widths of 50 groups): the per-step scale loads
    "wide_prefill": Workload(12, "wide_prefill", 3200, 8, 2, 128, 3200, tokens=5),
    # the largest expert count the kernels take (512), narrow experts
    "max_experts_decode": Workload(11, "max_experts_decode", 512, 512, 8, 64, 128, tokens=2,
                                   rmsnorm=True),
}


def seed(wid: int, layer: int, tid: int) -> int:
    return 1000 * wid + 10 * layer + tid


# ----------------------------------------------------------------- rounding
def to_fp16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> IEEE fp16 (numpy's round-to-nearest-even), as uint16 bits."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 (torch's round-to-nearest-even), as uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen stored bf16 bits to float32 (exact; used for reporting only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------- quantized data
@dataclasses.dataclass
class QMat:
    """One quantized matrix in storage form (host arrays)."""

    q: np.ndarray   # uint32 [rows][cols*bits/32]
    s: np.ndarray   # uint16 (fp16 bits) [rows][cols/64]
    b: np.ndarray   # uint16 (fp16 bits) [rows][cols/64]
    rows: int
    cols: int
    bits: int


def draw_qmat(rng: np.random.Generator, rows: int, cols: int, bits: int) -> QMat:
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 64")
    words = cols * bits // 32
    q = rng.integers(0, 2**32, size=(rows, words), dtype=np.uint32)
    s64 = rng.uniform(0.005, 0.02, size=(rows, cols // GROUP))
    s = to_fp16_bits(s64)
    s_back = s.view(np.float16).astype(np.float64)
    b = to_fp16_bits(-8.0 * s_back + rng.normal(0.0, 1e-3, size=s64.shape))
    return QMat(q, s, b, rows, cols, bits)


def _al(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


@dataclasses.dataclass(frozen=True)
class BlobLayout:
    """Byte offsets of the parts of one routed-expert blob."""

    hidden: int
    inter: int
    offsets: Tuple[Tuple[str, int, int], ...]  # (name, offset, nbytes)
    nbytes: int

    def off(self, name: str) -> int:
        for n, o, _ in self.offsets:
            if n == name:
                return o
        raise KeyError(name)


def blob_layout(hidden: int, inter: int) -> BlobLayout:
    H, I = hidden, inter
    parts = [
        ("gate.q", I * H // 2), ("up.q", I * H // 2), ("down.q", H * I // 2),
        ("gate.s", I * (H // GROUP) * 2), ("gate.b", I * (H // GROUP) * 2),
        ("up.s", I * (H // GROUP) * 2), ("up.b", I * (H // GROUP) * 2),
        ("down.s", H * (I // GROUP) * 2), ("down.b", H * (I // GROUP) * 2),
    ]
    offs, o = [], 0
    for name, n in parts:
        offs.append((name, o, n))
        o = _al(o + n)
    return BlobLayout(H, I, tuple(offs), o)


def pack_blob(layout: BlobLayout, gate: QMat, up: QMat, down: QMat) -> np.ndarray:
    """Lay one expert's three matrices out as a blob (pure byte copying)."""
    blob = np.zeros(layout.nbytes, dtype=np.uint8)
    src = {"gate.q": gate.q, "up.q": up.q, "down.q": down.q,
           "gate.s": gate.s, "gate.b": gate.b, "up.s": up.s, "up.b": up.b,
           "down.s": down.s, "down.b": down.b}
    for name, o, n in layout.offsets:
        raw = np.ascontiguousarray(src[name]).view(np.uint8).reshape(-1)
        assert raw.size == n, (name, raw.size, n)
        blob[o:o + n] = raw
    return blob


def blob_views(layout: BlobLayout, blob: np.ndarray) -> Tuple[QMat, QMat, QMat]:
    """Typed views of the three matrices inside one blob (no copy)."""
    H, I = layout.hidden, layout.inter

    def v(name, dtype, shape):
        o = layout.off(name)
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        return blob[o:o + n].view(dtype).reshape(shape)

    g = QMat(v("gate.q", np.uint32, (I, H // 8)), v("gate.s", np.uint16, (I, H // 64)),
             v("gate.b", np.uint16, (I, H // 64)), I, H, 4)
    u = QMat(v("up.q", np.uint32, (I, H // 8)), v("up.s", np.uint16, (I, H // 64)),
             v("up.b", np.uint16, (I, H // 64)), I, H, 4)
    d = QMat(v("down.q", np.uint32, (H, I // 8)), v("down.s", np.uint16, (H, I // 64)),
             v("down.b", np.uint16, (H, I // 64)), H, I, 4)
    return g, u, d


@dataclasses.dataclass
class LayerWeights:
    """All host arrays of one MoE layer."""

    wl: Workload
    layer: int
    router: QMat                 # 8-bit [E x H]
    blobs: np.ndarray            # uint8 [E][blob_bytes]
    layout: BlobLayout
    sh_gate: QMat
    sh_up: QMat
    sh_down: QMat
    gamma: Optional[np.ndarray]  # bf16 bits [H] or None
    prior: Optional[np.ndarray]  # float32 [E] Zipf log-prior or None

    def expert(self, e: int) -> Tuple[QMat, QMat, QMat]:
        return blob_views(self.layout, self.blobs[e])

    def algorithmic_bytes_decode(self) -> int:
        """Bytes one decode token reads from this layer's weights."""
        def qb(m: QMat) -> int:
            return m.q.nbytes + m.s.nbytes + m.b.nbytes
        g, u, d = self.expert(0)
        routed = qb(g) + qb(u) + qb(d)
        return qb(self.router) + qb(self.sh_gate) + qb(self.sh_up) + qb(self.sh_down) \
            + self.wl.top_k * routed


# ------------------------------------------------------------ Zipf prior
def router_logit_spread(hidden: int, bits: int = 8) -> float:
    """Across-expert standard deviation of router logits for N(0,1) inputs.

    Closed form for the weight distribution above (not a computation of the
    method): within one group of 64 columns of expert e the weight is
    ``s_e (q - 8) + eps``, so the group's contribution to the logit is
    ``s_e Z`` with ``Z = sum (q-8) h``.  Across experts its variance is
    ``E[s^2] E[Z^2] - E[s]^2 E[Z]^2``; summed over H/64 groups with
    ``E[(sum_g h)^2] = 64``.
    """
    lo, hi = 0.005, 0.02
    es = (lo + hi) / 2
    es2 = (hi**3 - lo**3) / (3 * (hi - lo))
    n = 2**bits
    var_q = (n * n - 1) / 12.0
    mu = (n - 1) / 2.0 - 8.0
    per_group = es2 * var_q * GROUP + (es2 - es * es) * mu * mu * GROUP
    return math.sqrt(hidden // GROUP * per_group)


def zipf_prior(wl: Workload, layer: int, scale: Optional[float] = None) -> np.ndarray:
    """Per-expert log-prior ``beta_e = -1.1 * ln(rank_e) * scale``.

    Ranks are a seeded permutation of ``1..E``.  ``scale`` defaults to the
    logit spread of the router distribution, so that the prior actually
    concentrates routing (the unscaled prior, ``scale=1``, is a few nats
    against a spread of ~58 and leaves routing essentially uniform).
    """
    rng = np.random.Generator(np.random.PCG64(seed(wl.wid, layer, _TID_PRIOR)))
    ranks = rng.permutation(wl.n_experts) + 1
    if scale is None:
        scale = router_logit_spread(wl.hidden)
    return (-1.1 * np.log(ranks.astype(np.float64)) * scale).astype(np.float32)


# ---------------------------------------------------------------- builders
def make_layer(wl: Workload, layer: int = 0, *, prior_scale: Optional[float] = None,
               n_experts_materialized: Optional[int] = None) -> LayerWeights:
    """Draw one layer.  ``n_experts_materialized`` limits how many expert
    blobs are drawn (the rest are zero) for tests that touch few experts."""
    H, E, I, Is = wl.hidden, wl.n_experts, wl.inter, wl.shared_inter
    r_router = np.random.Generator(np.random.PCG64(seed(wl.wid, layer, _TID_ROUTER)))
    router = draw_qmat(r_router, E, H, 8)
    r_sh = np.random.Generator(np.random.PCG64(seed(wl.wid, layer, _TID_SHARED)))
    sh_gate = draw_qmat(r_sh, Is, H, 4)
    sh_up = draw_qmat(r_sh, Is, H, 4)
    sh_down = draw_qmat(r_sh, H, Is, 4)
    layout = blob_layout(H, I)
    blobs = np.zeros((E, layout.nbytes), dtype=np.uint8)
    r_ex = np.random.Generator(np.random.PCG64(seed(wl.wid, layer, _TID_EXPERTS)))
    nmat = E if n_experts_materialized is None else n_experts_materialized
    for e in range(nmat):
        g = draw_qmat(r_ex, I, H, 4)
        u = draw_qmat(r_ex, I, H, 4)
        d = draw_qmat(r_ex, H, I, 4)
        blobs[e] = pack_blob(layout, g, u, d)
    gamma = None
    if wl.rmsnorm:
        r_g = np.random.Generator(np.random.PCG64(seed(wl.wid, layer, _TID_GAMMA)))
        gamma = to_bf16_bits(r_g.normal(1.0, 0.02, size=H))
    prior = zipf_prior(wl, layer, prior_scale) if wl.zipf else None
    return LayerWeights(wl, layer, router, blobs, layout, sh_gate, sh_up, sh_down,
                        gamma, prior)


def make_tokens(wl: Workload, n: int, stream: int = 0) -> np.ndarray:
    """``n`` token vectors ~N(0,1) as bf16 bits, shape [n][H]."""
    rng = np.random.Generator(np.random.PCG64(seed(wl.wid, 0, _TID_TOKENS) + 100000 * stream))
    return to_bf16_bits(rng.normal(0.0, 1.0, size=(n, wl.hidden)))


def dirichlet_routing(wl: Workload, n: int, stream: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Random distinct expert ids and Dirichlet(1) combine weights, sorted by
    descending weight: drives the combine with all k experts mattering."""
    rng = np.random.Generator(np.random.PCG64(seed(wl.wid, 0, 9) + 100000 * stream))
    idx = np.zeros((n, wl.top_k), dtype=np.int32)
    w = np.zeros((n, wl.top_k), dtype=np.float32)
    for t in range(n):
        idx[t] = rng.choice(wl.n_experts, size=wl.top_k, replace=False)
        p = rng.dirichlet(np.ones(wl.top_k)).astype(np.float32)
        order = np.argsort(-p, kind="stable")
        w[t] = p[order]
        idx[t] = idx[t][order]
    return idx, w


# ------------------------------------------------------ decode attention
@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Shapes of a decode-attention workload.  The pages give the layer
    split (25 sliding-window layers, 5 full-attention layers), an FP16
    cache and a 4,096-token context; head counts, head width, window length
    and RoPE base are not on them and are stated choices."""

    wid: int
    name: str
    n_heads: int         # Hq
    n_kv_heads: int      # Hkv
    head_dim: int        # D
    window: int          # slots of a sliding-window layer's circular store
    context: int         # slots of a full layer's linear store
    sliding_layers: int
    full_layers: int
    rope_base: float = 10000.0


ATTN_WORKLOADS: Dict[str, AttnWorkload] = {
    "attn30_decode": AttnWorkload(20, "attn30_decode", 16, 8, 256, 1024, 4096, 25, 5),
    "tiny_attn": AttnWorkload(21, "tiny_attn", 4, 2, 128, 48, 160, 2, 1),
}


def attn_inputs(aw: AttnWorkload, slots: int, layer: int = 0, stream: int = 0):
    """One token's projections and a filled cache: q fp32 [Hq][D], k and v
    fp32 [Hkv][D], all N(0,1); key and value caches fp16 bits [Hkv][slots][D],
    N(0,1) in every slot (a rotated Gaussian key is again Gaussian, so the
    stored keys need no rotation of their own)."""
    rng = np.random.Generator(np.random.PCG64(seed(aw.wid, layer, 8) + 100000 * stream))
    Hq, Hkv, D = aw.n_heads, aw.n_kv_heads, aw.head_dim
    q = rng.normal(size=(Hq, D)).astype(np.float32)
    k = rng.normal(size=(Hkv, D)).astype(np.float32)
    v = rng.normal(size=(Hkv, D)).astype(np.float32)
    kc = to_fp16_bits(rng.normal(size=(Hkv, slots, D)))
    vc = to_fp16_bits(rng.normal(size=(Hkv, slots, D)))
    return q, k, v, kc, vc


def random_qmat(rows: int, cols: int, bits: int, seed_: int) -> QMat:
    return draw_qmat(np.random.Generator(np.random.PCG64(seed_)), rows, cols, bits)


def random_bf16(shape, seed_: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_))
    return to_bf16_bits(rng.normal(0.0, std, size=shape))


__all__ = [
    "GROUP", "Workload", "WORKLOADS", "QMat", "BlobLayout", "LayerWeights",
    "seed", "draw_qmat", "blob_layout", "pack_blob", "blob_views", "make_layer",
    "make_tokens", "zipf_prior", "router_logit_spread", "dirichlet_routing",
    "to_fp16_bits", "to_bf16_bits", "bf16_bits_to_f32", "random_qmat", "random_bf16",
    "AttnWorkload", "ATTN_WORKLOADS", "attn_inputs",
]
