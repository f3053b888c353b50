"""Pins of the fp64 oracle against things other than itself.

Each test fixes one oracle function with a closed form, a special case, an
invariant, a library routine (numpy / torch / scipy) or a hand-worked
fixture, chosen so that a plausible slip (a wrong shift, a dropped bias, a
transposed index, a sign) fails at least one of them.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ number formats
def test_half_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_encode_round_trips_every_finite_value():
    L = oracle.lib()
    for b in range(0, 65536, 7):
        v = L.orc_bf16_to_double(b)
        if math.isnan(v):
            continue
        assert L.orc_double_to_bf16(v) == b


def _nearest_bf16_exact(x: float) -> int:
    """Brute force: among all finite bf16 values of x's sign, the nearest in
    exact rational arithmetic, ties to the even bit pattern."""
    L = oracle.lib()
    fx = Fraction(x)
    # candidate neighbourhood: torch's conversion (via float) is within 1 ulp
    t = int(torch.tensor([x], dtype=torch.float64).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    cands = [c & 0xFFFF for c in (t - 1, t, t + 1) if 0 <= (c & 0x7FFF) < 0x7F80]
    best = None
    for c in cands:
        v = L.orc_bf16_to_double(c)
        d = abs(Fraction(v) - fx)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_bf16_encode_is_nearest_ties_to_even():
    rng = np.random.default_rng(11)
    xs = list(rng.normal(0, 1, 400)) + list(rng.normal(0, 1e-3, 100)) + list(rng.normal(0, 1e4, 100))
    # exact midpoints between neighbours: must go to the even pattern
    L = oracle.lib()
    for b in (0x3F80, 0x3F81, 0x4000, 0x4001, 0x0001, 0x7F00):
        lo, hi = L.orc_bf16_to_double(b), L.orc_bf16_to_double(b + 1)
        xs.append((lo + hi) / 2)
        xs.append(-(lo + hi) / 2)
    for x in xs:
        assert oracle.double_to_bf16(float(x)) == _nearest_bf16_exact(float(x)), x


# --------------------------------------------------------------- unpacking
def test_unpack_hand_words():
    q = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    assert list(oracle.unpack(q, 1, 16, 4)[0]) == list(range(16))
    q8 = np.array([[0x03020100, 0xFFFE8180]], dtype=np.uint32)
    assert list(oracle.unpack(q8, 1, 8, 8)[0]) == [0, 1, 2, 3, 0x80, 0x81, 0xFE, 0xFF]


def _bytes_unpack(q: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Independent route: little-endian byte view, low nibble first."""
    by = np.ascontiguousarray(q).view(np.uint8).reshape(rows, -1)
    if bits == 8:
        return by[:, :cols].copy()
    out = np.empty((rows, by.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = by & 0xF
    out[:, 1::2] = by >> 4
    return out[:, :cols]


@pytest.mark.parametrize("bits", [4, 8])
def test_unpack_matches_byte_view(bits):
    m = synth.random_qmat(5, 192, bits, 3)
    assert np.array_equal(oracle.unpack(m.q, 5, 192, bits), _bytes_unpack(m.q, 5, 192, bits))


# ---------------------------------------------------------------- dequant
def _numpy_dequant(m) -> np.ndarray:
    codes = _bytes_unpack(m.q, m.rows, m.cols, m.bits).astype(np.float64)
    s = np.repeat(m.s.view(np.float16).astype(np.float64), 64, axis=1)
    b = np.repeat(m.b.view(np.float16).astype(np.float64), 64, axis=1)
    return s * codes + b


@pytest.mark.parametrize("bits", [4, 8])
def test_dequant_closed_form(bits):
    m = synth.random_qmat(7, 256, bits, 5)
    assert np.array_equal(oracle.dequant(m), _numpy_dequant(m))


def test_dequant_unit_scale_zero_bias_gives_codes():
    m = synth.random_qmat(3, 128, 4, 6)
    m.s[:] = np.float16(1.0).view(np.uint16)
    m.b[:] = 0
    assert np.array_equal(oracle.dequant(m), _bytes_unpack(m.q, 3, 128, 4).astype(np.float64))


def test_gemv_one_hot_column_and_group_sum():
    m = synth.random_qmat(6, 256, 4, 8)
    W = _numpy_dequant(m)
    for j in (0, 1, 7, 8, 63, 64, 200, 255):
        x = np.zeros(256)
        x[j] = 1.0
        assert np.array_equal(oracle.qgemv(m, x), W[:, j])
    # all-ones over group 2: s*sum(q) + 64*bias, exactly
    x = np.zeros(256)
    x[128:192] = 1.0
    codes = _bytes_unpack(m.q, 6, 256, 4).astype(np.float64)
    s = m.s.view(np.float16).astype(np.float64)[:, 2]
    b = m.b.view(np.float16).astype(np.float64)[:, 2]
    assert np.array_equal(oracle.qgemv(m, x), s * codes[:, 128:192].sum(1) + 64 * b)


@pytest.mark.parametrize("bits", [4, 8])
def test_gemv_matches_numpy_matmul(bits):
    m = synth.random_qmat(33, 512, bits, 9)
    x = np.random.default_rng(1).normal(size=512)
    ref = _numpy_dequant(m) @ x
    got = oracle.qgemv(m, x)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(_numpy_dequant(m)) @ np.abs(x))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    H = 256
    gamma = synth.random_bf16(H, 4, std=0.02)
    gamma = synth.to_bf16_bits(1.0 + synth.bf16_bits_to_f32(gamma).astype(np.float64))
    for c in (0.75, -3.0, 1e-4):
        x = synth.to_bf16_bits(np.full(H, c))
        cb = oracle.bf16_to_double(int(x[0]))
        g = np.array([oracle.bf16_to_double(int(v)) for v in gamma])
        exp = [oracle.double_to_bf16(cb * gi / math.sqrt(cb * cb + 1e-6)) for gi in g]
        assert list(oracle.rmsnorm(x, gamma)) == exp


def test_rmsnorm_matches_torch_fp64():
    H = 512
    x = synth.random_bf16(H, 12)
    gamma = synth.to_bf16_bits(np.random.default_rng(2).normal(1, 0.02, H))
    xd = torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64))
    gd = torch.from_numpy(synth.bf16_bits_to_f32(gamma).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xd, (H,), gd, eps=1e-6).numpy()
    exp = [oracle.double_to_bf16(v) for v in ref]
    assert list(oracle.rmsnorm(x, gamma)) == exp


# ------------------------------------------------------------------- GELU
def test_gelu_identities_and_torch():
    assert oracle.gelu_tanh(0.0) == 0.0
    for z in (0.1, 0.5, 1.0, 2.5, 7.0):
        assert abs(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z) - z) <= 1e-15 * max(1, z)
    assert abs(oracle.gelu_tanh(40.0) / 40.0 - 1.0) < 1e-15
    zs = np.linspace(-8, 8, 257)
    ref = torch.nn.functional.gelu(torch.from_numpy(zs), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(z) for z in zs])
    assert np.max(np.abs(got - ref)) < 1e-14


# ---------------------------------------------------------------- routing
def test_topk_matches_stable_argsort_and_scipy_softmax():
    from scipy.special import softmax

    rng = np.random.default_rng(3)
    for trial in range(20):
        lg = np.round(rng.normal(0, 50, 128), 0 if trial % 2 else 6)  # rounding makes ties
        idx, w = oracle.topk_softmax(lg, 8)
        ref_idx = np.argsort(-lg, kind="stable")[:8]
        assert list(idx) == list(ref_idx)
        assert np.allclose(w, softmax(lg[ref_idx]), rtol=1e-14, atol=1e-300)
        assert abs(w.sum() - 1.0) <= 32 * 2.0**-53
        assert np.all(np.diff(w) <= 0)


def test_topk_ties_and_full_softmax():
    from scipy.special import softmax

    idx, w = oracle.topk_softmax(np.full(32, 3.5), 8)
    assert list(idx) == list(range(8))
    assert np.all(w == 0.125)
    lg = np.random.default_rng(4).normal(0, 2, 16)
    idx, w = oracle.topk_softmax(lg, 16)
    assert np.allclose(w, softmax(lg)[idx], rtol=1e-14)
    lg = np.zeros(10)
    lg[7] = lg[3] = 1.0
    idx, _ = oracle.topk_softmax(lg, 3)
    assert list(idx) == [3, 7, 0]


# ------------------------------------------------------------- FFN, layer
def _np_ffn(g, u, d, hd):
    gv = _numpy_dequant(g) @ hd
    uv = _numpy_dequant(u) @ hd
    a = torch.nn.functional.gelu(torch.from_numpy(gv), approximate="tanh").numpy() * uv
    return _numpy_dequant(d) @ a


TINY = synth.Workload(90, "pin_tiny", 128, 6, 3, 64, 128)


def test_expert_ffn_matches_numpy_brute_force():
    lw = synth.make_layer(TINY)
    g, u, d = lw.expert(2)
    h = synth.random_bf16(128, 5)
    hd = synth.bf16_bits_to_f32(h).astype(np.float64)
    ref = _np_ffn(g, u, d, hd)
    got = oracle.expert_ffn(g, u, d, h)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


@pytest.mark.parametrize("residual", [False, True])
def test_layer_forward_matches_numpy_brute_force(residual):
    from scipy.special import softmax

    lw = synth.make_layer(TINY)
    L = oracle.OracleLayer(lw)
    x = synth.random_bf16(128, 6)
    r = L.forward(x, residual=residual)
    hd = synth.bf16_bits_to_f32(x).astype(np.float64)
    logits = _numpy_dequant(lw.router) @ hd
    assert np.allclose(r["logits"], logits, rtol=1e-12, atol=1e-12 * np.abs(logits).max())
    idx = np.argsort(-logits, kind="stable")[:3]
    assert list(r["idx"]) == list(idx)
    w = softmax(logits[idx])
    y = _np_ffn(lw.sh_gate, lw.sh_up, lw.sh_down, hd)
    for j, e in enumerate(idx):
        y = y + w[j] * _np_ffn(*lw.expert(e), hd)
    if residual:
        y = y + hd
    assert np.allclose(r["y"], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())
    assert list(r["out"]) == [oracle.double_to_bf16(v) for v in r["y"]]


def test_router_logit_bias_enters_once_with_its_sign():
    """logits_e = sum_c Wr[e][c] h_c + beta_e: against a numpy dequant matmul
    plus beta, with beta large enough to change the routing, so that a
    dropped, negated or rescaled bias term fails; the layer's routing and
    weights follow the biased logits."""
    from scipy.special import softmax

    lw = synth.make_layer(TINY)
    beta = np.random.default_rng(11).normal(0, 40, TINY.n_experts).astype(np.float32)
    h = synth.random_bf16(128, 12)
    hd = synth.bf16_bits_to_f32(h).astype(np.float64)
    plain = _numpy_dequant(lw.router) @ hd
    ref = plain + beta.astype(np.float64)
    L = oracle.OracleLayer(lw, logit_bias=beta)
    got = L.router_logits(h)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert not np.allclose(got, plain - beta, rtol=1e-6)
    assert not np.allclose(got, plain + 2 * beta.astype(np.float64), rtol=1e-6)
    unbiased = oracle.OracleLayer(lw, use_prior=False).router_logits(h)
    assert np.allclose(got - unbiased, beta.astype(np.float64), rtol=0, atol=1e-12 * np.abs(ref).max())
    r = L.forward(h)
    idx = np.argsort(-ref, kind="stable")[:TINY.top_k]
    assert list(r["idx"]) == list(idx)
    assert list(idx) != list(np.argsort(-plain, kind="stable")[:TINY.top_k])
    assert np.allclose(r["w"], softmax(ref[idx]), rtol=1e-12)
    assert np.allclose(r["logits"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layer_zero_input_gives_zero():
    lw = synth.make_layer(TINY)
    r = oracle.OracleLayer(lw).forward(np.zeros(128, dtype=np.uint16), residual=True)
    assert np.all(r["out"] == 0)


def test_layer_forced_one_hot_with_zero_shared_is_single_expert():
    lw = synth.make_layer(TINY)
    for m in (lw.sh_gate, lw.sh_up, lw.sh_down):
        m.s[:] = 0
        m.b[:] = 0
    x = synth.random_bf16(128, 7)
    r = oracle.OracleLayer(lw).forward(x, force_idx=[4, 1, 0], force_w=[1.0, 0.0, 0.0])
    assert np.array_equal(r["y"], oracle.expert_ffn(*lw.expert(4), x))


def test_layer_relabelling_invariance():
    lw = synth.make_layer(TINY)
    lw.prior = np.random.default_rng(8).normal(0, 30, TINY.n_experts).astype(np.float32)
    x = synth.random_bf16(128, 8)
    ref = oracle.OracleLayer(lw).forward(x)
    perm = np.array([3, 5, 0, 1, 4, 2])  # new expert p holds old expert perm[p]
    lw2 = synth.make_layer(TINY)
    lw2.blobs = lw.blobs[perm].copy()
    for a in ("q", "s", "b"):
        setattr(lw2.router, a, getattr(lw.router, a)[perm].copy())
    lw2.prior = lw.prior[perm].copy()
    got = oracle.OracleLayer(lw2).forward(x)
    assert np.array_equal(got["out"], ref["out"])
    assert list(perm[got["idx"]]) == list(ref["idx"])


# ----------------------------------------------------------- dispatch, LFU
def test_dispatch_matches_stable_sort():
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(16, 4, replace=False) for _ in range(37)]).astype(np.int32)
    counts, offsets, perm = oracle.dispatch(idx, 16)
    assert counts.sum() == idx.size
    assert np.array_equal(counts, np.bincount(idx.reshape(-1), minlength=16))
    assert np.array_equal(offsets[1:], np.cumsum(counts))
    assert np.array_equal(perm, np.argsort(idx.reshape(-1), kind="stable"))


def test_lfu_hand_trace():
    with open(os.path.join(GOLDEN, "lfu_hand_trace.json")) as f:
        g = json.load(f)
    r = oracle.lfu_replay(np.array(g["need"]), g["n_experts"], g["slots"])
    assert r["hits"] == g["hits"]
    assert r["hit"].tolist() == g["hit"]
    assert r["slot"].tolist() == g["slot"]
    assert r["victim"].tolist() == g["victim"]


def test_lfu_invariants():
    rng = np.random.default_rng(10)
    need = np.stack([rng.choice(40, 8, replace=False) for _ in range(300)]).astype(np.int32)
    r = oracle.lfu_replay(need, 40, 16)
    # every needed expert sits in a distinct slot after its step
    for t in range(300):
        assert len(set(r["slot"][t])) == 8
    # an expert that hit was not evicted since its last use; evictions only on misses
    assert np.all(r["victim"][r["hit"] == 1] == -1)
    # with as many slots as experts nothing is ever evicted
    r2 = oracle.lfu_replay(need, 40, 40)
    assert np.all(r2["victim"] == -1)
    assert r2["hits"] == need.size - len(np.unique(need))
