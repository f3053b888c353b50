"""Pins of the oracle's sampling step against closed forms: the
defaults of the pages (elsolitario.org, TurboFieldfare article, section
"Cómo empezar": temperature 0.2, top-K 64, top-P 0.95; temperature 0 is
deterministic) and cases whose answer follows from the definition alone.
Each case fails under a plausible slip: a missing temperature, the wrong
side of a boundary in the top-P cut or in the draw, ties to the higher id."""
import math

import numpy as np
import pytest

import oracle


def test_temperature_zero_and_top_k_one_are_argmax():
    rng = np.random.default_rng(1)
    lg = rng.normal(0, 3, 5000).astype(np.float32)
    lg[4321] = lg.max() + 1.0
    for u in (0.0, 0.3, 0.999):
        assert oracle.sample(lg, 0.0, 64, 0.95, u)["token"] == 4321
        assert oracle.sample(lg, 0.2, 1, 0.95, u)["token"] == 4321


def test_ties_rank_the_lower_id_first():
    lg = np.array([1, 5, 5, 3, 5], dtype=np.float32)
    r = oracle.sample(lg, 0.0, 4, 1.0, 0.5)
    assert list(r["ranked"]) == [1, 2, 4, 3]


def test_uniform_logits_closed_form():
    """All logits equal: p = 1 for each kept rank, ranks in id order; the
    cut keeps ceil(top_p K) ranks (mass before rank r is r); the draw picks
    rank floor(u m)."""
    lg = np.full(1000, 0.25, dtype=np.float32)
    K, P = 64, 0.95
    m = math.ceil(P * K)  # 61
    for u in (0.0, 0.013, 0.5, 0.74, 0.9999):
        r = oracle.sample(lg, 0.2, K, P, u)
        assert r["kept"] == m
        assert r["token"] == math.floor(u * m)
        assert list(r["ranked"]) == list(range(K))


def test_top_p_boundary_is_strict_and_draw_boundary_is_strict():
    """Four equal logits, top-P 0.5: mass before ranks 0..3 is 0, 1, 2, 3 of
    4, so ranks 0 and 1 are kept (2 is not below 2).  u = 0.5 targets a
    cumulative mass of exactly 1, which rank 0 does not exceed: rank 1."""
    lg = np.zeros(4, dtype=np.float32)
    r = oracle.sample(lg, 1.0, 4, 0.5, 0.5)
    assert r["kept"] == 2 and r["token"] == 1
    assert oracle.sample(lg, 1.0, 4, 0.5, 0.4999)["token"] == 0


def test_temperature_scales_the_logits():
    """Logits T ln(w) for w = 1, 2, 3, 4 give masses 0.1 .. 0.4 at
    temperature T: ranked 4, 3, 2, 1 with cumulative 0.4, 0.7, 0.9, 1.0."""
    T = 0.2
    w = np.array([1.0, 2.0, 3.0, 4.0])
    lg = (T * np.log(w)).astype(np.float32)
    r = oracle.sample(lg, T, 4, 1.0, 0.0)
    assert list(r["ranked"]) == [3, 2, 1, 0]
    assert np.allclose(r["cum"], [0.4, 0.7, 0.9, 1.0], atol=1e-6)
    for u, tok in ((0.05, 3), (0.39, 3), (0.41, 2), (0.69, 2), (0.71, 1), (0.95, 0)):
        assert oracle.sample(lg, T, 4, 1.0, u)["token"] == tok
    # the same logits read at temperature 1 are a different distribution
    r1 = oracle.sample(lg, 1.0, 4, 1.0, 0.0)
    assert not np.allclose(r1["cum"], r["cum"], atol=1e-3)


def test_top_p_cut_renormalises():
    """Masses 0.4, 0.3, 0.2, 0.1 and top-P 0.65: ranks 0 and 1 kept (mass
    0.7); u = 0.6 targets 0.42 > 0.4, so rank 1; u = 0.5 targets 0.35."""
    T = 0.2
    lg = (T * np.log(np.array([1.0, 2.0, 3.0, 4.0]))).astype(np.float32)
    r = oracle.sample(lg, T, 4, 0.65, 0.6)
    assert r["kept"] == 2 and r["token"] == 2
    assert oracle.sample(lg, T, 4, 0.65, 0.5)["token"] == 3


def test_two_tokens_probability():
    """Two tokens: the higher one is drawn for u below 1/(1+exp(-d/T))."""
    a, b, T = 1.5, 1.1, 0.2
    lg = np.array([b, a], dtype=np.float32)
    p_hi = 1.0 / (1.0 + math.exp((float(np.float32(b)) - float(np.float32(a))) / T))
    assert oracle.sample(lg, T, 2, 1.0, p_hi - 1e-9)["token"] == 1
    assert oracle.sample(lg, T, 2, 1.0, p_hi + 1e-9)["token"] == 0
