"""Pins of the oracle's decode attention (orc_attn_step), its RoPE and its
fp16 encoder against facts fixed outside the oracle: every fp16 bit pattern,
numpy's own double -> float16 rounding, hand-computed rotations, the
relative-position property of RoPE, and closed forms of the softmax average
(one token, equal scores, two tokens), the window, the grouping of query
heads and the score scale.  Each one fails for a plausible slip (a wrong
rotation sign or pairing, a frequency exponent off by a factor, a window off
by one, a wrong key/value head, a missing scale)."""
import math

import numpy as np
import pytest

import oracle


def _h2f(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_half_encoder_round_trips_every_finite_pattern():
    L = oracle.lib()
    for b in range(0, 1 << 16, 7):
        if (b & 0x7C00) == 0x7C00:
            continue  # inf / nan
        v = L.orc_half_to_double(b)
        e = L.orc_double_to_half(v)
        if v == 0.0:
            assert e in (0, 0x8000)
        else:
            assert e == b, hex(b)


def test_half_encoder_matches_numpy_rounding():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 1e4, 2000),
                        rng.normal(0, 1e-5, 2000), [65504.0, 65519.9, 65520.0, 1e6, -70000.0]])
    # midpoints between neighbouring fp16 values: ties go to even
    h = np.arange(0x3C00, 0x3C40, dtype=np.uint16).view(np.float16).astype(np.float64)
    v = np.concatenate([v, (h[:-1] + h[1:]) / 2])
    got = np.array([oracle.double_to_half(x) for x in v], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).normal(size=64)
    assert np.array_equal(oracle.rope(x, 0, 10000.0), x)


def test_rope_hand_rotations():
    # D = 2: one plane at angle pos * base^0 = pos, positive sense
    r = oracle.rope(np.array([1.0, 0.0]), 1, 10000.0)
    assert np.allclose(r, [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    r = oracle.rope(np.array([0.0, 1.0]), 1, 10000.0)
    assert np.allclose(r, [-math.sin(1.0), math.cos(1.0)], rtol=0, atol=1e-15)
    # D = 4: plane (0, 2) turns by pos, plane (1, 3) by pos * base^(-1/2)
    r = oracle.rope(np.array([0.0, 1.0, 0.0, 0.0]), 3, 100.0)
    assert np.allclose(r, [0.0, math.cos(0.3), 0.0, math.sin(0.3)], rtol=0, atol=1e-15)
    r = oracle.rope(np.array([1.0, 0.0, 0.0, 0.0]), 3, 100.0)
    assert np.allclose(r, [math.cos(3.0), 0.0, math.sin(3.0), 0.0], rtol=0, atol=1e-15)


def test_rope_keeps_plane_norms_and_scores_depend_on_distance_only():
    rng = np.random.default_rng(2)
    D, base = 128, 10000.0
    q, k = rng.normal(size=D), rng.normal(size=D)
    for pos in (1, 17, 4095):
        r = oracle.rope(q, pos, base)
        assert np.allclose(r[:D // 2] ** 2 + r[D // 2:] ** 2, q[:D // 2] ** 2 + q[D // 2:] ** 2)
    a = oracle.rope(q, 100, base) @ oracle.rope(k, 40, base)
    b = oracle.rope(q, 1060, base) @ oracle.rope(k, 1000, base)
    c = oracle.rope(q, 40, base) @ oracle.rope(k, 100, base)
    assert abs(a - b) <= 1e-9 * np.abs(q).sum() * np.abs(k).sum()
    assert abs(a - c) > 1e-3  # the sign of the distance matters


def _case(rng, Hq, Hkv, D, T):
    q = rng.normal(size=(Hq, D)).astype(np.float32)
    k = rng.normal(size=(Hkv, D)).astype(np.float32)
    v = rng.normal(size=(Hkv, D)).astype(np.float32)
    kh = rng.normal(size=(T, Hkv, D)).astype(np.float16).view(np.uint16)
    vh = rng.normal(size=(T, Hkv, D)).astype(np.float16).view(np.uint16)
    return q, k, v, kh, vh


def test_first_token_returns_its_own_value_and_stores_rope_key():
    rng = np.random.default_rng(3)
    q, k, v, kh, vh = _case(rng, 4, 2, 16, 1)
    out = oracle.attn_step(q, k, v, kh, vh, 0, 0, 0.25, 10000.0)
    vv = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(out, np.repeat(vv, 2, axis=0))
    assert np.array_equal(vh[0], v.astype(np.float16).view(np.uint16))
    # position 0: RoPE is the identity, so the stored key is fp16(k)
    assert np.array_equal(kh[0], k.astype(np.float16).view(np.uint16))
    # position 5: the stored key is fp16 of the rotated key
    q, k, v, kh, vh = _case(rng, 2, 1, 8, 6)
    oracle.attn_step(q, k, v, kh, vh, 5, 0, 0.3, 50.0)
    ref = np.array([oracle.double_to_half(x) for x in oracle.rope(k[0].astype(np.float64), 5, 50.0)])
    assert np.array_equal(kh[5, 0], ref)


def test_equal_scores_average_the_values_in_the_window():
    """Zero keys and a zero current key: every score is 0, so each head's
    output is the plain mean of the values in its window."""
    rng = np.random.default_rng(4)
    Hq, Hkv, D, T = 4, 2, 8, 40
    q, k, v, kh, vh = _case(rng, Hq, Hkv, D, T)
    kh[:] = 0
    k[:] = 0
    pos = 30
    for window, t0 in ((0, 0), (8, 23), (31, 0), (1, 30)):
        khc, vhc = kh.copy(), vh.copy()
        out = oracle.attn_step(q, k, v, khc, vhc, pos, window, 0.5, 10000.0)
        vals = _h2f(vhc[t0:pos + 1])  # [n][Hkv][D], time pos included
        mean = vals.mean(axis=0)
        assert np.allclose(out, np.repeat(mean, Hq // Hkv, axis=0), rtol=1e-12, atol=1e-12)


def test_two_tokens_closed_form():
    """Two times with scores s0 and s1: out = sigma(s0 - s1) v0 + sigma(s1 - s0) v1."""
    D = 4
    q = np.array([[1.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    k = np.array([[0.0, 0.0, 0.0, 0.0]], dtype=np.float32)  # current score 0
    v = np.array([[0.0, 1.0, 0.0, 0.0]], dtype=np.float32)
    kh = np.zeros((2, 1, D), dtype=np.uint16)
    vh = np.zeros((2, 1, D), dtype=np.uint16)
    kh[0, 0] = np.array([2.0, 0.0, 0.0, 0.0], dtype=np.float16).view(np.uint16)
    vh[0, 0] = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float16).view(np.uint16)
    # q rotated at pos 1: plane (0, 2) by 1 rad, so q'.K0 = 2 cos(1)
    s0 = 0.7 * 2.0 * math.cos(1.0)
    out = oracle.attn_step(q, k, v, kh, vh, 1, 0, 0.7, 10000.0)
    w0 = 1.0 / (1.0 + math.exp(-s0))
    assert np.allclose(out[0], [w0, 1.0 - w0, 0.0, 0.0], rtol=0, atol=1e-15)


def test_window_excludes_older_times_only():
    rng = np.random.default_rng(6)
    q, k, v, kh, vh = _case(rng, 2, 1, 16, 50)
    pos, W = 45, 10
    base = oracle.attn_step(q, k, v, kh.copy(), vh.copy(), pos, W, 0.25, 1e4)
    kh2, vh2 = kh.copy(), vh.copy()
    kh2[:pos - W + 1] ^= 0x1234  # times 0..35 lie outside the window
    vh2[:pos - W + 1] ^= 0x0101
    assert np.array_equal(oracle.attn_step(q, k, v, kh2, vh2, pos, W, 0.25, 1e4), base)
    vh3 = vh.copy()
    vh3[pos - W + 1] ^= 0x0400  # time 36 is the oldest inside it
    assert not np.array_equal(oracle.attn_step(q, k, v, kh.copy(), vh3, pos, W, 0.25, 1e4), base)


def test_query_heads_use_their_group_key_value_head():
    """Value head g is constant c_g: every query head of group g returns c_g
    whatever the scores; equal queries in one group give equal outputs."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D, T = 6, 3, 8, 12
    q, k, v, kh, vh = _case(rng, Hq, Hkv, D, T)
    c = np.array([0.5, -2.0, 3.0])
    for g in range(Hkv):
        vh[:, g, :] = np.float16(c[g]).view(np.uint16)
        v[g, :] = c[g]
    q[3] = q[2]  # heads 2 and 3 share key/value head 1
    out = oracle.attn_step(q, k, v, kh, vh, 9, 0, 0.3, 1e4)
    for h in range(Hq):
        assert np.allclose(out[h], c[h // 2], rtol=1e-14, atol=0)
    assert not np.array_equal(out[2], out[4])
    vh[:, 1, :] = rng.normal(size=(T, D)).astype(np.float16).view(np.uint16)
    out = oracle.attn_step(q, k, v, kh, vh, 9, 0, 0.3, 1e4)
    assert np.array_equal(out[2], out[3])


def test_scale_multiplies_the_scores():
    rng = np.random.default_rng(8)
    q, k, v, kh, vh = _case(rng, 2, 1, 32, 20)
    a = oracle.attn_step(q, k, v, kh.copy(), vh.copy(), 19, 0, 0.5, 1e4)
    b = oracle.attn_step(q * np.float32(2.0), k, v, kh.copy(), vh.copy(), 19, 0, 0.25, 1e4)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    vc = vh.copy()
    c = oracle.attn_step(q, k, v, kh.copy(), vc, 19, 0, 0.0, 1e4)  # scale 0: equal scores
    assert np.allclose(c[0], _h2f(vc[:20, 0]).mean(axis=0), rtol=1e-12, atol=1e-12)


def test_one_dominant_score_selects_its_value():
    """A history key aligned with the rotated query and scaled up dominates
    the softmax: the output is that time's value to within e^-50."""
    rng = np.random.default_rng(9)
    D = 16
    q, k, v, kh, vh = _case(rng, 1, 1, D, 9)
    pos, t = 8, 3
    qr = oracle.rope(q[0].astype(np.float64), pos, 1e4)
    kh[t, 0] = (qr / np.linalg.norm(qr) * 8.0).astype(np.float16).view(np.uint16)
    out = oracle.attn_step(q, k, v, kh, vh, pos, 0, 100.0 / np.linalg.norm(qr), 1e4)
    assert np.allclose(out[0], _h2f(vh[t, 0]), rtol=0, atol=1e-12)


def test_bad_shapes_are_rejected():
    rng = np.random.default_rng(10)
    q, k, v, kh, vh = _case(rng, 3, 2, 8, 4)
    with pytest.raises(ValueError):
        oracle.attn_step(q, k, v, kh, vh, 2, 0, 0.3, 1e4)  # 3 heads over 2 groups
