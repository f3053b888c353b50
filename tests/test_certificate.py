"""CPU checks of the routing certificate the GPU tests use to accept a
routing difference (tests.helpers.routing_certified / routing_bound)."""
import numpy as np

import oracle
import synth
from tests.helpers import gemv8_bound, routing_bound, routing_certified


def test_certificate_without_slack_is_the_exact_ranking():
    rng = np.random.default_rng(1)
    for _ in range(50):
        lg = rng.normal(0, 50, 32)
        order = list(np.argsort(-lg, kind="stable")[:8])
        B = np.zeros(32)
        assert routing_certified(B, lg, order)
        swapped = order.copy()
        swapped[2], swapped[3] = swapped[3], swapped[2]
        assert not routing_certified(B, lg, swapped)
        outsider = order[:7] + [int(np.argsort(-lg, kind="stable")[8])]
        assert routing_certified(B, lg, outsider) is False
        assert not routing_certified(B, lg, order[:7] + [order[0]])  # repeated id


def test_certificate_accepts_swaps_within_the_bound_only():
    lg = np.array([10.0, 9.5, 3.0, 2.9, -1.0, -4.0])
    B = np.full(6, 0.06)
    assert routing_certified(B, lg, [0, 1, 3, 2])        # gap 0.1 <= 0.06 + 0.06
    assert not routing_certified(B, lg, [1, 0, 2, 3])    # gap 0.5
    assert not routing_certified(B, lg, [0, 1, 2, 4])    # 3 ranked below 4: gap 3.9
    B[2] = B[3] = 0.04
    assert not routing_certified(B, lg, [0, 1, 3, 2])    # 0.1 > 0.08


def test_bound_covers_the_gemv_bound_and_the_bias_rounding():
    wl = synth.Workload(91, "cert", 256, 16, 4, 64, 128, rmsnorm=True)
    lw = synth.make_layer(wl)
    x = synth.random_bf16(256, 3)
    L = oracle.OracleLayer(lw, use_prior=False)
    h = oracle.rmsnorm(x, lw.gamma)
    lg = L.router_logits(h)
    B0 = routing_bound(lw.router, h, lg)
    hd = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(B0, gemv8_bound(lw.router, hd) + 2 * np.abs(lg) * 2.0**-24, rtol=1e-12)
    # with the RMSNorm in front the bound can only grow
    B1 = routing_bound(lw.router, x, lg, gamma=lw.gamma)
    assert np.all(B1 >= B0 - 1e-15)
    assert np.all(np.isfinite(B1))


def test_weights_check_follows_the_logit_bounds():
    from tests.helpers import weights_consistent

    lg = np.array([4.0, 3.0, 1.0, -2.0, 0.5])
    sel = [0, 1, 4]
    w = np.exp(lg[sel] - 4.0)
    w /= w.sum()
    assert weights_consistent(np.zeros(5), lg, sel, w.astype(np.float32))
    assert not weights_consistent(np.zeros(5), lg, sel, w[::-1])
    assert not weights_consistent(np.zeros(5), lg, sel, np.full(3, 1 / 3))
    # a logit moved by 0.01 moves log-weights by at most 0.02
    w2 = np.exp(lg[sel] + np.array([0.01, -0.01, 0.0]) - 4.0)
    w2 /= w2.sum()
    assert not weights_consistent(np.zeros(5), lg, sel, w2)
    assert weights_consistent(np.full(5, 0.01), lg, sel, w2)
