"""GPU parity of the token sampling step (qmoe_sample) against the fp64
oracle, through the C ABI.  The kept candidates (top-K ids in rank
order) are integer work on the same fp32 logits: bit-exact.  The drawn token
is decided in fp32 on the GPU and fp64 in the oracle: equal, or the draw or
the top-P cut lies within the fp32 rounding of a cumulative mass
(certified from the oracle's own masses)."""
import numpy as np
import pytest

import oracle
from tests.helpers import log

pytestmark = pytest.mark.gpu

# fp32 sums of up to 64 terms in [0, 1], exp() and one division: a margin
# on cumulative masses (relative to the total) far above their rounding
CERT = 1e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def q():
    import bit_quantized_gemv_amd as q

    return q


def _run(torch, q, lg, T, K, P, u):
    V = lg.size
    d = torch.from_numpy(lg).cuda()
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ranked = torch.full((K,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(q.qmoe_sample_workspace_bytes(V, K), 8), dtype=torch.uint8, device="cuda")
    q.qmoe_sample(d, V, T, K, P, u, tok, ranked, ws)
    torch.cuda.synchronize()
    return int(tok.item()), ranked.cpu().numpy()


def _certified(ref, T, P, u, got):
    """The GPU's token differs from the oracle's only where an fp32 decision
    sits at a boundary: the draw target u*(kept mass) or the top-P cut
    within CERT of a cumulative mass."""
    cum, m = ref["cum"], ref["kept"]
    kept_mass = cum[m - 1]
    near_draw = np.any(np.abs(cum[:m] - u * kept_mass) <= CERT)
    near_cut = np.any(np.abs(cum - P) <= CERT)
    in_candidates = got in set(int(i) for i in ref["ranked"])
    return in_candidates and (near_draw or near_cut)


@pytest.mark.parametrize("V,K,T,P", [(262144, 64, 0.2, 0.95), (100003, 64, 0.2, 0.95),
                                     (4096, 40, 1.0, 0.9), (65, 64, 0.5, 1.0),
                                     (1 << 20, 64, 0.2, 0.95), (777, 1, 0.2, 0.95),
                                     (5000, 64, 0.0, 0.95)])
def test_sample_matches_oracle(torch_cuda, q, V, K, T, P):
    torch = torch_cuda
    rng = np.random.default_rng(V + K)
    for trial in range(4):
        lg = rng.normal(0.0, 2.0, V).astype(np.float32)
        u = float(rng.random())
        log(f"sample V={V} K={K} T={T} P={P} trial {trial} u={u:.4f}")
        tok, ranked = _run(torch, q, lg, T, K, P, u)
        ref = oracle.sample(lg, T, K, P, u)
        assert np.array_equal(ranked, ref["ranked"]), "top-K candidates differ"
        if tok != ref["token"]:
            assert _certified(ref, T, P, u, tok), (tok, ref["token"])


def test_sample_ties_and_duplicates(torch_cuda, q):
    """Many equal logits across block boundaries: ranks by lower id."""
    torch = torch_cuda
    V = 50000
    lg = np.round(np.random.default_rng(3).normal(0, 1, V), 1).astype(np.float32)
    for u in (0.1, 0.6):
        tok, ranked = _run(torch, q, lg, 0.3, 64, 0.95, u)
        ref = oracle.sample(lg, 0.3, 64, 0.95, u)
        assert np.array_equal(ranked, ref["ranked"])
        assert tok == ref["token"] or _certified(ref, 0.3, 0.95, u, tok)


def test_sample_uniform_logits_closed_form(torch_cuda, q):
    """All logits equal: exact masses (p = 1), so the GPU must match the
    closed form token = floor(u * ceil(top_p K)) exactly."""
    torch = torch_cuda
    lg = np.full(9000, -1.25, dtype=np.float32)
    for u in (0.0, 0.2, 0.51, 0.99):
        tok, ranked = _run(torch, q, lg, 0.2, 64, 0.95, u)
        assert list(ranked) == list(range(64))
        assert tok == int(np.floor(u * 61))


def test_sample_temperature_zero_is_argmax(torch_cuda, q):
    torch = torch_cuda
    lg = np.random.default_rng(9).normal(0, 1, 300000).astype(np.float32)
    lg[123457] = 50.0
    for u in (0.0, 0.5, 0.99):
        assert _run(torch, q, lg, 0.0, 64, 0.95, u)[0] == 123457


@pytest.mark.parametrize("V", [262144, 9000, 300])
def test_sample_bound_and_filter_extremes(torch_cuda, q, V):
    """Inputs that leave the most keys at or above the final block's bound:
    equal logits (every block's keys tie; the bound keeps up to K * K of
    them) and logits rising with the token id within each block of 1024
    (every block's leading keys alike)."""
    torch = torch_cuda
    for lg in (np.full(V, 0.75, dtype=np.float32),
               (np.arange(V) % 1024).astype(np.float32) * 1e-3):
        for u in (0.05, 0.7):
            tok, ranked = _run(torch, q, lg, 0.2, 64, 0.95, u)
            ref = oracle.sample(lg, 0.2, 64, 0.95, u)
            assert np.array_equal(ranked, ref["ranked"])
            assert tok == ref["token"] or _certified(ref, 0.2, 0.95, u, tok)
