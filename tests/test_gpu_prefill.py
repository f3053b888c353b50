"""GPU parity of the chunked prefill (expert dispatch, grouped dequantizing
GEMMs on the matrix cores, fixed-order combine) against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import (bf16_to_f64, log, rel_l2, routing_bound, routing_certified,
                           to_u16, weights_consistent)

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_layer_decode"]
PF = synth.WORKLOADS["prefill128"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def q():
    import bit_quantized_gemv_amd as q

    return q


@pytest.fixture(scope="module")
def tiny_layer():
    lw = synth.make_layer(TINY, 0)
    return lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)


@pytest.fixture(scope="module")
def pf_layer():
    lw = synth.make_layer(PF, 0)
    return lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)


def _dev_u16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _prefill(torch, q, L, X, idx, w, residual=False, ws=None):
    T = X.shape[0]
    ws = L.new_workspace(T) if ws is None else ws
    Xd = _dev_u16(torch, X)
    out = torch.empty(T, L.hidden, dtype=torch.int16, device="cuda")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    q.qmoe_prefill_grouped(L, Xd, T, idx_d, w_d, Xd if residual else None, out, ws)
    torch.cuda.synchronize()
    return to_u16(out), ws


def _dispatch_of(torch, q, L, T, ws):
    c, o, p = q.qmoe_prefill_dispatch_offsets(L, T)
    b = ws.cpu().numpy()
    E, K = L.n_experts, L.top_k
    counts = b[c:c + 4 * E].view(np.int32).copy()
    offsets = b[o:o + 4 * (E + 1)].view(np.int32).copy()
    perm = b[p:p + 4 * T * K].view(np.int32).copy()
    return counts, offsets, perm


def _router(torch, q, dl, X):
    L = dl.layer
    T = X.shape[0]
    ws = torch.zeros(q.qmoe_router_workspace_bytes(L.n_experts, T), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty(T, L.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, L.top_k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, L.n_experts, dtype=torch.float32, device="cuda")
    q.qmoe_router_topk(L.router, dl.logit_bias, _dev_u16(torch, X), T, L.top_k, idx, w, lg, ws)
    return idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy().astype(np.float64)


def _oracle_rows_forced(ol, X, idx, w, residual=False):
    from concurrent.futures import ThreadPoolExecutor

    T = X.shape[0]
    with ThreadPoolExecutor(max_workers=min(T, 8)) as ex:
        res = list(ex.map(lambda t: ol.forward(X[t], residual=residual, force_idx=idx[t],
                                               force_w=w[t].astype(np.float64)), range(T)))
    return np.stack([r["out"] for r in res])


def _check_rows(got, ref, tol=2e-3):
    worst = 0.0
    for t in range(got.shape[0]):
        e = rel_l2(bf16_to_f64(got[t]), bf16_to_f64(ref[t]))
        worst = max(worst, e)
        assert e <= tol, (t, e)
    log(f"  worst row relL2 vs oracle bf16 = {worst:.2e}")


# ----------------------------------------------------------------- dispatch
def test_prefill_dispatch_matches_oracle_bit_exactly(torch_cuda, q, pf_layer):
    """Router over a 128-token chunk with the Zipf prior, then the device
    dispatch: counts, offsets and the stable (expert, token, rank) order are
    those of the oracle's dispatch of the same ids."""
    torch = torch_cuda
    lw, ol, dl = pf_layer
    T = PF.tokens
    X = synth.make_tokens(PF, T, stream=61)
    idx, w, _ = _router(torch, q, dl, X)
    _, ws = _prefill(torch, q, dl.layer, X, idx, w)
    counts, offsets, perm = _dispatch_of(torch, q, dl.layer, T, ws)
    rc, ro, rp = oracle.dispatch(idx, PF.n_experts)
    assert np.array_equal(counts, rc)
    assert np.array_equal(offsets, ro)
    assert np.array_equal(perm, rp)
    assert counts.sum() == T * PF.top_k and counts.max() <= T
    assert sorted(perm) == list(range(T * PF.top_k))
    log(f"  distinct experts {np.count_nonzero(counts)}, hottest {counts.max()} rows")


@pytest.mark.parametrize("T", [1, 2, 37, 128])
def test_prefill_dispatch_ragged_and_repeated(torch_cuda, q, tiny_layer, T):
    """Ragged T and ids that repeat inside a token (an expert with more rows
    than tokens) keep the stable order."""
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    rng = np.random.default_rng(T)
    idx = rng.integers(0, 5, size=(T, TINY.top_k)).astype(np.int32)
    w = np.full((T, TINY.top_k), 1.0 / TINY.top_k, np.float32)
    X = synth.make_tokens(TINY, T, stream=62)
    _, ws = _prefill(torch, q, dl.layer, X, idx, w)
    counts, offsets, perm = _dispatch_of(torch, q, dl.layer, T, ws)
    rc, ro, rp = oracle.dispatch(idx, TINY.n_experts)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro) and np.array_equal(perm, rp)


# ---------------------------------------------------------------- results
@pytest.mark.parametrize("T", [1, 4, 37, 128])
def test_prefill_forced_routing_tiny(torch_cuda, q, tiny_layer, T):
    """Dirichlet(1) weights over random distinct ids: every row against the
    oracle's layer with the same routing; odd T adds the residual."""
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    log(f"prefill tiny T={T}")
    X = synth.make_tokens(TINY, T, stream=63 + T)
    idx, w = synth.dirichlet_routing(TINY, T, stream=T)
    residual = bool(T % 2)
    got, _ = _prefill(torch, q, dl.layer, X, idx, w, residual=residual)
    ref = _oracle_rows_forced(ol, X, idx, w, residual=residual)
    _check_rows(got, ref)


@pytest.mark.parametrize("T", [5, 33])
def test_prefill_odd_widths(torch_cuda, q, T):
    """Hidden and intermediate widths that are not multiples of 128 (576,
    192, 320: the fp16 operand rows carry zero padding), 24 experts, top-4;
    forced routing, residual on odd rows counts."""
    torch = torch_cuda
    wl = synth.WORKLOADS["odd_prefill"]
    lw = synth.make_layer(wl, 0)
    ol, dl = oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)
    log(f"prefill odd widths T={T}")
    X = synth.make_tokens(wl, T, stream=70 + T)
    idx, w = synth.dirichlet_routing(wl, T, stream=30 + T)
    got, _ = _prefill(torch, q, dl.layer, X, idx, w, residual=True)
    _check_rows(got, _oracle_rows_forced(ol, X, idx, w, residual=True))


def test_prefill_wide_widths(torch_cuda, q):
    """Hidden and shared widths of 3200 (50 scale groups per row, more than
    the GEMMs' LDS scale tables hold): both GEMMs take their scales and
    biases with per-step loads instead; forced routing, residual."""
    torch = torch_cuda
    wl = synth.WORKLOADS["wide_prefill"]
    lw = synth.make_layer(wl, 0)
    ol, dl = oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)
    log("prefill wide widths T=5")
    X = synth.make_tokens(wl, wl.tokens, stream=75)
    idx, w = synth.dirichlet_routing(wl, wl.tokens, stream=35)
    got, _ = _prefill(torch, q, dl.layer, X, idx, w, residual=True)
    _check_rows(got, _oracle_rows_forced(ol, X, idx, w, residual=True))


def test_prefill_hot_and_repeated_experts(torch_cuda, q, tiny_layer):
    """Every token on the same 8 experts (128 rows each), then one expert
    repeated 8 times per token (1024 rows, more than one pass of 128)."""
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    T = 128
    X = synth.make_tokens(TINY, T, stream=64)
    _, w = synth.dirichlet_routing(TINY, T, stream=5)
    idx = np.tile(np.arange(8, dtype=np.int32) * 3, (T, 1))
    got, _ = _prefill(torch, q, dl.layer, X, idx, w)
    _check_rows(got, _oracle_rows_forced(ol, X, idx, w))
    idx = np.full((T, 8), 11, np.int32)
    got, _ = _prefill(torch, q, dl.layer, X, idx, w)
    _check_rows(got, _oracle_rows_forced(ol, X, idx, w))


def test_prefill_chunk_end_to_end(torch_cuda, q, pf_layer):
    """The 128-token chunk at full size: device router (Zipf prior) then the
    grouped prefill.  Routing equals the oracle's, up to certified
    near-ties; every row within 2e-3 of the oracle's layer output."""
    torch = torch_cuda
    lw, ol, dl = pf_layer
    T = PF.tokens
    X = synth.make_tokens(PF, T, stream=65)
    idx, w, lg = _router(torch, q, dl, X)
    got, _ = _prefill(torch, q, dl.layer, X, idx, w)
    ref = oracle.forward_many(ol, X)
    flips = 0
    for t in range(T):
        if list(idx[t]) != list(ref[t]["idx"]):
            l64 = ref[t]["logits"]
            B = routing_bound(lw.router, X[t], l64)
            assert routing_certified(B, l64, idx[t]), (t, "routing flip is not a certified near-tie")
            flips += 1
    log(f"  certified near-tie routing differences: {flips} of {T}")
    # outputs against the oracle driven by the device's routing decisions
    refo = _oracle_rows_forced(ol, X, idx, w)
    _check_rows(got, refo)
    # and the device weights are the softmax of the fp64 logits over the
    # device's experts, within what the logits' bounds allow
    for t in range(T):
        l64 = ref[t]["logits"]
        assert weights_consistent(routing_bound(lw.router, X[t], l64), l64, idx[t], w[t]), t


def test_prefill_token_permutation_is_bitwise(torch_cuda, q, pf_layer):
    """GEMM rows are independent and the combine order is fixed: permuting
    the tokens permutes the outputs bit for bit."""
    torch = torch_cuda
    lw, ol, dl = pf_layer
    T = 96
    X = synth.make_tokens(PF, T, stream=66)
    idx, w, _ = _router(torch, q, dl, X)
    a, ws = _prefill(torch, q, dl.layer, X, idx, w, residual=True)
    p = np.random.default_rng(7).permutation(T)
    b, _ = _prefill(torch, q, dl.layer, X[p], idx[p], w[p], residual=True, ws=ws)
    assert np.array_equal(a[p], b)


def test_prefill_row_equals_single_row_chunk(torch_cuda, q, tiny_layer):
    """A row's output does not depend on which other rows share its chunk."""
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    T = 40
    X = synth.make_tokens(TINY, T, stream=67)
    idx, w = synth.dirichlet_routing(TINY, T, stream=9)
    a, _ = _prefill(torch, q, dl.layer, X, idx, w)
    for t in (0, 17, 39):
        b, _ = _prefill(torch, q, dl.layer, X[t:t + 1], idx[t:t + 1], w[t:t + 1])
        assert np.array_equal(a[t], b[0])


def test_prefill_zero_input_is_zero(torch_cuda, q, tiny_layer):
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    T = 9
    idx, w = synth.dirichlet_routing(TINY, T, stream=1)
    got, _ = _prefill(torch, q, dl.layer, np.zeros((T, TINY.hidden), np.uint16), idx, w)
    assert np.all(got == 0)


def test_prefill_rejects_bad_arguments(torch_cuda, q, tiny_layer):
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    L = dl.layer
    X = torch.zeros(4, L.hidden, dtype=torch.int16, device="cuda")
    idx = torch.zeros(4, 8, dtype=torch.int32, device="cuda")
    w = torch.zeros(4, 8, dtype=torch.float32, device="cuda")
    out = torch.empty_like(X)
    with pytest.raises(q.QmoeError):
        q.qmoe_prefill_grouped(L, X, 0, idx, w, None, out, L.new_workspace(4))
    with pytest.raises(q.QmoeError):
        q.qmoe_prefill_grouped(L, X, 4, idx, w, None, out, L.new_workspace(1)[:1024])
