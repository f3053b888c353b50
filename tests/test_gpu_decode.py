"""GPU parity of the decode path (quantized GEMV, router top-k, expert FFN,
one-launch decode step) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import (bf16_to_f64, gemv4_bound, gemv8_bound, log, rel_l2, routing_bound,
                           routing_certified, to_u16, weights_consistent)

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_layer_decode"]
LAYER = synth.WORKLOADS["layer_decode"]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def q():
    import bit_quantized_gemv_amd as q

    return q


def _dev_u16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


# ------------------------------------------------------------ 4-bit GEMV
@pytest.mark.parametrize("rows,cols", [(64, 512), (37, 2816), (2816, 704), (100, 2112), (8, 64)])
def test_gemv_unit_scale_one_hot_is_bit_exact(torch_cuda, q, rows, cols):
    """x = e_j, s = 1, b = 0: y must equal the code q[r][j] exactly."""
    torch = torch_cuda
    log(f"gemv one-hot rows={rows} cols={cols}")
    m = synth.random_qmat(rows, cols, 4, 100 + rows)
    m.s[:] = np.float16(1.0).view(np.uint16)
    m.b[:] = 0
    W = synth.device.qtensor(m)
    codes = oracle.unpack(m.q, rows, cols, 4)
    cols_to_check = range(cols) if cols <= 512 else np.random.default_rng(0).choice(cols, 24, replace=False)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    for j in cols_to_check:
        x = np.zeros(cols, dtype=np.uint16)
        x[j] = 0x3F80  # bf16 1.0
        q.qmoe_gemv_affine4(W, _dev_u16(torch, x), y)
        assert np.array_equal(y.cpu().numpy(), codes[:, j].astype(np.float32)), j


def test_gemv_one_hot_affine_is_fp32_of_exact_weight(torch_cuda, q):
    """x = e_j with real scales and biases: y = fl32(s q + b) exactly."""
    torch = torch_cuda
    m = synth.random_qmat(96, 2816, 4, 7)
    W = synth.device.qtensor(m)
    Wd = oracle.dequant(m)
    y = torch.empty(96, dtype=torch.float32, device="cuda")
    for j in (0, 5, 63, 64, 1000, 2815):
        x = np.zeros(2816, dtype=np.uint16)
        x[j] = 0x3F80
        q.qmoe_gemv_affine4(W, _dev_u16(torch, x), y)
        assert np.array_equal(y.cpu().numpy(), Wd[:, j].astype(np.float32)), j


@pytest.mark.parametrize("rows,cols", [(2112, 2816), (704, 2816), (2816, 704), (2816, 2112),
                                       (13, 512), (256, 64)])
def test_gemv_matches_oracle_within_bound(torch_cuda, q, rows, cols):
    torch = torch_cuda
    log(f"gemv parity rows={rows} cols={cols}")
    m = synth.random_qmat(rows, cols, 4, rows * 7 + cols)
    x = synth.random_bf16(cols, 3)
    xd = bf16_to_f64(x)
    ref = oracle.qgemv(m, xd)
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    q.qmoe_gemv_affine4(synth.device.qtensor(m), _dev_u16(torch, x), y)
    got = y.cpu().numpy().astype(np.float64)
    bound = gemv4_bound(m, xd)
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)
    assert rel_l2(got, ref) <= 1e-5


@pytest.mark.parametrize("rows,cols", [(20003, 2816), (40000, 2112), (70001, 704)])
def test_gemv_large_matches_oracle_within_bound(torch_cuda, q, rows, cols):
    """Matrices large enough for the persistent form (more row-blocks than
    resident waves), with a ragged last row-block: every row within the
    bound of the oracle's fp64 GEMV."""
    torch = torch_cuda
    log(f"gemv parity (persistent) rows={rows} cols={cols}")
    m = synth.random_qmat(rows, cols, 4, rows + cols)
    x = synth.random_bf16(cols, 5)
    xd = bf16_to_f64(x)
    ref = oracle.qgemv(m, xd)
    y = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    q.qmoe_gemv_affine4(synth.device.qtensor(m), _dev_u16(torch, x), y)
    got = y.cpu().numpy().astype(np.float64)
    bound = gemv4_bound(m, xd)
    assert np.all(np.abs(got - ref) <= bound), np.nanmax(np.abs(got - ref) / bound)
    assert rel_l2(got, ref) <= 1e-5


def test_gemv_rejects_bad_arguments(torch_cuda, q):
    torch = torch_cuda
    m = synth.random_qmat(8, 128, 4, 1)
    W = synth.device.qtensor(m)
    y = torch.empty(8, dtype=torch.float32, device="cuda")
    x = torch.zeros(128, dtype=torch.int16, device="cuda")
    W.cols = 100
    with pytest.raises(q.QmoeError, match="BAD_SHAPE"):
        q.qmoe_gemv_affine4(W, x, y)
    W.cols, W.bits = 128, 8
    with pytest.raises(q.QmoeError, match="UNSUPPORTED"):
        q.qmoe_gemv_affine4(W, x, y)


# ---------------------------------------------------------------- router
def _router(torch, q, Wr, X, K, bias=None):
    T, H = X.shape
    E = Wr.rows
    ws = torch.zeros(q.qmoe_router_workspace_bytes(E, T), dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    q.qmoe_router_topk(synth.device.qtensor(Wr), b, _dev_u16(torch, X), T, K, idx, w, lg, ws)
    return idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wl,T", [(TINY, 3), (LAYER, 1), (LAYER, 37), (LAYER, 128),
                                  (synth.WORKLOADS["max_experts_decode"], 5)])
def test_router_topk_parity(torch_cuda, q, wl, T):
    """GPU logits within the fp32 bound of the fp64 logits; GPU idx equal to
    the oracle's top-k of the GPU's own logits; weights its softmax."""
    torch = torch_cuda
    log(f"router T={T} E={wl.n_experts}")
    Wr = synth.make_layer(wl, 0, n_experts_materialized=0).router
    X = synth.make_tokens(wl, T, stream=5)
    bias = synth.zipf_prior(wl, 0) if T > 1 else None
    idx, w, lg = _router(torch, q, Wr, X, wl.top_k, bias)
    for t in range(T):
        xd = bf16_to_f64(X[t])
        ref = oracle.qgemv(Wr, xd) + (0 if bias is None else bias.astype(np.float64))
        bound = gemv8_bound(Wr, xd) + np.abs(ref) * 2**-24
        assert np.all(np.abs(lg[t] - ref) <= bound), t
        oi, ow = oracle.topk_softmax(lg[t], wl.top_k)
        assert list(idx[t]) == list(oi), t
        assert np.allclose(w[t], ow, rtol=2e-6, atol=1e-7)
        assert abs(w[t].sum() - 1) <= 32 * 2**-24
        assert np.all(np.diff(w[t]) <= 0)


def test_router_exact_ties_go_to_lower_index(torch_cuda, q):
    torch = torch_cuda
    Wr = synth.random_qmat(64, 512, 8, 77)
    for a, b in ((3, 40), (10, 11), (0, 63)):
        Wr.q[b] = Wr.q[a]
        Wr.s[b] = Wr.s[a]
        Wr.b[b] = Wr.b[a]
    X = synth.random_bf16((6, 512), 78)
    # bias that makes the duplicated experts win
    bias = np.full(64, -1e4, np.float32)
    bias[[3, 40, 10, 11, 0, 63]] = 0
    idx, w, lg = _router(torch, q, Wr, X, 6, bias)
    for t in range(6):
        assert lg[t, 3] == lg[t, 40] and lg[t, 10] == lg[t, 11] and lg[t, 0] == lg[t, 63]
        pos = {e: list(idx[t]).index(e) for e in (3, 40, 10, 11, 0, 63)}
        assert pos[3] < pos[40] and pos[10] < pos[11] and pos[0] < pos[63]


def test_router_equal_logits_give_uniform_weights(torch_cuda, q):
    torch = torch_cuda
    Wr = synth.random_qmat(16, 128, 8, 5)
    Wr.s[:] = 0
    Wr.b[:] = 0
    idx, w, _ = _router(torch, q, Wr, synth.random_bf16((2, 128), 6), 8)
    assert np.all(idx == np.arange(8)[None, :])
    assert np.all(w == 0.125)


# ------------------------------------------------------- FFN and decode
@pytest.fixture(scope="module")
def tiny_layer():
    lw = synth.make_layer(TINY, 0)
    return lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)


@pytest.fixture(scope="module")
def big_layer():
    lw = synth.make_layer(LAYER, 0)
    return lw, oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)


def _expert_ffn(torch, q, dl, h, idx, w, residual=None):
    L = dl.layer
    ws = L.new_workspace(1)
    out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
    q.qmoe_expert_ffn(L, _dev_u16(torch, h), torch.from_numpy(np.asarray(idx, np.int32)).cuda(),
                      torch.from_numpy(np.asarray(w, np.float32)).cuda(), None,
                      None if residual is None else _dev_u16(torch, residual), out, ws)
    assert q.qmoe_workspace_status(ws) == 0
    return to_u16(out)


@pytest.mark.parametrize("which", ["tiny", "big"])
def test_expert_ffn_dirichlet_combine(torch_cuda, q, tiny_layer, big_layer, which):
    """All k experts matter: random distinct ids, Dirichlet(1) weights."""
    torch = torch_cuda
    lw, ol, dl = tiny_layer if which == "tiny" else big_layer
    wl = lw.wl
    n = 4 if which == "tiny" else 2
    X = synth.make_tokens(wl, n, stream=11)
    idx, w = synth.dirichlet_routing(wl, n, stream=3)
    for t in range(n):
        log(f"expert_ffn {which} token {t}")
        res = X[(t + 1) % n] if t % 2 else None
        got = _expert_ffn(torch, q, dl, X[t], idx[t], w[t], residual=res)
        # the oracle's layer with forced routing; residual handled by hand
        r = ol.forward(X[t], force_idx=idx[t], force_w=w[t].astype(np.float64))
        y = r["y"] + (bf16_to_f64(res) if res is not None else 0)
        ref = np.array([oracle.double_to_bf16(v) for v in y], dtype=np.uint16)
        e = rel_l2(bf16_to_f64(got), bf16_to_f64(ref))
        log(f"  relL2 vs oracle bf16 = {e:.2e}")
        assert e <= 2e-3


def test_expert_ffn_zero_input_is_zero(torch_cuda, q, tiny_layer):
    torch = torch_cuda
    lw, ol, dl = tiny_layer
    got = _expert_ffn(torch, q, dl, np.zeros(TINY.hidden, np.uint16), np.arange(8), np.full(8, 0.125))
    assert np.all(got == 0)


def _decode(torch, q, dl, x, residual=False, phased=False, ws=None):
    L = dl.layer
    ws = L.new_workspace(1) if ws is None else ws
    out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
    idx = torch.empty(L.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(L.top_k, dtype=torch.float32, device="cuda")
    q.qmoe_moe_decode(L, _dev_u16(torch, x), None, residual, out, idx, w, ws, phased=phased)
    assert q.qmoe_workspace_status(ws) == 0
    return to_u16(out), idx.cpu().numpy(), w.cpu().numpy()


def _check_decode_token(ol, x, got, gidx, gw, residual=False):
    """Oracle comparison; a routing difference must be a certified near-tie:
    the device's ranking consistent with the fp64 logits moved by at most
    each router row's fp32 error bound."""
    r = ol.forward(x, residual=residual)
    B = routing_bound(ol.lw.router, x, r["logits"], gamma=ol.lw.gamma)
    assert weights_consistent(B, r["logits"], gidx, gw), "combine weights"
    if list(gidx) != list(r["idx"]):
        lg = r["logits"]
        log(f"  routing differs {list(gidx)} vs {list(r['idx'])}")
        assert routing_certified(B, lg, gidx), "routing flip is not a certified near-tie"
        from scipy.special import softmax

        r = ol.forward(x, residual=residual, force_idx=gidx, force_w=softmax(lg[gidx]))
    e = rel_l2(bf16_to_f64(got), bf16_to_f64(r["out"]))
    log(f"  decode relL2 vs oracle bf16 = {e:.2e}")
    assert e <= 2e-3


@pytest.mark.parametrize("which,n", [("tiny", 4), ("big", 3)])
def test_moe_decode_end_to_end(torch_cuda, q, tiny_layer, big_layer, which, n):
    torch = torch_cuda
    lw, ol, dl = tiny_layer if which == "tiny" else big_layer
    X = synth.make_tokens(lw.wl, n, stream=21)
    ws = dl.layer.new_workspace(1)
    for t in range(n):
        log(f"decode {which} token {t}")
        got, gidx, gw = _decode(torch, q, dl, X[t], residual=bool(t % 2), ws=ws)
        _check_decode_token(ol, X[t], got, gidx, gw, residual=bool(t % 2))


def test_moe_decode_odd_expert_count(torch_cuda, q):
    """E = 21 (the last router block holds 5 rows), H = 576, RMSNorm: the
    one-launch step against the oracle, with and without the residual."""
    torch = torch_cuda
    wl = synth.WORKLOADS["odd_experts_decode"]
    lw = synth.make_layer(wl, 0)
    ol, dl = oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)
    X = synth.make_tokens(wl, wl.tokens, stream=23)
    ws = dl.layer.new_workspace(1)
    for t in range(wl.tokens):
        log(f"decode odd experts token {t}")
        got, gidx, gw = _decode(torch, q, dl, X[t], residual=bool(t % 2), ws=ws)
        _check_decode_token(ol, X[t], got, gidx, gw, residual=bool(t % 2))


def test_moe_decode_max_expert_count(torch_cuda, q):
    """E = 512 (the most the kernels take; 64 router blocks, top-k over 8
    values per lane), I = 64, Is = 128: widths with no compile-time
    specialisation, whose down blocks take their tasks pass by pass."""
    torch = torch_cuda
    wl = synth.WORKLOADS["max_experts_decode"]
    lw = synth.make_layer(wl, 0)
    ol, dl = oracle.OracleLayer(lw), synth.device.DeviceLayer(lw)
    X = synth.make_tokens(wl, wl.tokens, stream=25)
    ws = dl.layer.new_workspace(1)
    for t in range(wl.tokens):
        log(f"decode max experts token {t}")
        got, gidx, gw = _decode(torch, q, dl, X[t], residual=bool(t % 2), ws=ws)
        _check_decode_token(ol, X[t], got, gidx, gw, residual=bool(t % 2))


def test_moe_decode_single_launch_equals_phased(torch_cuda, q, big_layer):
    """One launch with in-kernel waits and three ordered launches run the
    same arithmetic: outputs are bitwise equal, repeatedly."""
    torch = torch_cuda
    lw, ol, dl = big_layer
    X = synth.make_tokens(lw.wl, 4, stream=31)
    ws = dl.layer.new_workspace(1)
    for t in range(4):
        a = _decode(torch, q, dl, X[t], residual=True, ws=ws)
        b = _decode(torch, q, dl, X[t], residual=True, phased=True, ws=ws)
        c = _decode(torch, q, dl, X[t], residual=True, ws=ws)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[0], c[0])
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_moe_decode_relabelling_is_bitwise_invariant(torch_cuda, q):
    torch = torch_cuda
    lw = synth.make_layer(TINY, 0)
    lw.prior = np.random.default_rng(3).normal(0, 40, TINY.n_experts).astype(np.float32)
    x = synth.make_tokens(TINY, 1, stream=41)[0]
    a, ia, _ = _decode(torch, q, synth.device.DeviceLayer(lw), x)
    perm = np.random.default_rng(4).permutation(TINY.n_experts)
    lw2 = synth.make_layer(TINY, 0)
    lw2.blobs = lw.blobs[perm].copy()
    for f in ("q", "s", "b"):
        setattr(lw2.router, f, getattr(lw.router, f)[perm].copy())
    lw2.prior = lw.prior[perm].copy()
    b, ib, _ = _decode(torch, q, synth.device.DeviceLayer(lw2), x)
    assert np.array_equal(a, b)
    assert list(perm[ib]) == list(ia)


def test_rmsnorm_matches_oracle(torch_cuda, q):
    torch = torch_cuda
    T, H = 5, 2816
    X = synth.random_bf16((T, H), 51)
    g = synth.to_bf16_bits(np.random.default_rng(52).normal(1, 0.02, H))
    out = torch.empty(T, H, dtype=torch.int16, device="cuda")
    q.qmoe_rmsnorm(_dev_u16(torch, X), _dev_u16(torch, g), 1e-6, T, H, out)
    got = to_u16(out)
    for t in range(T):
        ref = oracle.rmsnorm(X[t], g)
        d = np.abs(got[t].astype(np.int32) - ref.astype(np.int32))
        # equal, or one bf16 step apart at a rounding boundary (fp32 vs fp64)
        assert np.all(d <= 1) and np.mean(d) < 1e-2


def test_moe_decode_timed_equals_untimed(torch_cuda, q, big_layer):
    """The timing variant records its events and computes the same bits."""
    torch = torch_cuda
    lw, ol, dl = big_layer
    L = dl.layer
    x = synth.make_tokens(lw.wl, 1, stream=71)[0]
    ref, ridx, rw = _decode(torch, q, dl, x, residual=True)
    ws = L.new_workspace(1)
    xd = _dev_u16(torch, x)
    out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
    idx = torch.empty(L.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(L.top_k, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    q.qmoe_moe_decode_timed(L, xd, None, True, out, idx, w, ws, e0.cuda_event, e1.cuda_event)
    torch.cuda.synchronize()
    assert q.qmoe_workspace_status(ws) == 0
    assert np.array_equal(to_u16(out), ref)
    assert list(idx.cpu().numpy()) == list(ridx)
    ms = e0.elapsed_time(e1)
    log(f"  timed step kernel {ms * 1e3:.1f} us")
    assert 0 < ms < 100


def test_expert_ffn_split_equals_one_launch(torch_cuda, q, big_layer):
    """Shared gate/up first, routed part second (same stream and workspace):
    the same bits as qmoe_expert_ffn, with and without an expert->slot map."""
    torch = torch_cuda
    lw, ol, dl = big_layer
    L = dl.layer
    X = synth.make_tokens(lw.wl, 2, stream=72)
    idx, w = synth.dirichlet_routing(lw.wl, 2, stream=7)
    ws = L.new_workspace(1)
    for t in range(2):
        h = _dev_u16(torch, X[t])
        idx_d = torch.from_numpy(idx[t]).cuda()
        w_d = torch.from_numpy(w[t]).cuda()
        ref = _expert_ffn(torch, q, dl, X[t], idx[t], w[t], residual=X[1 - t])
        out = torch.empty(L.hidden, dtype=torch.int16, device="cuda")
        q.qmoe_expert_ffn_shared(L, h, ws)
        q.qmoe_expert_ffn_routed(L, h, idx_d, w_d, None, _dev_u16(torch, X[1 - t]), out, ws)
        assert np.array_equal(to_u16(out), ref)
        ident = torch.arange(L.n_experts, dtype=torch.int32, device="cuda")
        q.qmoe_expert_ffn_shared(L, h, ws)
        q.qmoe_expert_ffn_routed(L, h, idx_d, w_d, ident, _dev_u16(torch, X[1 - t]), out, ws)
        assert np.array_equal(to_u16(out), ref)
    assert q.qmoe_workspace_status(ws) == 0
