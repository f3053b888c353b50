"""GPU parity of the decode attention (qmoe_attn_decode) against the fp64
oracle (oracle.attn_step): one step at the attention workload's full sizes
(a 4,096-slot linear cache at its last position, a 1,024-slot circular cache
after it has wrapped) and at ragged and degenerate positions, plus whole
token sequences on small caches that cross the circular wrap.

Bars: each output element within one bf16 step of the fp64 value (plus
1e-5 of the head's largest magnitude for the fp32 sums), relative L2 per
head <= 2e-3 against the fp64 value rounded to bf16; the cache slot of the current token bit-exact to the oracle's
fp16 of RoPE(k) and of v (where the fp64 key lies within 1e-9 of an fp16
rounding midpoint either neighbour passes); every other slot untouched.
Slots that hold no token of the window are filled with fp16 NaN, so a read
of one would show in the output."""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import bf16_to_f64, log

pytestmark = pytest.mark.gpu

NAN16 = np.uint16(0x7E00)
AW = synth.ATTN_WORKLOADS["attn30_decode"]
TINY = synth.ATTN_WORKLOADS["tiny_attn"]


@pytest.fixture(scope="module")
def q():
    import torch

    assert torch.cuda.is_available()
    import bit_quantized_gemv_amd as q

    return q


def _slot(t, S, circ):
    return t % S if circ else t


def _history_times(pos, S, circ):
    """Times of the window other than the current token."""
    t0 = max(0, pos - S + 1) if circ else 0
    return range(t0, pos)


def _bf16_step(v):
    a = np.maximum(np.abs(v), 2.0**-126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _check_out(got_bits, ref, what):
    """got: the device's bf16 output; ref: the oracle's fp64 output, which
    the output format rounds to bf16 (the oracle's own encoder) for the
    relative L2 bar."""
    got = bf16_to_f64(got_bits.reshape(-1)).reshape(ref.shape)
    assert np.all(np.isfinite(got)), (what, "non-finite output: a slot outside the window was read")
    tol = _bf16_step(ref) + 1e-5 * np.abs(ref).max(axis=1, keepdims=True)
    err = np.abs(got - ref)
    assert np.all(err <= tol), (what, float((err / tol).max()))
    refb = bf16_to_f64(np.array([oracle.double_to_bf16(x) for x in ref.reshape(-1)],
                                dtype=np.uint16)).reshape(ref.shape)
    rel = np.linalg.norm(got - refb, axis=1) / np.linalg.norm(refb, axis=1)
    assert rel.max() <= 2e-3, (what, rel.max())
    return rel.max()


def _check_key(got, ref_bits, kf64, what):
    """Stored key fp16 bits: equal, or both neighbours of an fp64 value
    within 1e-9 (relative) of their midpoint."""
    bad = got != ref_bits
    if not bad.any():
        return
    a = got[bad].view(np.float16).astype(np.float64)
    b = ref_bits[bad].view(np.float16).astype(np.float64)
    x = kf64[bad]
    mid = (a + b) / 2
    ok = ((np.abs(x - mid) <= 1e-9 * np.abs(x)) & (np.minimum(a, b) <= x) & (x <= np.maximum(a, b)))
    assert ok.all(), (what, "stored key differs from fp16(RoPE(k))")


def _shape(q, Hq, Hkv, D, S, circ, base=10000.0):
    return q.AttnShape(Hq, Hkv, D, S, int(circ), base, 1.0 / np.sqrt(D))


def _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, ws):
    import torch

    out = torch.empty(shape.n_heads, shape.head_dim, dtype=torch.int16, device="cuda")
    q.qmoe_attn_decode(shape, torch.from_numpy(qv).cuda(), torch.from_numpy(kv).cuda(),
                       torch.from_numpy(vv).cuda(), pos, kc_d, vc_d, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def _ws(q, shape):
    import torch

    return torch.zeros(q.qmoe_attn_workspace_bytes(shape), dtype=torch.uint8, device="cuda")


CASES = [
    # Hq, Hkv, D, S, circular, pos
    (16, 8, 256, 4096, False, 4095),   # full layer, last position of the 4,096-token cache
    (16, 8, 256, 1024, True, 4095),    # sliding layer, wrapped (current slot 1023)
    (16, 8, 256, 1024, True, 5000),    # wrapped, current slot inside the store
    (16, 8, 256, 1024, True, 700),     # not yet full
    (16, 8, 256, 4096, False, 0),      # first token: the current one only
    (16, 8, 256, 4096, False, 20),     # one split
    (8, 8, 256, 333, True, 1000),      # ragged store, one query head per group
    (8, 4, 128, 64, True, 63),         # last position before the wrap
    (8, 4, 128, 64, True, 64),         # first position after it
    (8, 2, 128, 5000, False, 4999),    # four query heads per group, ragged splits
    (2, 1, 128, 100, False, 32),       # one group, one split plus one slot
    (4, 4, 256, 3000, True, 2999),     # many splits, one block row per head
]


@pytest.mark.parametrize("Hq,Hkv,D,S,circ,pos", CASES)
def test_attn_step_matches_oracle(q, Hq, Hkv, D, S, circ, pos):
    import torch

    log(f"attention step Hq={Hq} Hkv={Hkv} D={D} S={S} circular={circ} pos={pos}")
    aw = synth.AttnWorkload(30, "case", Hq, Hkv, D, S, S, 1, 0)
    qv, kv, vv, kc, vc = synth.attn_inputs(aw, S, stream=pos)
    hist = list(_history_times(pos, S, circ))
    cur = _slot(pos, S, circ)
    held = np.zeros(S, dtype=bool)
    held[[_slot(t, S, circ) for t in hist]] = True
    kc[:, ~held] = NAN16
    vc[:, ~held] = NAN16
    assert not held[cur]
    # the oracle's history, in time order
    kh = np.zeros((pos + 1, Hkv, D), dtype=np.uint16)
    vh = np.zeros((pos + 1, Hkv, D), dtype=np.uint16)
    for t in hist:
        kh[t] = kc[:, _slot(t, S, circ)]
        vh[t] = vc[:, _slot(t, S, circ)]
    ref = oracle.attn_step(qv, kv, vv, kh, vh, pos, S if circ else 0, 1.0 / np.sqrt(D), 10000.0)

    shape = _shape(q, Hq, Hkv, D, S, circ)
    kc_d = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    vc_d = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    ws = _ws(q, shape)
    got = _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, ws)
    rel = _check_out(got.reshape(Hq, D), ref, "output")
    assert q.qmoe_attn_workspace_status(ws, Hkv) == 0
    kc2 = kc_d.cpu().numpy().view(np.uint16)
    vc2 = vc_d.cpu().numpy().view(np.uint16)
    others = np.ones(S, dtype=bool)
    others[cur] = False
    assert np.array_equal(kc2[:, others], kc[:, others]), "a key slot other than the current changed"
    assert np.array_equal(vc2[:, others], vc[:, others]), "a value slot other than the current changed"
    assert np.array_equal(vc2[:, cur], vh[pos])
    kf = np.stack([oracle.rope(kv[g].astype(np.float64), pos, 10000.0) for g in range(Hkv)])
    _check_key(kc2[:, cur], kh[pos], kf, "current key")
    log(f"  worst head relL2 {rel:.2e}")


@pytest.mark.parametrize("S,circ,steps", [(TINY.window, True, 130), (TINY.context, False, 150)])
def test_attn_sequence_matches_oracle(q, S, circ, steps):
    """Token after token from an empty cache (all NaN): the device's cache
    evolves by its own writes, the oracle's history by its own; every
    step's output is compared, and at the end every slot of the window."""
    import torch

    Hq, Hkv, D = TINY.n_heads, TINY.n_kv_heads, TINY.head_dim
    log(f"attention sequence S={S} circular={circ} steps={steps}")
    shape = _shape(q, Hq, Hkv, D, S, circ)
    kc_d = torch.full((Hkv, S, D), int(NAN16.view(np.int16)), dtype=torch.int16, device="cuda")
    vc_d = torch.full((Hkv, S, D), int(NAN16.view(np.int16)), dtype=torch.int16, device="cuda")
    ws = _ws(q, shape)
    kh = np.zeros((steps, Hkv, D), dtype=np.uint16)
    vh = np.zeros((steps, Hkv, D), dtype=np.uint16)
    worst = 0.0
    for pos in range(steps):
        qv, kv, vv, _, _ = synth.attn_inputs(TINY, 1, stream=1000 + pos)
        ref = oracle.attn_step(qv, kv, vv, kh, vh, pos, S if circ else 0, 1.0 / np.sqrt(D),
                               10000.0)
        got = _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, ws)
        worst = max(worst, _check_out(got.reshape(Hq, D), ref, f"step {pos}"))
    assert q.qmoe_attn_workspace_status(ws, Hkv) == 0
    kc2 = kc_d.cpu().numpy().view(np.uint16)
    vc2 = vc_d.cpu().numpy().view(np.uint16)
    for t in range(max(0, steps - S) if circ else 0, steps):  # every token still cached
        s = _slot(t, S, circ)
        assert np.array_equal(vc2[:, s], vh[t]), t
        assert np.array_equal(kc2[:, s], kh[t]), t
    if not circ:
        assert np.all(kc2[:, steps:] == NAN16), "slots past the last token were written"
    log(f"  {steps} steps: worst head relL2 {worst:.2e}")


def test_attn_zero_keys_give_the_window_mean(q):
    """Zero keys everywhere and a zero current key: every score is 0, so
    every query head returns the mean of its group's values in the window
    (times pos - S + 1 .. pos of a wrapped circular store)."""
    import torch

    Hq, Hkv, D, S, pos = 16, 8, 256, 1024, 3000
    aw = synth.AttnWorkload(31, "zero", Hq, Hkv, D, S, S, 1, 0)
    qv, kv, vv, kc, vc = synth.attn_inputs(aw, S, stream=7)
    kc[:] = 0
    kv[:] = 0
    shape = _shape(q, Hq, Hkv, D, S, True)
    kc_d = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    vc_d = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    got = _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, _ws(q, shape))
    vals = vc_d.cpu().numpy().view(np.float16).astype(np.float64)  # current value written in
    mean = vals.mean(axis=1)  # [Hkv][D]
    _check_out(got.reshape(Hq, D), np.repeat(mean, Hq // Hkv, axis=0), "window mean")


def test_attn_workspace_error_word_and_reset(q):
    """A merging block whose epoch word disagrees with the split blocks'
    (set from the host) never sees its call's tags: its bounded wait gives
    up, the error word is set, qmoe_attn_workspace_status reports it and
    zeroes the workspace, and the next call is correct again."""
    import torch

    Hq, Hkv, D, S, pos = 16, 8, 256, 1024, 2000
    aw = synth.AttnWorkload(32, "err", Hq, Hkv, D, S, S, 1, 0)
    qv, kv, vv, kc, vc = synth.attn_inputs(aw, S, stream=9)
    shape = _shape(q, Hq, Hkv, D, S, True)
    ws = _ws(q, shape)
    # epoch words start at byte 64, 8 per key/value head: head 0's first
    # one (read by the split blocks and merging block 0) moves ahead
    ws[64:68] = torch.tensor([5, 0, 0, 0], dtype=torch.uint8)
    kc_d = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    vc_d = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, ws)
    with pytest.raises(q.QmoeError, match="DEVICE"):
        q.qmoe_attn_workspace_status(ws, Hkv)
    assert not ws.any(), "the workspace is zeroed after an error"
    # a correct call on the reset workspace (the cache now holds this
    # call's first write at slot pos mod S, which the next step overwrites)
    kh = np.zeros((pos + 1, Hkv, D), dtype=np.uint16)
    vh = np.zeros((pos + 1, Hkv, D), dtype=np.uint16)
    kc2 = kc_d.cpu().numpy().view(np.uint16)
    vc2 = vc_d.cpu().numpy().view(np.uint16)
    for t in _history_times(pos, S, True):
        kh[t] = kc2[:, _slot(t, S, True)]
        vh[t] = vc2[:, _slot(t, S, True)]
    ref = oracle.attn_step(qv, kv, vv, kh, vh, pos, S, 1.0 / np.sqrt(D), 10000.0)
    got = _step(q, shape, qv, kv, vv, pos, kc_d, vc_d, ws)
    _check_out(got.reshape(Hq, D), ref, "after reset")
    assert q.qmoe_attn_workspace_status(ws, Hkv) == 0
