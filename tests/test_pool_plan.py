"""The expert pool's replacement bookkeeping (host code of the library,
planning-only pool: no GPU needed) against the hand-worked trace and the
oracle's LFU replay."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _replay(q, need, n_experts, slots, layers=1):
    pool = q.Pool(layers, n_experts, slots, 0)
    steps, k = need.shape
    out = {f: np.zeros((layers, steps, k), np.int32) for f in ("slot", "hit", "victim")}
    for t in range(steps):
        for l in range(layers):
            s, h, v = pool.plan(l, need[t])
            out["slot"][l, t], out["hit"][l, t], out["victim"][l, t] = s, h, v
    pool.close()
    return out


def test_pool_plan_matches_hand_trace():
    import bit_quantized_gemv_amd as q

    with open(os.path.join(GOLDEN, "lfu_hand_trace.json")) as f:
        g = json.load(f)
    r = _replay(q, np.array(g["need"], np.int32), g["n_experts"], g["slots"])
    assert r["hit"][0].tolist() == g["hit"]
    assert r["slot"][0].tolist() == g["slot"]
    assert r["victim"][0].tolist() == g["victim"]


def _zipf_needs(rng, steps, E, k, s=1.1):
    p = 1.0 / np.arange(1, E + 1) ** s
    p = p[rng.permutation(E)]
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(steps)]).astype(np.int32)


@pytest.mark.parametrize("E,k,slots,seed", [(128, 8, 16, 1), (32, 8, 16, 2), (128, 8, 8, 3),
                                            (40, 4, 6, 4)])
def test_pool_plan_matches_oracle_replay(E, k, slots, seed):
    """Zipf-skewed needs (heavy eviction): slots, hits and victims equal the
    oracle's replay step for step, on two layers kept apart."""
    import bit_quantized_gemv_amd as q

    rng = np.random.default_rng(seed)
    need = _zipf_needs(rng, 600, E, k)
    r = _replay(q, need, E, slots, layers=2)
    ref = oracle.lfu_replay(need, E, slots)
    for l in range(2):
        assert np.array_equal(r["hit"][l], ref["hit"])
        assert np.array_equal(r["slot"][l], ref["slot"])
        assert np.array_equal(r["victim"][l], ref["victim"])
    assert 0 < ref["hits"] < need.size


def test_pool_rejects_bad_arguments():
    import bit_quantized_gemv_amd as q

    pool = q.Pool(2, 32, 16, 0)
    with pytest.raises(q.QmoeError):
        pool.plan(0, [1, 1, 2])            # repeated id in one step
    with pytest.raises(q.QmoeError):
        pool.plan(2, [1, 2])               # layer out of range
    with pytest.raises(q.QmoeError):
        pool.plan(0, list(range(17)))      # more needed than slots
    with pytest.raises(q.QmoeError):
        pool.plan(0, [40])                 # expert out of range
    with pytest.raises(q.QmoeError):
        q.Pool(1, 8, 16, 0)                # more slots than experts
    pool.close()
