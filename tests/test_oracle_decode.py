"""Pins of the oracle's decode step (one token per request) to facts fixed by the pages
and by mathematics: the hand-worked example taken one token per call through the pool,
closed forms at saturated gates, and the rank-one form of a single step."""
import json
import math
import os

import numpy as np
import pytest

import gdn_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def decode_problem(q, k, v, a, b, A_log, dt_bias, state, cache_indices, H=1, HV=1,
                   dtype="f32"):
    """B requests of one token each; q, k [B, H, dk], v [B, HV, dv], a, b [B, HV]."""
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    B = q.shape[0]
    return gdn_synth.Problem(
        name="decode", dtype=dtype, H=H, HV=HV, dk=q.shape[2], dv=v.shape[2], q=q, k=k, v=v,
        a=np.asarray(a, np.float32).reshape(B, HV), b=np.asarray(b, np.float32).reshape(B, HV),
        A_log=np.asarray(A_log, np.float32).reshape(HV),
        dt_bias=np.asarray(dt_bias, np.float32).reshape(HV),
        state_pool=np.asarray(state, np.float32),
        cache_indices=np.asarray(cache_indices, np.int64),
        cu_seqlens=np.arange(B + 1, dtype=np.int64))


def unit(x):
    x = np.asarray(x, np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_worked_example_one_token_per_call():
    """The hand-worked dk = dv = 2 example, fed as three decode calls that carry the state
    through slot 1 of a 3-slot pool (slots 0 and 2 must stay as they are)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_dk2.json")))
    pool = np.zeros((3, 1, 2, 2), np.float32)
    pool[0, 0] = [[5.0, -1.0], [2.0, 7.0]]
    pool[2, 0] = [[-3.0, 0.5], [0.25, 9.0]]
    expect_S = {1: ex["S_after_2"], 2: ex["S_after_3"]}
    state = pool.astype(np.float64)
    for t in range(3):
        p = decode_problem([[ex["q"][t]]], [[ex["k"][t]]], [[ex["v"][t]]], [ex["a"][t]],
                           [ex["b"][t]], ex["A_log"], ex["dt_bias"], state.astype(np.float32),
                           [1])
        r = oracle.decode(p, eps=ex["eps"])
        # Between calls the state sits in the fp32 pool: S1 = [[1/2, 0], [0, 0]] is exact
        # there, S2 (entries sqrt2/4) is rounded, which moves o3 by up to ~1e-7 |S2|.
        np.testing.assert_allclose(r.out[0, 0], ex["o"][t], rtol=0,
                                   atol=1e-15 if t < 2 else 2e-7)
        if t in expect_S:
            np.testing.assert_allclose(r.state_pool[1, 0], expect_S[t], rtol=0, atol=1e-7)
        np.testing.assert_array_equal(r.state_pool[[0, 2]], pool[[0, 2]].astype(np.float64))
        state = r.state_pool
    # The first step alone: S1 = beta v k^T = [[1/2, 0], [0, 0]] from a zero state.
    p = decode_problem([[ex["q"][0]]], [[ex["k"][0]]], [[ex["v"][0]]], [ex["a"][0]],
                       [ex["b"][0]], ex["A_log"], ex["dt_bias"], np.zeros((1, 1, 2, 2)), [0])
    r = oracle.decode(p, eps=ex["eps"])
    np.testing.assert_array_equal(r.state_pool[0, 0], [[0.5, 0.0], [0.0, 0.0]])


@pytest.mark.parametrize("seed", [31, 32])
def test_overwrite_at_saturated_gates(seed):
    """alpha = 1 (a = -1e4) and beta = 1 (b = 1e4): S_new = S + (v - S kh) kh^T, so
    S_new kh = v, and with q = k the read returns v; rows orthogonal to kh keep S."""
    rng = np.random.default_rng(seed)
    B, H, HV, dk, dv, pool = 5, 2, 4, 8, 6, 9
    k = rng.standard_normal((B, H, dk))
    v = rng.standard_normal((B, HV, dv))
    state = rng.standard_normal((pool, HV, dv, dk)).astype(np.float32)
    idx = rng.permutation(pool)[:B]
    p = decode_problem(k, k, v, np.full((B, HV), -1e4), np.full((B, HV), 1e4),
                       rng.uniform(-1, 1, HV), rng.normal(0, 0.3, HV), state, idx, H=H, HV=HV)
    r = oracle.decode(p, eps=0.0)
    for bi in range(B):
        for hv in range(HV):
            kh = unit(p.k[bi, hv // (HV // H)])
            S_new = r.state_pool[idx[bi], hv]
            np.testing.assert_allclose(S_new @ kh, p.v[bi, hv], rtol=0, atol=1e-13)
            np.testing.assert_allclose(r.out[bi, hv], p.v[bi, hv], rtol=0, atol=1e-13)
            P = np.eye(dk) - np.outer(kh, kh)    # projector onto kh's complement
            np.testing.assert_allclose(S_new @ P, state[idx[bi], hv].astype(np.float64) @ P,
                                       rtol=0, atol=1e-13)
    untouched = sorted(set(range(pool)) - set(idx.tolist()))
    np.testing.assert_array_equal(r.state_pool[untouched], state[untouched].astype(np.float64))


def test_decay_only_step():
    """beta = 0 (b = -1e4), A_log = 0 and a = -dt_bias: alpha = exp(-ln 2) = 1/2, so
    S_new = S / 2 and out = (S qh) / 2."""
    rng = np.random.default_rng(33)
    B, HV, dk, dv = 3, 2, 6, 4
    q = rng.standard_normal((B, 1, dk))
    k = rng.standard_normal((B, 1, dk))
    v = rng.standard_normal((B, HV, dv))
    dtb = np.array([0.375, -1.25], np.float32)
    state = rng.standard_normal((B, HV, dv, dk)).astype(np.float32)
    p = decode_problem(q, k, v, np.tile(-dtb, (B, 1)), np.full((B, HV), -1e4), [0.0, 0.0], dtb,
                       state, [2, 0, 1], H=1, HV=HV)
    r = oracle.decode(p, eps=0.0)
    for bi, slot in enumerate([2, 0, 1]):
        qh = unit(p.q[bi, 0])
        for hv in range(HV):
            S = state[slot, hv].astype(np.float64)
            np.testing.assert_allclose(r.state_pool[slot, hv], S / 2, rtol=1e-15, atol=0)
            np.testing.assert_allclose(r.out[bi, hv], (S @ qh) / 2, rtol=1e-14, atol=1e-15)


def test_one_step_is_rank_one_update():
    """For any gates: S_new - alpha S = u kh^T with u = beta (v - alpha S kh), and
    out = alpha S qh + (kh . qh) u. alpha and beta in closed form from A_log = ln 8,
    a + dt_bias = 0 (alpha = exp(-8 ln 2) = 2^-8) and b = ln 3 (beta = 3/4)."""
    rng = np.random.default_rng(34)
    B, H, HV, dk, dv = 4, 1, 2, 16, 8
    q = rng.standard_normal((B, H, dk))
    k = rng.standard_normal((B, H, dk))
    v = rng.standard_normal((B, HV, dv))
    state = rng.standard_normal((B, HV, dv, dk)).astype(np.float32)
    b = np.float32(math.log(3.0))
    p = decode_problem(q, k, v, np.zeros((B, HV)), np.full((B, HV), b), [math.log(8.0)] * HV,
                       [0.0] * HV, state, [3, 1, 0, 2], H=H, HV=HV)
    r = oracle.decode(p, eps=0.0)
    # softplus(0) = ln 2; A_log and b are the fp32 roundings of ln 8 and ln 3
    alpha = math.exp(-math.exp(float(np.float32(math.log(8.0)))) * math.log(2.0))
    beta = 1.0 / (1.0 + math.exp(-float(b)))
    assert abs(alpha / 2.0 ** -8 - 1) < 1e-6 and abs(beta - 0.75) < 1e-7
    for bi, slot in enumerate([3, 1, 0, 2]):
        kh, qh = unit(p.k[bi, 0]), unit(p.q[bi, 0])
        for hv in range(HV):
            S = state[slot, hv].astype(np.float64)
            u = beta * (p.v[bi, hv] - alpha * (S @ kh))
            np.testing.assert_allclose(r.state_pool[slot, hv], alpha * S + np.outer(u, kh),
                                       rtol=0, atol=2e-14)
            np.testing.assert_allclose(r.out[bi, hv], alpha * (S @ qh) + (kh @ qh) * u,
                                       rtol=0, atol=2e-14)


def test_decode_requires_one_token_per_request():
    p = gdn_synth.make_problem(35, [2, 1], 1, 1, 8, 8, dtype="f32")
    with pytest.raises(ValueError):
        oracle.decode(p)


def test_decode_problem_generator_shapes():
    p = gdn_synth.make_decode_problem(36, 6, 2, 4, 64, 128, dtype="bf16", pool=10,
                                      cache_indices=[9, 0, 3, 4, 8, 1])
    assert p.q.shape == (6, 2, 64) and p.v.shape == (6, 4, 128) and p.a.shape == (6, 4)
    assert p.state_pool.shape == (10, 4, 128, 64)
    np.testing.assert_array_equal(p.cu_seqlens, np.arange(7))
    r = oracle.decode(p, heads=[1, 2], rows=(0, 16))
    assert r.out.shape == (6, 2, 16)
