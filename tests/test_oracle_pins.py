"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

None of these retypes the oracle's loop: each checks it against a closed form, a
hand-worked example, a 40-digit brute force of the product form, the chunkwise
forms of the pages, or an invariant of the map.
"""
import json
import math
import os

import numpy as np
import pytest

import gdn_synth
import oracle
from oracle import bruteforce, chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def custom_problem(q, k, v, a, b, A_log, dt_bias, lengths, H=1, HV=1, state=None,
                   cache_indices=None, pool=None, dtype="f32"):
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    N = q.shape[0]
    if q.ndim == 2:
        q = q.reshape(N, 1, -1)
        k = k.reshape(N, 1, -1)
        v = v.reshape(N, 1, -1)
    dk, dv = q.shape[2], v.shape[2]
    B = len(lengths)
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    if pool is None:
        pool = B
    if cache_indices is None:
        cache_indices = list(range(B))
    if state is None:
        state = np.zeros((pool, HV, dv, dk), np.float32)
    return gdn_synth.Problem(
        name="custom", dtype=dtype, H=H, HV=HV, dk=dk, dv=dv, q=q, k=k, v=v,
        a=np.asarray(a, np.float32).reshape(N, HV), b=np.asarray(b, np.float32).reshape(N, HV),
        A_log=np.asarray(A_log, np.float32).reshape(HV),
        dt_bias=np.asarray(dt_bias, np.float32).reshape(HV),
        state_pool=np.asarray(state, np.float32), cache_indices=np.asarray(cache_indices, np.int64),
        cu_seqlens=cu)


def rel(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


# ---------------------------------------------------------------- gates
def test_gate_closed_forms():
    # A_log = 0, a = -dt_bias: softplus(0) = ln 2, so alpha = 1/2; b = 0: beta = 1/2.
    for dtb in (0.0, 0.37, -1.25):
        al, be, g = oracle.gates(-dtb, 0.0, 0.0, dtb)
        assert al == pytest.approx(0.5, rel=2e-16, abs=0)
        assert be == 0.5
        assert g == pytest.approx(-math.log(2.0), rel=2e-16)
    # saturated gates are exact
    assert oracle.gates(0.0, 1e4, 0.0, 0.0)[1] == 1.0
    assert oracle.gates(0.0, -1e4, 0.0, 0.0)[1] == 0.0
    assert oracle.gates(-1e4, 0.0, 3.0, 0.0)[0] == 1.0
    # A_log scales the log-decay: g = -exp(A_log) ln 2 at a + dt_bias = 0
    al, _, g = oracle.gates(0.0, 0.0, math.log(8.0), 0.0)
    assert g == pytest.approx(-8.0 * math.log(2.0), rel=4e-16)
    assert al == pytest.approx(2.0 ** -8, rel=4e-15)
    # large argument: softplus(x) -> x, so alpha = exp(-x)
    al, _, g = oracle.gates(30.0, 0.0, 0.0, 0.0)
    assert g == pytest.approx(-(30.0 + math.log1p(math.exp(-30.0))), rel=1e-16)


# ---------------------------------------------------------------- worked example
def test_worked_example_dk2():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_dk2.json")))
    p = custom_problem(ex["q"], ex["k"], ex["v"], ex["a"], ex["b"], ex["A_log"], ex["dt_bias"],
                       [3])
    r = oracle.prefill(p, eps=ex["eps"])
    np.testing.assert_allclose(r.out[:, 0, :], np.array(ex["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r.state_pool[0, 0], np.array(ex["S_after_3"]), rtol=0, atol=1e-15)
    # the first two tokens alone
    p2 = custom_problem(ex["q"][:2], ex["k"][:2], ex["v"][:2], ex["a"][:2], ex["b"][:2],
                        ex["A_log"], ex["dt_bias"], [2])
    r2 = oracle.prefill(p2, eps=ex["eps"])
    np.testing.assert_allclose(r2.state_pool[0, 0], np.array(ex["S_after_2"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_bruteforce_product_form(seed):
    rng = np.random.default_rng(seed)
    T, dk, dv = int(rng.integers(1, 9)), 4, 3
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = rng.standard_normal(T) * 2
    b = rng.standard_normal(T) * 2
    A_log, dt_bias = float(rng.uniform(-1, 2)), float(rng.normal(0, 0.5))
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    p = custom_problem(q, k, v, a, b, A_log, dt_bias, [T], state=S0[None, None])
    r = oracle.prefill(p)
    O_bf, S_bf = bruteforce.forward(p.q[:, 0], p.k[:, 0], p.v[:, 0], p.a[:, 0], p.b[:, 0],
                                    p.A_log[0], p.dt_bias[0], p.state_pool[0, 0])
    assert rel(r.out[:, 0, :], O_bf) < 1e-13
    assert rel(r.state_pool[0, 0], S_bf) < 1e-13


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("seed", [5, 6])
def test_delta_rule_overwrite(seed):
    """beta = 1 and q = k: S_t k_t = v_t for any alpha, S0 and key correlations, so o_t = v_t."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 40, 8, 6
    base = rng.standard_normal(dk)
    k = base + 0.3 * rng.standard_normal((T, dk))      # strongly correlated keys
    v = rng.standard_normal((T, dv))
    a = rng.standard_normal(T) * 3
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    p = custom_problem(k, k, v, a, np.full(T, 1e4), 0.7, 0.1, [T], state=S0[None, None])
    r = oracle.prefill(p, eps=0.0)      # exactly unit keys
    np.testing.assert_allclose(r.out[:, 0, :], p.v[:, 0, :], rtol=0, atol=1e-12)


def test_decay_only():
    """beta = 0: S_t = gamma_t S0 and o_t = gamma_t S0 q_t with gamma_t = prod alpha."""
    rng = np.random.default_rng(7)
    T, dk, dv = 30, 5, 4
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = rng.standard_normal(T) - 2
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    p = custom_problem(q, k, v, a, np.full(T, -1e4), 0.3, -0.2, [T], state=S0[None, None])
    r = oracle.prefill(p)
    x = a.astype(np.float32).astype(np.float64) + np.float64(np.float32(-0.2))
    g = -math.exp(np.float64(np.float32(0.3))) * (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x))))
    gamma = np.exp(np.cumsum(g))
    qn = p.q[:, 0].astype(np.float64)
    qn /= np.sqrt((qn ** 2).sum(1, keepdims=True) + 1e-6)
    S0d = S0.astype(np.float64)
    np.testing.assert_allclose(r.out[:, 0, :], gamma[:, None] * (qn @ S0d.T), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r.state_pool[0, 0], gamma[-1] * S0d, rtol=1e-13, atol=0)


def test_orthogonal_keys_linear_attention():
    """Mutually orthogonal keys and S0 = 0: the erase term never touches earlier
    writes, so S_T = sum_t (gamma_T/gamma_t) beta_t v_t k_t^T (decayed linear
    attention); with alpha = beta = 1 it is sum_t v_t k_t^T."""
    rng = np.random.default_rng(8)
    dk, dv = 12, 5
    T = 9
    perm = rng.permutation(dk)[:T]
    scale = rng.uniform(0.5, 3.0, T) * rng.choice([-1, 1], T)
    k = np.zeros((T, dk))
    k[np.arange(T), perm] = scale
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    a = rng.standard_normal(T)
    b = rng.standard_normal(T)
    p = custom_problem(q, k, v, a, b, 0.2, 0.05, [T])
    r = oracle.prefill(p, eps=0.0)
    g = np.array([oracle.gates(p.a[t, 0], p.b[t, 0], p.A_log[0], p.dt_bias[0])[2] for t in range(T)])
    beta = np.array([oracle.gates(p.a[t, 0], p.b[t, 0], p.A_log[0], p.dt_bias[0])[1] for t in range(T)])
    G = np.cumsum(g)
    kn = np.zeros((T, dk))
    kn[np.arange(T), perm] = np.sign(scale)
    v64 = p.v[:, 0].astype(np.float64)
    S_exp = sum(np.exp(G[-1] - G[t]) * beta[t] * np.outer(v64[t], kn[t]) for t in range(T))
    np.testing.assert_allclose(r.state_pool[0, 0], S_exp, rtol=1e-13, atol=1e-15)
    # alpha = 1 (a = -1e4) and beta = 1 (b = 1e4): plain linear attention sum v k^T
    p1 = custom_problem(q, k, v, np.full(T, -1e4), np.full(T, 1e4), 0.2, 0.0, [T])
    r1 = oracle.prefill(p1, eps=0.0)
    S_lin = sum(np.outer(v64[t], kn[t]) for t in range(T))
    np.testing.assert_allclose(r1.state_pool[0, 0], S_lin, rtol=1e-14, atol=1e-15)
    qn = p.q[:, 0].astype(np.float64)
    qn /= np.linalg.norm(qn, axis=1, keepdims=True)
    o_lin = np.stack([sum(np.outer(v64[s], kn[s]) for s in range(t + 1)) @ qn[t] for t in range(T)])
    np.testing.assert_allclose(r1.out[:, 0, :], o_lin, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- chunk forms
def gentle_problem(seed, lengths, dk, dv, H=1, HV=1, state_std=0.5):
    """Slow decay (a ~ N(-4,1)), so 1/gamma stays finite inside a 128-token chunk."""
    return gdn_synth.make_problem(seed, lengths, H, HV, dk, dv, dtype="f32", a_mean=-4.0,
                                  state_std=state_std)


@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 16, 64, 128])
def test_chunk_forms_equal_recurrence_gentle(C):
    p = gentle_problem(100 + C, [1, 37, 130, 64], 8, 6, H=1, HV=2)
    r = oracle.prefill(p)
    for variant in chunked.VARIANTS:
        out, pool = chunked.problem_forward(p, C, variant)
        assert rel(out, r.out) < 1e-12, variant
        assert rel(pool, r.state_pool) < 1e-12, variant


@pytest.mark.parametrize("C", [4, 16, 64, 128])
def test_chunk_forms_equal_recurrence_strong_decay(C):
    """a ~ N(0,1), exp(A_log) up to 16: the log cumulative gate reaches hundreds
    inside a chunk; only the forms without 1/gamma stay finite."""
    p = gdn_synth.make_problem(200 + C, [200, 65], 1, 2, 8, 6, dtype="f32", state_std=0.5)
    r = oracle.prefill(p)
    for variant in ("two_inverses", "safe"):
        out, pool = chunked.problem_forward(p, C, variant)
        assert rel(out, r.out) < 1e-12, variant
        assert rel(pool, r.state_pool) < 1e-12, variant


def test_save_one_invert_identity():
    """N^-1 = G M^-1 G^-1 ("Simple math to speed up GDN prefill", Save one invert):
    both sides formed independently in fp64."""
    rng = np.random.default_rng(11)
    n, dk = 64, 16
    K = chunked.l2norm_rows(rng.standard_normal((n, dk)) + 0.5, 0.0)
    beta = rng.uniform(0, 1, n)
    alpha = np.exp(-rng.uniform(0.0, 0.08, n))
    gamma = np.cumprod(alpha)
    Gam = np.tril(gamma[:, None] / gamma[None, :])
    KKt = K @ K.T
    M = np.eye(n) + np.tril(np.diag(beta) @ KKt, -1)
    N = np.eye(n) + np.tril(np.diag(beta) @ (Gam * KKt), -1)
    lhs = np.linalg.inv(N)
    rhs = np.diag(gamma) @ np.linalg.inv(M) @ np.diag(1.0 / gamma)
    assert rel(lhs, rhs) < 1e-12
    # and entry by entry: (N^-1)_{ri} = (gamma_r / gamma_i) (M^-1)_{ri}
    assert rel(lhs, Gam * np.linalg.inv(M)) < 1e-12


# ---------------------------------------------------------------- invariants
def test_linearity_in_state_and_values():
    p = gdn_synth.make_problem(21, [50, 17], 1, 1, 8, 8, dtype="f32", state_std=1.0)
    r = oracle.prefill(p)
    c = 4.0                      # exact in fp32
    p2 = gdn_synth.make_problem(21, [50, 17], 1, 1, 8, 8, dtype="f32", state_std=1.0)
    p2.v = p.v * np.float32(c)
    p2.state_pool = p.state_pool * np.float32(c)
    r2 = oracle.prefill(p2)
    np.testing.assert_allclose(r2.out, c * r.out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r2.state_pool, c * r.state_pool, rtol=1e-13, atol=1e-14)


def test_split_invariance_through_slot():
    """One call over [0,T) equals two calls [0,t1) and [t1,T) through the same slot."""
    p = gdn_synth.make_problem(22, [90], 2, 4, 8, 6, dtype="f32", state_std=0.3)
    r = oracle.prefill(p)
    t1 = 37
    first = custom_problem(p.q[:t1], p.k[:t1], p.v[:t1], p.a[:t1], p.b[:t1], p.A_log, p.dt_bias,
                           [t1], H=2, HV=4, state=p.state_pool)
    r1 = oracle.prefill(first)
    second = custom_problem(p.q[t1:], p.k[t1:], p.v[t1:], p.a[t1:], p.b[t1:], p.A_log, p.dt_bias,
                            [90 - t1], H=2, HV=4, state=r1.state_pool.astype(np.float32))
    # fp32 pool between the calls, as on the device; compare to the fp64 path loosely
    r2 = oracle.prefill(second)
    assert rel(np.concatenate([r1.out, r2.out]), r.out) < 1e-6
    assert rel(r2.state_pool, r.state_pool) < 1e-6
    # and exactly in fp64 through the raw entry point
    S0 = p.state_pool.astype(np.float64)[[0]][:, range(4)]
    o1, S1 = oracle.recurrence_raw("f32", p.q[:t1], p.k[:t1], p.v[:t1], p.a[:t1], p.b[:t1],
                                   p.A_log, p.dt_bias, [0, t1], 2, 4, 8, 6, S0, range(4))
    o2, S2 = oracle.recurrence_raw("f32", p.q[t1:], p.k[t1:], p.v[t1:], p.a[t1:], p.b[t1:],
                                   p.A_log, p.dt_bias, [0, 90 - t1], 2, 4, 8, 6, S1, range(4))
    np.testing.assert_array_equal(np.concatenate([o1, o2]), r.out)
    np.testing.assert_array_equal(S2[0], r.state_pool[0])


def test_varlen_packing_and_untouched_slots():
    lengths = [5, 0, 70, 1]
    p = gdn_synth.make_problem(23, lengths, 1, 2, 8, 8, dtype="bf16", pool=7,
                               cache_indices=[6, 2, 0, 4], state_std=0.2)
    r = oracle.prefill(p)
    cu = p.cu_seqlens
    for bi, L in enumerate(lengths):
        single = custom_problem(p.values_f32("q")[cu[bi]:cu[bi + 1]], p.values_f32("k")[cu[bi]:cu[bi + 1]],
                                p.values_f32("v")[cu[bi]:cu[bi + 1]], p.a[cu[bi]:cu[bi + 1]],
                                p.b[cu[bi]:cu[bi + 1]], p.A_log, p.dt_bias, [L], H=1, HV=2,
                                state=p.state_pool[[p.cache_indices[bi]]])
        rs = oracle.prefill(single)
        np.testing.assert_array_equal(rs.out, r.out[cu[bi]:cu[bi + 1]])
        np.testing.assert_array_equal(rs.state_pool[0], r.state_pool[p.cache_indices[bi]])
    untouched = [s for s in range(7) if s not in (6, 0, 4)]   # slot 2 has L = 0
    np.testing.assert_array_equal(r.state_pool[untouched], p.state_pool[untouched].astype(np.float64))


def test_gqa_equals_duplicated_heads():
    """HV = 2H with value head hv reading q/k head hv // 2 equals H' = HV with each
    q/k head duplicated (the head-sharing convention; not fixed by the pages)."""
    p = gdn_synth.make_problem(24, [33, 20], 2, 4, 8, 8, dtype="bf16", state_std=0.2)
    r = oracle.prefill(p)
    dup = gdn_synth.make_problem(24, [33, 20], 2, 4, 8, 8, dtype="bf16", state_std=0.2)
    dup.q = np.repeat(p.q, 2, axis=1)
    dup.k = np.repeat(p.k, 2, axis=1)
    dup.H = 4
    r2 = oracle.prefill(dup)
    np.testing.assert_array_equal(r.out, r2.out)
    np.testing.assert_array_equal(r.state_pool, r2.state_pool)


def test_contraction_bound_per_step():
    """beta in [0,1], unit keys: ||S_t||_2 <= alpha_t ||S_{t-1}||_2 + beta_t ||v_t||
    because I - beta k k^T has spectral norm <= 1."""
    p = gdn_synth.make_problem(25, [60], 1, 1, 6, 5, dtype="f32", state_std=1.0, a_mean=-2.0)
    S = p.state_pool.astype(np.float64)[[0]]
    for t in range(60):
        o, S_new = oracle.recurrence_raw("f32", p.q[t:t + 1], p.k[t:t + 1], p.v[t:t + 1],
                                         p.a[t:t + 1], p.b[t:t + 1], p.A_log, p.dt_bias, [0, 1],
                                         1, 1, 6, 5, S, [0], eps=0.0)
        al, be, _ = oracle.gates(p.a[t, 0], p.b[t, 0], p.A_log[0], p.dt_bias[0])
        lhs = np.linalg.norm(S_new[0, 0], 2)
        rhs = al * np.linalg.norm(S[0, 0], 2) + be * np.linalg.norm(p.v[t, 0].astype(np.float64))
        assert lhs <= rhs * (1 + 1e-12) + 1e-300
        S = S_new


def test_fp32_arithmetic_floor():
    """The same loop in fp32 arithmetic stays within the fp32 tolerances of the fp64 run
    (shows the fp32 bars are reachable)."""
    p = gdn_synth.workload(0)
    r64 = oracle.prefill(p)
    r32 = oracle.prefill(p, fp32_arith=True)
    rms = np.sqrt(np.mean(r64.out ** 2))
    assert np.max(np.abs(r32.out - r64.out)) <= 1e-4 * rms
    assert rel(r32.state_pool, r64.state_pool) <= 1e-5


def test_row_and_head_selection_is_exact():
    """Computing a subset of heads/rows gives bit-identical values (rows of S evolve
    independently), which is what sampled parity at full size relies on."""
    p = gdn_synth.make_problem(26, [40, 25], 2, 4, 16, 32, dtype="bf16", state_std=0.1)
    full = oracle.prefill(p)
    part = oracle.prefill(p, heads=[3, 1], rows=(8, 24))
    np.testing.assert_array_equal(part.out, full.out[:, [3, 1], 8:24])
    np.testing.assert_array_equal(part.state_pool[:, [3, 1], 8:24], full.state_pool[:, [3, 1], 8:24])


def test_empty_batch_and_zero_lengths():
    p = gdn_synth.make_problem(27, [0, 0], 1, 1, 8, 8, dtype="f32", state_std=1.0)
    r = oracle.prefill(p)
    assert r.out.shape == (0, 1, 8)
    np.testing.assert_array_equal(r.state_pool, p.state_pool.astype(np.float64))
