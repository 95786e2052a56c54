"""Pins of the Promote update-scan oracle (awehrs.io "NRM training kernels", Promote):
closed forms, retrieval at orthonormal keys, the order-free (simultaneous) writes the
page defines, and one pair per firing against the token recurrence of the main oracle."""
import math

import numpy as np
import pytest

import gdn_synth
import oracle
from oracle.promote import promote_scan


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rel(x, y):
    return float(np.linalg.norm(np.asarray(x) - np.asarray(y)) / np.linalg.norm(y))


def test_decay_only():
    """beta = w = 0: M_F = diag(exp(sum_f gamma_f)) M0, and every kept state likewise."""
    rng = np.random.default_rng(41)
    BH, F, n, dk, dv = 3, 5, 4, 8, 6
    K = unit_rows(rng.standard_normal((BH, F, n, dk)))
    gamma = -rng.uniform(0, 1, (BH, F, dk))
    M0 = rng.standard_normal((BH, dk, dv))
    z = np.zeros((BH, F, n))
    M, states = promote_scan(M0, K, rng.standard_normal((BH, F, n, dv)), z, z, gamma)
    np.testing.assert_allclose(M, np.exp(gamma.sum(1))[:, :, None] * M0, rtol=1e-14, atol=0)
    np.testing.assert_allclose(states[:, 2], np.exp(gamma[:, :3].sum(1))[:, :, None] * M0,
                               rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", [42, 43])
def test_orthonormal_keys_store_values(seed):
    """Orthonormal keys (K_f K_f^T = I), no decay: after firing f,
    K_f M_f = (1 - beta_f) o (K_f M_{f-1}) + w_f o V_f row by row, and the part of M outside
    the keys' span is unchanged. At beta = w = 1 each key retrieves exactly its own value."""
    rng = np.random.default_rng(seed)
    BH, F, n, dk, dv = 2, 4, 5, 12, 7
    K = np.empty((BH, F, n, dk))
    for b in range(BH):
        for f in range(F):
            q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
            K[b, f] = q[:n]
    V = rng.standard_normal((BH, F, n, dv))
    M0 = rng.standard_normal((BH, dk, dv))
    for bet, wr in ((rng.uniform(0, 1, (BH, F, n)), rng.uniform(0, 1, (BH, F, n))),
                    (np.ones((BH, F, n)), np.ones((BH, F, n)))):
        M, states = promote_scan(M0, K, V, bet, wr, np.zeros((BH, F, dk)))
        prev = M0
        for f in range(F):
            expect = (1 - bet[:, f])[:, :, None] * (K[:, f] @ prev) + wr[:, f][:, :, None] * V[:, f]
            np.testing.assert_allclose(K[:, f] @ states[:, f], expect, rtol=0, atol=1e-12)
            P = np.eye(dk) - np.swapaxes(K[:, f], 1, 2) @ K[:, f]   # projector off the keys
            np.testing.assert_allclose(P @ states[:, f], P @ prev, rtol=0, atol=1e-12)
            prev = states[:, f]
    np.testing.assert_allclose(K[:, -1] @ M, V[:, -1], rtol=0, atol=1e-12)


def test_pairs_are_order_free():
    """The pairs of a firing act on the state as it stood before the firing: permuting
    them within each firing changes nothing (up to rounding)."""
    p = gdn_synth.make_promote_problem(44, 2, 6, 16, 32, 24, dtype="f32")
    M, S = promote_scan(p.M0, p.K, p.V, p.beta, p.w, p.gamma)
    perm = np.random.default_rng(45).permutation(16)
    M2, S2 = promote_scan(p.M0, p.K[:, :, perm], p.V[:, :, perm], p.beta[:, :, perm],
                          p.w[:, :, perm], p.gamma)
    assert rel(M2, M) < 1e-13 and rel(S2, S) < 1e-13


def gates_for(g, beta):
    """Raw a, b of the main oracle's gate (A_log = 0, dt_bias = 0) for log-decay g < 0 and
    erase gate beta, and the exact gates the recurrence then uses."""
    a = np.float32(math.log(math.expm1(-g)))       # softplus(a) = -g
    b = np.float32(math.log(beta / (1.0 - beta)))  # sigmoid(b) = beta
    al, be, gg = oracle.gates(float(a), float(b), 0.0, 0.0)
    return a, b, gg, be


@pytest.mark.parametrize("seed", [46, 47])
def test_one_pair_per_firing_is_the_token_recurrence(seed):
    """n = 1, a uniform log-decay g and w = beta: a firing is one step of the gated delta
    rule with M = S^T ("Simple math to speed up GDN prefill", Reminder), so F firings equal
    the main oracle's recurrence over F tokens."""
    rng = np.random.default_rng(seed)
    F, dk, dv = 9, 6, 5
    k = unit_rows(rng.standard_normal((F, dk)))
    v = rng.standard_normal((F, dv)).astype(np.float32)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    a = np.empty(F, np.float32)
    b = np.empty(F, np.float32)
    g = np.empty(F)
    be = np.empty(F)
    for t in range(F):
        a[t], b[t], g[t], be[t] = gates_for(-rng.uniform(0.05, 1.0), rng.uniform(0.1, 0.9))
    q = rng.standard_normal((F, dk)).astype(np.float32)
    k32 = k.astype(np.float32)
    _, S = oracle.recurrence_raw("f32", q[:, None], k32[:, None], v[:, None], a[:, None],
                                 b[:, None], np.zeros(1, np.float32), np.zeros(1, np.float32),
                                 [0, F], 1, 1, dk, dv, S0.astype(np.float64)[None, None], [0],
                                 eps=0.0)
    kk = unit_rows(k32.astype(np.float64))          # the recurrence normalises k again
    M, _ = promote_scan(S0.T[None].astype(np.float64), kk[None, :, None], v[None, :, None],
                        be[None, :, None], be[None, :, None], np.repeat(g[None, :, None], dk, 2))
    np.testing.assert_allclose(M[0], S[0, 0].T, rtol=0, atol=1e-12)


def test_simultaneous_is_not_sequential():
    """Two correlated pairs in one firing differ from the same pairs written one after the
    other (the page's point that higher levels are a different operation); with orthogonal
    keys and no decay the two agree."""
    rng = np.random.default_rng(48)
    dk, dv = 8, 4
    k1 = unit_rows(rng.standard_normal(dk))
    k2 = unit_rows(k1 + 0.5 * rng.standard_normal(dk))
    V = rng.standard_normal((2, dv))
    bet = np.array([0.7, 0.6])
    M0 = rng.standard_normal((dk, dv))

    def sequential(ka, kb):
        M = M0.copy()
        for kv, vv, b_ in ((ka, V[0], bet[0]), (kb, V[1], bet[1])):
            M = M - b_ * np.outer(kv, kv @ M) + b_ * np.outer(kv, vv)
        return M

    def simultaneous(ka, kb):
        K = np.stack([ka, kb])[None, None]
        M, _ = promote_scan(M0[None], K, V[None, None], bet[None, None], bet[None, None],
                            np.zeros((1, 1, dk)))
        return M[0]

    assert rel(simultaneous(k1, k2), sequential(k1, k2)) > 1e-2
    q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    np.testing.assert_allclose(simultaneous(q[0], q[1]), sequential(q[0], q[1]), rtol=0,
                               atol=1e-13)


def test_generator_shapes_and_ranges():
    p = gdn_synth.make_promote_problem(49, 2, 3, 16, 64, 128, dtype="bf16")
    assert p.K.shape == (2, 3, 16, 64) and p.V.shape == (2, 3, 16, 128)
    assert p.gamma.shape == (2, 3, 64) and p.M0.shape == (2, 64, 128)
    assert np.all(p.gamma <= 0) and np.all((p.beta >= 0) & (p.beta < 1))
    kn = np.linalg.norm(p.values_f32("K").astype(np.float64), axis=-1)
    assert np.all(np.abs(kn - 1) < 1e-2)


# ---------------------------------------------------------------- planted mistakes
import inspect

import oracle.promote as _promote_mod

MUTANTS = {
    "no decay": ("M = np.exp(gamma[:, f])[:, :, None] * M", "M = M"),
    "decay on value columns": ("np.exp(gamma[:, f])[:, :, None] * M",
                               "np.exp(gamma[:, f])[:, None, :] * M"),
    "erase sign": ("M = M - np.matmul(np.swapaxes(Kf, 1, 2), beta",
                   "M = M + np.matmul(np.swapaxes(Kf, 1, 2), beta"),
    "erase with w": ("beta[:, f][:, :, None] * np.matmul(Kf, M)", "w[:, f][:, :, None] * np.matmul(Kf, M)"),
    "write with beta": ("w[:, f][:, :, None] * V[:, f]", "beta[:, f][:, :, None] * V[:, f]"),
    "no write": ("M = M + np.matmul(np.swapaxes(Kf, 1, 2), w[:, f][:, :, None] * V[:, f])", "M = M"),
    "erase after write": (
        "        M = M - np.matmul(np.swapaxes(Kf, 1, 2), beta[:, f][:, :, None] * np.matmul(Kf, M))\n"
        "        # write: + K^T (w o V)\n"
        "        M = M + np.matmul(np.swapaxes(Kf, 1, 2), w[:, f][:, :, None] * V[:, f])",
        "        M = M + np.matmul(np.swapaxes(Kf, 1, 2), w[:, f][:, :, None] * V[:, f])\n"
        "        M = M - np.matmul(np.swapaxes(Kf, 1, 2), beta[:, f][:, :, None] * np.matmul(Kf, M))"),
}


def _mutant(old, new):
    src = inspect.getsource(_promote_mod)
    assert src.count(old) == 1, old
    ns = {}
    exec(compile(src.replace(old, new), "promote_mutant", "exec"), ns)
    return ns["promote_scan"]


def _pins_pass(fn):
    """The pins above, run against fn; False as soon as one fails (or fn raises)."""
    global promote_scan
    saved = promote_scan
    promote_scan = fn
    try:
        for t in (test_decay_only, lambda: test_orthonormal_keys_store_values(42),
                  test_pairs_are_order_free, lambda: test_one_pair_per_firing_is_the_token_recurrence(46),
                  test_simultaneous_is_not_sequential):
            try:
                t()
            except Exception:
                return False
        return True
    finally:
        promote_scan = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name):
    assert _pins_pass(promote_scan)
    assert not _pins_pass(_mutant(*MUTANTS[name])), f"mutant '{name}' passes every pin"
