"""Pins of the fp64 backward oracle (oracle/backward.py) against what the forward fixes.

* Central finite differences (with one Richardson step) of the C oracle's forward -- a
  separate implementation of the recurrence, itself pinned by test_oracle_pins.py -- for
  every input: q, k, v, a, b, A_log, dt_bias and each request's initial state, on ragged
  requests (one empty) with grouped value heads. Inputs and steps are dyadic, so every
  perturbed fp32 input is exact.
* The decay-only closed form (beta = 0): S_t = gamma_t S_0, so dL/dS_0 = gamma_T dS_T +
  sum_t gamma_t dout_t qh_t^T, and dv = dk = 0.
* Linearity in the upstream gradients.
* Planted mistakes (a dropped term, a wrong sign, a wrong index, a transposed operand, a
  missing factor) each fail a pin.
"""
import numpy as np
import pytest

import gdn_synth
import oracle
from oracle import backward as bw

H_STEP = 2.0 ** -10


def _dyadic(x, step=2.0 ** -6, lim=3.0):
    return np.clip(np.round(np.asarray(x, dtype=np.float64) / step) * step, -lim, lim)


def _problem(seed=1, lengths=(5, 0, 7), H=1, HV=2, d=4):
    p = gdn_synth.make_problem(seed, list(lengths), H, HV, d, d, dtype="f32", pool=4,
                               cache_indices=[3, 0, 1][:len(lengths)], state_std=0.5,
                               a_mean=-1.0, b_mean=0.5)
    for name in ("q", "k", "v", "a", "b", "A_log", "dt_bias"):
        setattr(p, name, _dyadic(getattr(p, name)).astype(np.float32))
    p.A_log = np.abs(p.A_log) + np.float32(0.25)
    p.state_pool = _dyadic(p.state_pool).astype(np.float32)
    return p


def _upstream(p, seed=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((p.N, p.HV, p.dv)),
            rng.standard_normal((p.B, p.HV, p.dv, p.dk)))


def _loss(p, dout, dstate, S0=None):
    """L = <dout, out> + sum_b <dstate_b, S_b final>, from the C oracle (fp64 arithmetic)."""
    idx = np.asarray(p.cache_indices)
    if S0 is None:
        S0 = p.state_pool.astype(np.float64)[idx]
    out, S = oracle.recurrence_raw("f32", p.q, p.k, p.v, p.a, p.b, p.A_log, p.dt_bias,
                                   p.cu_seqlens, p.H, p.HV, p.dk, p.dv, S0, list(range(p.HV)))
    return float(np.sum(out * dout) + np.sum(S * dstate))


def _fd(f, h):
    """Central difference with one Richardson step: O(h^4)."""
    d1 = (f(h) - f(-h)) / (2 * h)
    d2 = (f(h / 2) - f(-h / 2)) / h
    return (4 * d2 - d1) / 3


def _check_fd(p, g, dout, dstate, tol=1e-8):
    worst = {}
    for name, grad in (("q", g.dq), ("k", g.dk), ("v", g.dv), ("a", g.da), ("b", g.db),
                       ("A_log", g.dA_log), ("dt_bias", g.ddt_bias)):
        base = getattr(p, name).copy()
        for e in np.ndindex(base.shape):
            def f(h):
                x = base.copy()
                x[e] = np.float32(x[e] + h)
                setattr(p, name, x)
                return _loss(p, dout, dstate)
            fd = _fd(f, H_STEP)
            setattr(p, name, base)
            err = abs(fd - grad[e]) / (1.0 + abs(fd))
            worst[name] = max(worst.get(name, 0.0), err)
    S0 = p.state_pool.astype(np.float64)[np.asarray(p.cache_indices)]
    for e in np.ndindex(S0.shape):
        def f(h):
            x = S0.copy()
            x[e] += h
            return _loss(p, dout, dstate, S0=x)
        fd = _fd(f, H_STEP)
        worst["state0"] = max(worst.get("state0", 0.0),
                              abs(fd - g.dstate0[e]) / (1.0 + abs(fd)))
    bad = {k_: v_ for k_, v_ in worst.items() if not v_ <= tol}
    return worst, bad


def test_finite_differences_of_every_input():
    p = _problem()
    dout, dstate = _upstream(p)
    g = bw.prefill_backward(p, dout, dstate)
    worst, bad = _check_fd(p, g, dout, dstate)
    assert not bad, worst
    # the empty request passes its state gradient through unchanged
    np.testing.assert_array_equal(g.dstate0[1], dstate[1])


def test_finite_differences_gqa4_and_longer_requests():
    p = _problem(seed=5, lengths=(9, 3), H=1, HV=4, d=4)
    dout, dstate = _upstream(p, seed=6)
    g = bw.prefill_backward(p, dout, dstate)
    worst, bad = _check_fd(p, g, dout, dstate)
    assert not bad, worst


def test_decay_only_closed_form():
    """beta = 0 (b = -1e4): S_t = gamma_t S_0, out_t = gamma_t S_0 qh_t."""
    p = _problem(seed=7, lengths=(6,), HV=1)
    p.b[:] = -1e4
    dout, dstate = _upstream(p, seed=8)
    g = bw.prefill_backward(p, dout, dstate)
    alpha = np.array([oracle.gates(p.a[t, 0], p.b[t, 0], p.A_log[0], p.dt_bias[0])[0]
                      for t in range(p.N)])
    gam = np.cumprod(alpha)
    q = p.q[:, 0].astype(np.float64)
    qh = q / np.sqrt((q * q).sum(axis=1) + bw.EPS)[:, None]
    want = gam[-1] * dstate[0, 0] + sum(gam[t] * np.outer(dout[t, 0], qh[t]) for t in range(p.N))
    np.testing.assert_allclose(g.dstate0[0, 0], want, rtol=1e-13, atol=1e-13)
    assert np.all(g.dv == 0) and np.all(g.dk == 0) and np.all(g.db == 0)


def test_linear_in_the_upstream_gradients():
    p = _problem(seed=9)
    d1, s1 = _upstream(p, seed=10)
    d2, s2 = _upstream(p, seed=11)
    g1 = bw.prefill_backward(p, d1, s1)
    g2 = bw.prefill_backward(p, d2, s2)
    g12 = bw.prefill_backward(p, d1 + 2 * d2, s1 + 2 * s2)
    for name in ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dstate0"):
        np.testing.assert_allclose(getattr(g12, name),
                                   getattr(g1, name) + 2 * getattr(g2, name), rtol=1e-10,
                                   atol=1e-12)


MUTANTS = {
    "dropped erase term in dS_prev": ("D = alpha[t] * (D - beta[t] * np.outer(Dk, kh[t]))",
                                      "D = alpha[t] * D"),
    "wrong sign in dbeta": ("dbeta[t] = Dk @ (vs[t] - alpha[t] * Spk)",
                            "dbeta[t] = Dk @ (vs[t] + alpha[t] * Spk)"),
    "dropped symmetric term in dkh": ("(D.T @ Spk + Sp.T @ Dk)", "(D.T @ Spk)"),
    "read before write in dqh": ("dqh[t] = S[t + 1].T @ do", "dqh[t] = S[t].T @ do"),
    "wrong state in dalpha": ("np.sum(D * Sp)", "np.sum(D * S[t + 1])"),
    "missing beta in dv": ("g.dv[t0 + t, hv] = beta[t] * Dk", "g.dv[t0 + t, hv] = Dk"),
    "wrong sign in the norm chain rule": ("dqh / nq[:, None] - qs", "dqh / nq[:, None] + qs"),
    "missing exp(A_log) in dA_log": ("(dalpha * (-alpha * A * _softplus(x)))",
                                     "(dalpha * (-alpha * _softplus(x)))"),
    "transposed operand in dkh": ("beta[t] * (D.T @ vs[t])", "beta[t] * (D @ vs[t])"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_fail_a_pin(name):
    import types
    old, new = MUTANTS[name]
    src = open(bw.__file__).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType("backward_mutant")
    exec(compile(src.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    p = _problem()
    dout, dstate = _upstream(p)
    g = mod.prefill_backward(p, dout, dstate)
    _, bad = _check_fd(p, g, dout, dstate)
    assert bad, f"mutant '{name}' passed every finite-difference pin"
