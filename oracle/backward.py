"""Backward of the GDN prefill in fp64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this module. It shares no code with the HIP library.

What it computes: the gradients of a scalar loss

    L = sum_t <dout_t, out_t> + sum_b <dstate_b, S_b(final)>

with respect to every input of a prefill call (q, k, v, a, b, A_log, dt_bias and each
request's initial state), given the upstream gradients ``dout`` [N, HV, dv] and
``dstate`` [B, HV, dv, dk]. The forward is the token recurrence (state-transition
equation of "Simple math to speed up GDN prefill", section Reminder), with the gates and
normalisation of the pymllm gdn_chunkwise page (Module Contents):

    qh = q / sqrt(|q|^2 + eps),  kh = k / sqrt(|k|^2 + eps)
    x  = a + dt_bias,  alpha = exp(-exp(A_log) softplus(x)),  beta = sigmoid(b)
    S_t = alpha S_{t-1} - alpha beta (S_{t-1} kh) kh^T + beta v kh^T,   out_t = S_t qh

The chunked forward reaches the same map (awehrs.io "NRM training kernels", General
implementation: at level 0 the chunkwise algorithm gives what sequential application
gives), so these are also the gradients of the chunked forward; the awehrs page's Results
note that this sequential structure is what makes the GDN backward expensive.

Reverse mode, one (request, value head) at a time: a forward sweep keeps every S_t, then
a reverse sweep carries D = dL/dS_t. With Sp = S_{t-1}, for each token from the last:

    D     += dout_t qh^T                      (out_t = S_t qh)
    dqh    = S_t^T dout_t
    dv     = beta D kh
    dbeta  = (D kh) . (v - alpha Sp kh)
    dalpha = <D, Sp> - beta (D kh) . (Sp kh)
    dkh    = -alpha beta (D^T Sp + Sp^T D) kh + beta D^T v
    D     <- alpha (D - beta (D kh) kh^T)     (dL/dS_{t-1})

and the chain rule through the normalisation (dq = dqh / n - q (q . dqh) / n^3 with
n = sqrt(|q|^2 + eps)), the sigmoid (dbeta/db = beta (1 - beta)) and the decay
(dalpha/dx = -alpha exp(A_log) sigmoid(x), dalpha/dA_log = -alpha exp(A_log) softplus(x)).
q and k gradients of a q/k head sum over the value heads that share it (hv // (HV/H)).

Arithmetic in fp64 with plain numpy; pinned by tests/test_oracle_backward.py (central
finite differences of the C oracle's forward, the decay-only closed form, linearity in the
upstream gradients, planted mistakes).
"""
from __future__ import annotations

import dataclasses

import numpy as np

EPS = 1e-6


@dataclasses.dataclass
class Grads:
    dq: np.ndarray        # [N, H, dk]
    dk: np.ndarray        # [N, H, dk]
    dv: np.ndarray        # [N, HV, dv]
    da: np.ndarray        # [N, HV]
    db: np.ndarray        # [N, HV]
    dA_log: np.ndarray    # [HV]
    ddt_bias: np.ndarray  # [HV]
    dstate0: np.ndarray   # [B, HV, dv, dk]: gradient w.r.t. each request's initial state


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _sigmoid(x):
    e = np.exp(-np.abs(x))  # never overflows
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def prefill_backward(p, dout, dstate, eps: float = EPS) -> Grads:
    """Gradients of L (see the module docstring) for the prefill call on the
    ``gdn_synth.Problem`` ``p``. dout [N, HV, dv]; dstate [B, HV, dv, dk] (the gradient of
    each request's final state, request order). Inputs of any float dtype; fp64 result."""
    q = p.values_f32("q").astype(np.float64)
    k = p.values_f32("k").astype(np.float64)
    v = p.values_f32("v").astype(np.float64)
    a = np.asarray(p.a, dtype=np.float64)
    bb = np.asarray(p.b, dtype=np.float64)
    A_log = np.asarray(p.A_log, dtype=np.float64)
    dt_bias = np.asarray(p.dt_bias, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    dstate = np.asarray(dstate, dtype=np.float64)
    cu = np.asarray(p.cu_seqlens, dtype=np.int64)
    H, HV, dk, dv = p.H, p.HV, p.dk, p.dv
    grp = HV // H
    N, B = int(cu[-1]), len(cu) - 1
    g = Grads(dq=np.zeros((N, H, dk)), dk=np.zeros((N, H, dk)), dv=np.zeros((N, HV, dv)),
              da=np.zeros((N, HV)), db=np.zeros((N, HV)), dA_log=np.zeros(HV),
              ddt_bias=np.zeros(HV), dstate0=np.zeros((B, HV, dv, dk)))
    pool = np.asarray(p.state_pool, dtype=np.float64)
    for bi in range(B):
        t0, t1 = int(cu[bi]), int(cu[bi + 1])
        T = t1 - t0
        slot = int(p.cache_indices[bi])
        for hv in range(HV):
            h = hv // grp
            qs, ks = q[t0:t1, h], k[t0:t1, h]
            nq = np.sqrt((qs * qs).sum(axis=1) + eps)
            nk = np.sqrt((ks * ks).sum(axis=1) + eps)
            qh, kh = qs / nq[:, None], ks / nk[:, None]
            x = a[t0:t1, hv] + dt_bias[hv]
            A = np.exp(A_log[hv])
            alpha = np.exp(-A * _softplus(x))
            beta = _sigmoid(bb[t0:t1, hv])
            vs = v[t0:t1, hv]
            # forward sweep, keeping S_0 .. S_T
            S = np.empty((T + 1, dv, dk))
            S[0] = pool[slot, hv]
            for t in range(T):
                Sp = S[t]
                S[t + 1] = (alpha[t] * Sp - alpha[t] * beta[t] * np.outer(Sp @ kh[t], kh[t])
                            + beta[t] * np.outer(vs[t], kh[t]))
            # reverse sweep
            D = dstate[bi, hv].copy()
            dqh = np.zeros((T, dk))
            dkh = np.zeros((T, dk))
            dalpha = np.zeros(T)
            dbeta = np.zeros(T)
            for t in range(T - 1, -1, -1):
                do = dout[t0 + t, hv]
                D += np.outer(do, qh[t])
                dqh[t] = S[t + 1].T @ do
                Sp = S[t]
                Dk = D @ kh[t]
                Spk = Sp @ kh[t]
                g.dv[t0 + t, hv] = beta[t] * Dk
                dbeta[t] = Dk @ (vs[t] - alpha[t] * Spk)
                dalpha[t] = np.sum(D * Sp) - beta[t] * (Dk @ Spk)
                dkh[t] = (-alpha[t] * beta[t] * (D.T @ Spk + Sp.T @ Dk)
                          + beta[t] * (D.T @ vs[t]))
                D = alpha[t] * (D - beta[t] * np.outer(Dk, kh[t]))
            g.dstate0[bi, hv] = D
            # chain rule: normalisation (summed over the value heads of this q/k head)
            g.dq[t0:t1, h] += dqh / nq[:, None] - qs * ((qs * dqh).sum(axis=1) / nq ** 3)[:, None]
            g.dk[t0:t1, h] += dkh / nk[:, None] - ks * ((ks * dkh).sum(axis=1) / nk ** 3)[:, None]
            # gates
            g.db[t0:t1, hv] = dbeta * beta * (1.0 - beta)
            dx = dalpha * (-alpha * A * _sigmoid(x))
            g.da[t0:t1, hv] = dx
            g.ddt_bias[hv] += dx.sum()
            g.dA_log[hv] += (dalpha * (-alpha * A * _softplus(x))).sum()
    return g
