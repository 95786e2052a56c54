"""Brute-force GDN forward on tiny inputs in 40-digit arithmetic -- TEST INFRASTRUCTURE ONLY.

Instead of the rank-1 update loop, this forms each token's transition matrix
A_t = alpha_t (I - beta_t k_t k_t^T) (dk x dk) and the closed product form of the
state-transition equation in "Simple math to speed up GDN prefill" (veitner),
section Reminder:
    S_t = S_0 A_1 ... A_t + sum_{s<=t} beta_s v_s k_s^T A_{s+1} ... A_t,
then reads o_t = S_t q_t. Gates and norms are recomputed here with mpmath.
"""
from __future__ import annotations

import mpmath as mp
import numpy as np


def _vec(x):
    return mp.matrix([mp.mpf(float(t)) for t in x])


def forward(q, k, v, a, b, A_log, dt_bias, S0, eps=1e-6, dps=40):
    """One sequence, one head. q, k: [T, dk]; v: [T, dv]; a, b: [T] (floats);
    S0: [dv, dk]. Returns (O [T, dv], S_T [dv, dk]) as float64 arrays."""
    with mp.workdps(dps):
        T, dk = np.asarray(k).shape
        dv = np.asarray(v).shape[1]
        I = mp.eye(dk)
        qs, ks, As, writes = [], [], [], []
        for t in range(T):
            qt, kt, vt = _vec(q[t]), _vec(k[t]), _vec(v[t])
            nq = mp.sqrt(sum(x * x for x in qt) + mp.mpf(eps))
            nk = mp.sqrt(sum(x * x for x in kt) + mp.mpf(eps))
            qt = qt / nq
            kt = kt / nk
            x = mp.mpf(float(a[t])) + mp.mpf(float(dt_bias))
            alpha = mp.exp(-mp.exp(mp.mpf(float(A_log))) * mp.log(1 + mp.exp(x)))
            beta = 1 / (1 + mp.exp(-mp.mpf(float(b[t]))))
            As.append(alpha * (I - beta * (kt * kt.T)))
            writes.append(beta * (vt * kt.T))
            qs.append(qt)
        S0m = mp.matrix(dv, dk)
        for i in range(dv):
            for j in range(dk):
                S0m[i, j] = mp.mpf(float(S0[i][j]))
        O = np.zeros((T, dv))
        S = None
        for t in range(T):
            # S_t = S_0 A_1..A_t + sum_{s<=t} write_s A_{s+1}..A_t
            prod = mp.eye(dk)
            for s in range(t + 1):
                prod = prod * As[s]
            S = S0m * prod
            for s in range(t + 1):
                tail = mp.eye(dk)
                for u in range(s + 1, t + 1):
                    tail = tail * As[u]
                S = S + writes[s] * tail
            o = S * qs[t]
            O[t] = [float(o[i]) for i in range(dv)]
        ST = np.array([[float(S[i, j]) for j in range(dk)] for i in range(dv)]) if S is not None \
            else np.array(S0, dtype=np.float64)
        return O, ST
