"""Chunkwise forms of the GDN forward in fp64 -- TEST INFRASTRUCTURE ONLY.

These evaluate the chunked method's equations, one (sequence, value head) at a time,
so the oracle's self-checks can show that the chunked method and the token recurrence
agree (awehrs.io "NRM training kernels", General implementation
item 1: at level 0 the chunkwise algorithm gives what sequential application
gives). Row convention: S is dv x dk; K, Q are n x dk with tokens as rows; V is
n x dv.

Variants (all must agree with the recurrence):

* ``two_inverses`` -- "Simple math to speed up GDN prefill" (veitner), section
  Reminder: W = M^-1 B K and U~ = N^-1 B V with N = I + tril(B (Gamma o K K^T), -1)
  formed and inverted on its own, Gamma^{r,i} = prod_{j=i+1..r} alpha_j, and the
  chunk transition S' = S-> + (U~ - W<- S^T)^T K->.
* ``saved_inverse`` -- same page, section Save one invert: N^-1 = G M^-1 G^-1 with
  the diagonal matrices G = diag(gamma), G^-1 = diag(1/gamma) taken literally
  (finite only while gamma does not underflow).
* ``decay_divided`` -- the form of the pymllm gdn_chunkwise page (section Algorithm): values
  divided by the cumulative decay before the WY solve, u~ = M^-1 B G^-1 V, with the
  decay multiplied back in the output and state equations.
  The extracted w_i recursion is ill-typed; it is read as the matrix form of the
  Reminder section, (I + tril(B K K^T, -1)) W = B K.
* ``safe`` -- the same map with every decay written as exp of a non-positive
  difference of chunk-local log cumulative gates, (N^-1)_{ri} = exp(G_r - G_i) (M^-1)_{ri}
  (the Save-one-invert identity applied entry by entry).

The decorations follow the Reminder section's transition: W<- = diag(gamma) W,
K-> = diag(gamma_n / gamma) K, S-> = gamma_n S. The output rule (not written on
page 4) is page 3's step 2 in row convention,
o_r = gamma_r S q_r + sum_{i<=r} (gamma_r/gamma_i)(q_r . k_i)(u~_i - gamma_i S w_i).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

VARIANTS = ("two_inverses", "saved_inverse", "decay_divided", "safe")


def l2norm_rows(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def log_gates(a, b, A_log, dt_bias):
    """g = log(alpha) = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), in fp64
    (pymllm gdn_chunkwise page, Module Contents: a is the raw decay-gate input before
    softplus/exp, b the raw update-gate input before sigmoid)."""
    x = np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64)
    sp = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    g = -np.exp(np.asarray(A_log, np.float64)) * sp
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64)))
    return g, beta


def unit_lower_inverse(M: np.ndarray) -> np.ndarray:
    n = M.shape[0]
    return solve_triangular(M, np.eye(n), lower=True, unit_diagonal=True)


def chunk_step(S, Q, K, V, g, beta, variant: str):
    """One chunk of n <= C tokens from state S. Returns (O [n, dv], S_new [dv, dk])."""
    n = K.shape[0]
    I = np.eye(n)
    Bm = np.diag(beta)
    KKt = K @ K.T
    QKt = Q @ K.T
    low_incl = np.tril(np.ones((n, n)))
    M = I + np.tril(Bm @ KKt, -1)
    if variant == "two_inverses":
        alpha = np.exp(g)
        gamma = np.cumprod(alpha)                      # gamma^r = prod_{j<=r} alpha^j
        Gam = np.zeros((n, n))
        for r in range(n):
            for i in range(r + 1):
                Gam[r, i] = np.prod(alpha[i + 1:r + 1])  # prod_{j=i+1..r}; empty product = 1
        Minv = unit_lower_inverse(M)
        W = Minv @ Bm @ K
        Nm = I + np.tril(Bm @ (Gam * KKt), -1)
        Ut = unit_lower_inverse(Nm) @ Bm @ V
        Wl = np.diag(gamma) @ W
        Kr = np.diag(Gam[-1]) @ K                      # gamma_n / gamma_i = Gamma^{n,i}
        U = Ut - Wl @ S.T
        S_new = gamma[-1] * S + U.T @ Kr
        O = np.diag(gamma) @ Q @ S.T + (Gam * low_incl * QKt) @ U
        return O, S_new
    if variant == "saved_inverse":
        gamma = np.cumprod(np.exp(g))
        Gd, Gi = np.diag(gamma), np.diag(1.0 / gamma)
        Minv = unit_lower_inverse(M)
        Ninv = Gd @ Minv @ Gi
        W = Minv @ Bm @ K
        Ut = Ninv @ Bm @ V
        Gam = (gamma[:, None] / gamma[None, :]) * low_incl
        U = Ut - Gd @ W @ S.T
        S_new = gamma[-1] * S + U.T @ (np.diag(gamma[-1] / gamma) @ K)
        O = Gd @ Q @ S.T + (Gam * QKt) @ U
        return O, S_new
    if variant == "decay_divided":
        gamma = np.cumprod(np.exp(g))
        dk, dv = K.shape[1], V.shape[1]
        W = np.zeros((n, dk))
        Ut = np.zeros((n, dv))
        for i in range(n):
            W[i] = beta[i] * K[i] - beta[i] * (K[:i] @ K[i]) @ W[:i]
            Ut[i] = (beta[i] / gamma[i]) * V[i] - beta[i] * (K[:i] @ K[i]) @ Ut[:i]
        tri = low_incl * QKt                            # causal mask j <= r
        O = np.diag(gamma) @ (Q @ S.T - tri @ (W @ S.T) + tri @ Ut)
        S_new = gamma[-1] * (S - S @ W.T @ K + Ut.T @ K)
        return O, S_new
    if variant == "safe":
        G = np.cumsum(g)
        D = G[:, None] - G[None, :]
        Gam = np.where(low_incl > 0, np.exp(np.minimum(D, 0.0)), 0.0)
        T = unit_lower_inverse(M)
        Wl = np.diag(np.exp(G)) @ T @ Bm @ K
        Ut = (Gam * T) @ Bm @ V
        U = Ut - Wl @ S.T
        S_new = np.exp(G[-1]) * S + U.T @ (np.diag(np.exp(G[-1] - G)) @ K)
        O = np.diag(np.exp(G)) @ Q @ S.T + (Gam * QKt) @ U
        return O, S_new
    raise ValueError(variant)


def sequence_forward(qn, kn, v, g, beta, S0, C: int, variant: str = "safe"):
    """Chunks [0,C), [C,2C), ... of one sequence; the last one may be partial.
    qn, kn: [T, dk] normalised; v: [T, dv]; g, beta: [T]; S0: [dv, dk]."""
    T = kn.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        O[s:e], S = chunk_step(S, qn[s:e], kn[s:e], v[s:e], g[s:e], beta[s:e], variant)
    return O, S


def problem_forward(p, C: int, variant: str = "safe", eps: float = 1e-6):
    """All sequences and value heads of a gdn_synth.Problem through the chunk form.
    Returns (out [N, HV, dv], new state_pool fp64)."""
    q = l2norm_rows(p.values_f32("q"), eps)
    k = l2norm_rows(p.values_f32("k"), eps)
    v = p.values_f32("v").astype(np.float64)
    out = np.zeros((p.N, p.HV, p.dv))
    pool = p.state_pool.astype(np.float64)
    grp = p.HV // p.H
    for bi in range(p.B):
        t0, t1 = int(p.cu_seqlens[bi]), int(p.cu_seqlens[bi + 1])
        slot = int(p.cache_indices[bi])
        for hv in range(p.HV):
            h = hv // grp
            g, beta = log_gates(p.a[t0:t1, hv], p.b[t0:t1, hv], p.A_log[hv], p.dt_bias[hv])
            O, S = sequence_forward(q[t0:t1, h], k[t0:t1, h], v[t0:t1, hv], g, beta,
                                    pool[slot, hv], C, variant)
            out[t0:t1, hv] = O
            pool[slot, hv] = S
    return out, pool
