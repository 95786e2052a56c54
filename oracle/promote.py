"""CPU oracle of the Promote update scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. It shares no code with the HIP library.

What it computes: the update stage of one level of the nested model (awehrs.io "NRM
training kernels", section General implementation, Promote algorithm; section Kernel, a
scan over firings split over batch, heads and value blocks). Each (batch, head) scan
holds a dk x dv memory M. At firing f the level receives n pairs together: unit write
keys K_f (n x dk), values V_f (n x dv), erase gates beta_f and write gates w_f (n each),
and one log-decay vector gamma_f (dk, one entry per key row). A firing is the composition
of three linear maps of M, taken in this order:

    M <- diag(exp(gamma_f)) M                 (per-row decay)
    M <- M - K_f^T (beta_f o K_f) M           (gated removal along the n keys)
    M <- M + K_f^T (w_f o V_f)                (gated rank-n write)

The n pairs enter as sums over pairs, so no pair sees another pair of its own firing and
their order does not matter. The probe that derives K, beta, w and gamma from
the level below (dense projections, normalisation, sigmoid, mean of -softplus) is not
part of this stage; its outputs are this stage's inputs.

Arithmetic in fp64 with numpy's matrix product as the only library step. Pinned by
tests/test_oracle_promote.py (closed forms, retrieval with orthonormal keys, pair-order
invariance, and one pair per firing against the token recurrence of the main oracle).
"""
from __future__ import annotations

import numpy as np


def promote_scan(M0, K, V, beta, w, gamma, keep_states: bool = True):
    """Run the scan for every (batch, head).

    M0 [BH, dk, dv]; K [BH, F, n, dk]; V [BH, F, n, dv]; beta, w [BH, F, n];
    gamma [BH, F, dk]. Inputs of any float dtype (bf16 values passed as their exact
    fp32 widening). Returns (M_final [BH, dk, dv], states [BH, F, dk, dv] or None), fp64;
    states[:, f] is the memory after firing f."""
    M = np.array(M0, dtype=np.float64, copy=True)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    BH, F = K.shape[0], K.shape[1]
    states = np.empty((BH, F) + M.shape[1:], dtype=np.float64) if keep_states else None
    for f in range(F):
        Kf = K[:, f]                                          # [BH, n, dk]
        # decay: one factor per key row of the memory
        M = np.exp(gamma[:, f])[:, :, None] * M
        # erase: M - K^T (beta o K) M, every pair against the decayed memory
        M = M - np.matmul(np.swapaxes(Kf, 1, 2), beta[:, f][:, :, None] * np.matmul(Kf, M))
        # write: + K^T (w o V)
        M = M + np.matmul(np.swapaxes(Kf, 1, 2), w[:, f][:, :, None] * V[:, f])
        if keep_states:
            states[:, f] = M
    return M, states
