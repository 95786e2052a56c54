"""GPU parity of the Promote update scan (gdn_promote_scan through the C ABI) against
the CPU oracle (oracle/promote.py) on the same seeded inputs. Bar, as for the bf16 state
of the prefill: for every scan, the final memory and every kept state within 1e-3
relative Frobenius error of the oracle's."""
import time

import numpy as np
import pytest

import gdn_synth
from gpu_util import announce
from oracle.promote import promote_scan

pytestmark = pytest.mark.gpu
TOL = 1e-3


def to_device(p):
    import torch

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to("cuda:0")

    return dict(K=t(p.K.view(np.int16), torch.bfloat16), V=t(p.V.view(np.int16), torch.bfloat16),
                beta=t(p.beta), w=t(p.w), gamma=t(p.gamma), M=t(p.M0.copy()))


def run(p, label, keep_states=True):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    d = to_device(p)
    BH, F, n, dk, dv = p.shape
    announce(f"{label} gdn_promote_scan BH={BH} F={F} n={n} dk={dk} dv={dv} seed={p.seed}")
    t0 = time.time()
    states = gdn.gdn_promote_scan(d["K"], d["V"], d["beta"], d["w"], d["gamma"], d["M"],
                                  keep_states=keep_states)
    torch.cuda.synchronize()
    announce(f"{label} done in {time.time() - t0:.3f}s")
    return d["M"].cpu().numpy(), None if states is None else states.cpu().numpy()


def oracle_of(p, scans=None):
    sel = slice(None) if scans is None else scans
    return promote_scan(p.M0[sel], p.values_f32("K")[sel], p.values_f32("V")[sel], p.beta[sel],
                        p.w[sel], p.gamma[sel])


def worst_rel(got, ref):
    """Largest relative Frobenius error over the leading (scan[, firing]) indices."""
    axes = (-2, -1)
    num = np.linalg.norm(got.astype(np.float64) - ref, axis=axes)
    den = np.linalg.norm(ref, axis=axes)
    return float(np.max(num / np.maximum(den, 1e-30)))


CASES = [  # BH, F, n, dk, dv
    (1, 1, 16, 64, 64),
    (3, 5, 32, 64, 128),
    (5, 7, 48, 128, 64),
    (2, 9, 64, 128, 128),
    (4, 3, 128, 128, 256),
    (9, 4, 16, 128, 192),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_promote_parity(case):
    BH, F, n, dk, dv = CASES[case]
    p = gdn_synth.make_promote_problem(600 + case, BH, F, n, dk, dv, dtype="bf16")
    M, S = run(p, f"promote case {case}")
    M_ref, S_ref = oracle_of(p)
    rm, rs = worst_rel(M, M_ref), worst_rel(S, S_ref)
    announce(f"promote case {case}: final {rm:.2e}, states {rs:.2e}")
    assert np.all(np.isfinite(S))
    assert rm <= TOL and rs <= TOL, (rm, rs)


def test_promote_without_states_and_empty_scan():
    p = gdn_synth.make_promote_problem(610, 3, 6, 32, 64, 64, dtype="bf16")
    M, S = run(p, "promote no states", keep_states=False)
    assert S is None
    M_ref, _ = oracle_of(p)
    assert worst_rel(M, M_ref) <= TOL
    z = gdn_synth.make_promote_problem(611, 2, 0, 16, 64, 64, dtype="bf16")
    M0, S0 = run(z, "promote zero firings")
    np.testing.assert_array_equal(M0, z.M0)
    assert S0.shape == (2, 0, 64, 64)


def test_promote_workload_sampled():
    """The benchmarked scan (128 scans, 64 firings of 64 pairs, dk = dv = 128) in one
    launch; 6 scans against the oracle, every firing's state."""
    p = gdn_synth.promote_workload()
    M, S = run(p, "promote workload")
    scans = [0, 7, 8, 63, 100, 127]
    M_ref, S_ref = oracle_of(p, scans)
    rm, rs = worst_rel(M[scans], M_ref), worst_rel(S[scans], S_ref)
    announce(f"promote workload sampled: final {rm:.2e}, states {rs:.2e}")
    assert rm <= TOL and rs <= TOL, (rm, rs)
