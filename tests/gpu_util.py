"""Helpers for GPU parity tests: move a gdn_synth.Problem to the device, call the
library through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np

import gdn_synth

TOL = {"f32": (1e-4, 1e-5), "bf16": (2e-2, 1e-3)}   # (output: x rms(o), state: rel Frobenius)
# The output has v's dtype (pymllm gdn_chunkwise page, Returns), so a bf16 output carries
# its own rounding of at most half an ulp, 2^-8 |o|, on top of the computation's error.
OUT_ROUNDING = {"f32": 0.0, "bf16": 2.0 ** -8}


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(p: gdn_synth.Problem, dev="cuda:0"):
    import torch

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    if p.dtype == "bf16":
        q = t(p.q.view(np.int16), torch.bfloat16)
        k = t(p.k.view(np.int16), torch.bfloat16)
        v = t(p.v.view(np.int16), torch.bfloat16)
    else:
        q, k, v = t(p.q), t(p.k), t(p.v)
    return dict(q=q, k=k, v=v, a=t(p.a), b=t(p.b), A_log=t(p.A_log), dt_bias=t(p.dt_bias),
                state_pool=t(p.state_pool.copy()), cache_indices=t(p.cache_indices),
                cu_seqlens=t(p.cu_seqlens))


def run_gpu(p: gdn_synth.Problem, label: str = "", dev_tensors=None, **kw):
    """One gdn_prefill_fwd call; returns (out fp64 numpy, state_pool fp32 numpy, tensors)."""
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn

    d = dev_tensors if dev_tensors is not None else to_device(p)
    announce(f"{label} gdn_prefill_fwd N={p.N} B={p.B} H={p.H} HV={p.HV} dk={p.dk} dv={p.dv} "
             f"dtype={p.dtype} seed={p.seed}")
    t0 = time.time()
    out = gdn.gdn_prefill_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                              d["state_pool"], d["cache_indices"], d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    announce(f"{label} done in {time.time() - t0:.3f}s")
    return out.float().cpu().numpy().astype(np.float64), d["state_pool"].cpu().numpy(), d


def compare(p: gdn_synth.Problem, out_gpu, pool_gpu, ref, tol=None, heads=None, rows=None):
    """Check the GPU result against an oracle result at the bars for p.dtype.

    Outputs: |do| <= tol_o * rms(o_oracle) + r |o_oracle| element by element, with r the
    half-ulp of the output dtype (2^-8 for bf16, 0 for fp32).
    State: for every touched slot (and compared head), ||dS||_F / ||S||_F <= tol_s.
    Slots no request touches must equal their input bit for bit.
    The report (printed) holds max|do| / rms(o), the worst element's share of its allowance,
    the compute-only margin max(|do| - r |o|) / rms(o) (the error beyond the output's own
    rounding, against tol_o) and the worst state error."""
    tol_o, tol_s = tol or TOL[p.dtype]
    heads = list(range(p.HV)) if heads is None else list(heads)
    r0, r1 = (0, p.dv) if rows is None else rows
    o_gpu = out_gpu[:, heads, r0:r1]
    o_ref = ref.out
    report = {}
    o_ok = True
    if o_ref.size:
        assert np.all(np.isfinite(o_gpu)), "non-finite outputs"
        rms = float(np.sqrt(np.mean(o_ref ** 2)))
        d = np.abs(o_gpu - o_ref)
        allow = tol_o * rms + OUT_ROUNDING[p.dtype] * np.abs(o_ref)
        report["o_maxerr_over_rms"] = float(d.max()) / max(rms, 1e-30)
        report["o_worst_err_over_allowance"] = float((d / allow).max())
        report["o_compute_over_rms"] = (float((d - OUT_ROUNDING[p.dtype] * np.abs(o_ref)).max())
                                        / max(rms, 1e-30))
        o_ok = bool(np.all(d <= allow))
    lengths = np.diff(p.cu_seqlens)
    worst = 0.0
    for bi, slot in enumerate(p.cache_indices):
        if lengths[bi] == 0:
            np.testing.assert_array_equal(pool_gpu[slot], p.state_pool[slot])
            continue
        g = pool_gpu[slot][heads, r0:r1].astype(np.float64)
        r = ref.state_pool[slot][heads, r0:r1]
        denom = np.linalg.norm(r)
        rel_err = float(np.linalg.norm(g - r) / denom) if denom > 0 else float(np.linalg.norm(g))
        worst = max(worst, rel_err)
    report["state_rel"] = worst
    announce("margins " + ", ".join(f"{k}={v:.3g}" for k, v in report.items()))
    assert o_ok, f"output error above the bar: {report}"
    assert worst <= tol_s, f"state rel err {worst:.3e} > {tol_s}: {report}"
    touched = set(int(s) for s, L in zip(p.cache_indices, lengths) if L > 0)
    for slot in range(p.pool):
        if slot not in touched:
            np.testing.assert_array_equal(pool_gpu[slot], p.state_pool[slot])
    return report
