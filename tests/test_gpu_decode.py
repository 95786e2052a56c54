"""GPU parity of the decode step (gdn_decode_fwd through the C ABI) against the CPU
oracle: the same seeded inputs, element by element at the bars of the prefill (fp32 inputs:
max |do| <= 1e-4 rms(o), state 1e-5 relative; bf16: 2e-2 rms(o) plus the output's own
half-ulp, state 1e-3), untouched slots bit for bit. Also the decode step continuing a
prefill on the GPU, and several steps in a row."""
import time

import numpy as np
import pytest

import gdn_synth
import oracle
from gpu_util import announce, compare, to_device, run_gpu

pytestmark = pytest.mark.gpu


def run_decode(p, label, d=None):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    d = d if d is not None else to_device(p)
    announce(f"{label} gdn_decode_fwd B={p.B} H={p.H} HV={p.HV} dk={p.dk} dv={p.dv} "
             f"pool={p.pool} dtype={p.dtype} seed={p.seed}")
    t0 = time.time()
    out = gdn.gdn_decode_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                             d["state_pool"], d["cache_indices"])
    torch.cuda.synchronize()
    announce(f"{label} done in {time.time() - t0:.3f}s")
    return out.float().cpu().numpy().astype(np.float64), d["state_pool"].cpu().numpy(), d


# (B, H, HV, dk, dv, dtype, pool, state_std, a_mean, b_mean)
CASES = [
    (1, 1, 1, 64, 64, "f32", 1, 0.0, 0.0, 0.0),
    (5, 2, 4, 128, 128, "bf16", 9, 0.1, 0.0, 0.0),
    (3, 1, 2, 256, 64, "bf16", 3, 0.5, -4.0, 2.0),
    (4, 2, 2, 64, 256, "f32", 6, 1.0, 0.0, 0.0),
    (7, 4, 8, 128, 256, "bf16", 7, 0.1, 2.0, -2.0),
    (2, 1, 1, 256, 256, "f32", 5, 0.3, 0.0, 0.0),
    (33, 2, 6, 128, 64, "f32", 40, 0.2, -1.0, 0.0),
    (64, 16, 32, 128, 128, "bf16", 64, 0.1, 0.0, 0.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_parity(case):
    B, H, HV, dk, dv, dtype, pool, sstd, am, bm = CASES[case]
    seed = 700 + case
    idx = gdn_synth.seeded_permutation(seed, gdn_synth.TID_PERM, pool)[:B]
    p = gdn_synth.make_decode_problem(seed, B, H, HV, dk, dv, dtype=dtype, pool=pool,
                                      cache_indices=idx, state_std=sstd, a_mean=am, b_mean=bm)
    out, pool_gpu, _ = run_decode(p, f"decode case {case}")
    ref = oracle.decode(p)
    rep = compare(p, out, pool_gpu, ref)
    announce(f"decode case {case}: {rep}")


def subproblem(p, reqs):
    """The requests `reqs` of a decode problem on their own (their slots renumbered 0..)."""
    reqs = np.asarray(reqs)
    sub = gdn_synth.make_decode_problem(p.seed, 0, p.H, p.HV, p.dk, p.dv, dtype=p.dtype, pool=1)
    sub.q, sub.k, sub.v = p.q[reqs], p.k[reqs], p.v[reqs]
    sub.a, sub.b = p.a[reqs], p.b[reqs]
    sub.A_log, sub.dt_bias = p.A_log, p.dt_bias
    sub.state_pool = p.state_pool[p.cache_indices[reqs]]
    sub.cache_indices = np.arange(len(reqs), dtype=np.int64)
    sub.cu_seqlens = np.arange(len(reqs) + 1, dtype=np.int64)
    return sub


def test_decode_full_workload_sampled():
    """The benchmarked decode workload (512 requests, H = 16, HV = 32, dk = dv = 128, bf16,
    1 GiB of state) in one launch; 12 requests, all heads, against the oracle."""
    p = gdn_synth.decode_workload()
    out, pool_gpu, _ = run_decode(p, "decode workload")
    reqs = gdn_synth.seeded_permutation(77, gdn_synth.TID_PERM, p.B)[:12]
    sub = subproblem(p, reqs)
    ref = oracle.decode(sub)
    sub_pool_gpu = pool_gpu[p.cache_indices[reqs]]
    rep = compare(sub, out[reqs], sub_pool_gpu, ref)
    announce(f"decode workload sampled: {rep}")
    assert np.all(np.isfinite(out))


def test_decode_continues_prefill():
    """Prefill of each request's first L tokens, then one decode step with token L + 1,
    both on the GPU, equals the oracle's prefill of L + 1 tokens: the decode output is the
    last token's output and the pool holds the same final states."""
    lengths = [100, 64, 1, 257]
    B, H, HV, dk, dv = len(lengths), 2, 4, 128, 128
    full = gdn_synth.make_problem(800, [L + 1 for L in lengths], H, HV, dk, dv, dtype="bf16",
                                  pool=6, cache_indices=[4, 0, 5, 2], state_std=0.1)
    cu = full.cu_seqlens
    last = cu[1:] - 1                                  # row of each request's last token
    keep = np.concatenate([np.arange(cu[i], cu[i + 1] - 1) for i in range(B)])
    pre = gdn_synth.make_problem(800, lengths, H, HV, dk, dv, dtype="bf16", pool=6,
                                 cache_indices=[4, 0, 5, 2], state_std=0.1)
    for name in ("q", "k", "v", "a", "b"):
        setattr(pre, name, getattr(full, name)[keep])
    _, _, d = run_gpu(pre, "prefill before decode")
    dec = gdn_synth.make_decode_problem(800, B, H, HV, dk, dv, dtype="bf16", pool=6,
                                       cache_indices=[4, 0, 5, 2])
    for name in ("q", "k", "v", "a", "b"):
        setattr(dec, name, getattr(full, name)[last])
    dd = to_device(dec)
    dd["state_pool"] = d["state_pool"]                # the pool the prefill left
    out, pool_gpu, _ = run_decode(dec, "decode after prefill", dd)
    ref = oracle.prefill(full)
    ref_last = oracle.OracleResult(out=ref.out[last], state_pool=ref.state_pool,
                                   heads=ref.heads, rows=ref.rows)
    rep = compare(full_as_decode(full, dec), out, pool_gpu, ref_last)
    announce(f"prefill + decode: {rep}")


def full_as_decode(full, dec):
    """The decode problem, carrying the initial pool of the full problem (compare() checks
    untouched slots against it)."""
    dec.state_pool = full.state_pool
    return dec


def test_decode_steps_in_a_row():
    """Four decode calls in a row on the GPU (state kept in the device pool) equal the
    oracle's four-token prefill of each request."""
    B, H, HV, dk, dv, T = 6, 2, 4, 64, 128, 4
    full = gdn_synth.make_problem(801, [T] * B, H, HV, dk, dv, dtype="f32", pool=8,
                                  cache_indices=[7, 1, 3, 0, 6, 2], state_std=0.5)
    ref = oracle.prefill(full)
    d = None
    outs = []
    for t in range(T):
        rows = full.cu_seqlens[:-1] + t
        dec = gdn_synth.make_decode_problem(801, B, H, HV, dk, dv, dtype="f32", pool=8,
                                           cache_indices=[7, 1, 3, 0, 6, 2])
        for name in ("q", "k", "v", "a", "b"):
            setattr(dec, name, getattr(full, name)[rows])
        dd = to_device(dec)
        if d is None:
            dd["state_pool"] = to_device(full)["state_pool"]
        else:
            dd["state_pool"] = d["state_pool"]
        o, pool_gpu, d = run_decode(dec, f"decode step {t}", dd)
        outs.append(o)
    out = np.stack(outs, axis=1).reshape(B * T, HV, dv)   # request-major, like full's rows
    rep = compare(full, out, pool_gpu, ref)
    announce(f"four decode steps: {rep}")


def test_decode_empty_batch():
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    dev = torch.device("cuda:0")
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device=dev)
    pool = torch.randn(2, 2, 64, 64, device=dev)
    before = pool.clone()
    out = gdn.gdn_decode_fwd(z(0, 1, 64, dt=torch.bfloat16), z(0, 1, 64, dt=torch.bfloat16),
                             z(0, 2, 64, dt=torch.bfloat16), z(0, 2), z(0, 2), z(2), z(2), pool,
                             z(0, dt=torch.int64))
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 64)
    assert torch.equal(pool, before)
