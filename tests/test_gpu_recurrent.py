"""GPU parity of the chunk-free recurrent path (gdn_recurrent_fwd through the C ABI)
against the CPU oracle's prefill: short variable-length requests (the speculative-
verification shape, 0 to 16 tokens) plus longer ones, fp32 and bf16, grouped heads, every
head dim; the bars are the prefill's (fp32 inputs: max |do| <= 1e-4 rms(o), state 1e-5
relative; bf16: 2e-2 rms(o) plus the output's own half-ulp, state 1e-3), untouched and
empty-request slots bit for bit. Also agreement with the chunked path on the same call."""
import time

import numpy as np
import pytest

import gdn_synth
import oracle
from gpu_util import announce, compare, run_gpu, to_device

pytestmark = pytest.mark.gpu


def run_recurrent(p, label, d=None):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    d = d if d is not None else to_device(p)
    announce(f"{label} gdn_recurrent_fwd N={p.N} B={p.B} H={p.H} HV={p.HV} dk={p.dk} "
             f"dv={p.dv} dtype={p.dtype} seed={p.seed}")
    t0 = time.time()
    out = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                                d["dt_bias"], d["state_pool"], d["cache_indices"],
                                d["cu_seqlens"])
    torch.cuda.synchronize()
    announce(f"{label} done in {time.time() - t0:.3f}s")
    return out.float().cpu().numpy().astype(np.float64), d["state_pool"].cpu().numpy(), d


# (lengths, H, HV, dk, dv, dtype, pool, state_std, a_mean)
CASES = [
    ([1], 1, 1, 64, 64, "f32", 1, 0.0, 0.0),
    ([4, 0, 7, 1, 16, 3], 2, 4, 128, 128, "bf16", 9, 0.1, 0.0),
    ([5, 2, 0, 9], 1, 2, 256, 64, "bf16", 6, 0.5, -4.0),
    ([8, 8, 8], 2, 2, 64, 256, "f32", 4, 1.0, 0.0),
    ([2, 13, 6, 0, 1], 4, 8, 128, 256, "bf16", 7, 0.1, 2.0),
    ([3, 11], 1, 1, 256, 256, "f32", 3, 0.3, 0.0),
    ([70, 1, 129, 4], 2, 4, 128, 128, "f32", 5, 0.2, 0.0),
    ([200, 3, 64], 2, 6, 128, 64, "bf16", 4, 0.1, -1.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_recurrent_parity(case):
    lengths, H, HV, dk, dv, dtype, pool, sstd, am = CASES[case]
    seed = 900 + case
    idx = gdn_synth.seeded_permutation(seed, gdn_synth.TID_PERM, pool)[:len(lengths)]
    p = gdn_synth.make_problem(seed, lengths, H, HV, dk, dv, dtype=dtype, pool=pool,
                               cache_indices=idx, state_std=sstd, a_mean=am)
    out, pool_gpu, _ = run_recurrent(p, f"recurrent case {case}")
    rep = compare(p, out, pool_gpu, oracle.prefill(p))
    announce(f"recurrent case {case}: {rep}")


def test_recurrent_agrees_with_chunked_path():
    """The same bf16 call through gdn_recurrent_fwd and gdn_prefill_fwd. Each output is
    within 2e-2 rms(o) plus its own half-ulp of the oracle, so the two differ by at most
    the sum of both bars: 4e-2 rms(o) plus one bf16 ulp of the value; the pools within
    twice the state bar."""
    lengths = [3, 64, 1, 100, 0, 17]
    p = gdn_synth.make_problem(950, lengths, 2, 4, 128, 128, dtype="bf16", pool=8,
                               cache_indices=[6, 1, 0, 3, 7, 2], state_std=0.2)
    out_r, pool_r, _ = run_recurrent(p, "recurrent vs chunked")
    out_c, pool_c, _ = run_gpu(p, "chunked vs recurrent")
    rms = np.sqrt(np.mean(out_c ** 2))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(out_c), 1e-30))) - 7)  # 8-bit significand
    assert np.all(np.abs(out_r - out_c) <= 4e-2 * rms + ulp)
    scale = np.max(np.abs(pool_c)) + 1e-30
    assert np.max(np.abs(pool_r.astype(np.float64) - pool_c)) <= 2e-3 * scale


def test_recurrent_empty_tokens_leave_pool():
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    dev = torch.device("cuda:0")
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt, device=dev)
    pool = torch.randn(3, 2, 64, 64, device=dev)
    before = pool.clone()
    cu = torch.zeros(4, dtype=torch.int64, device=dev)
    out = gdn.gdn_recurrent_fwd(z(0, 1, 64, dt=torch.bfloat16), z(0, 1, 64, dt=torch.bfloat16),
                                z(0, 2, 64, dt=torch.bfloat16), z(0, 2), z(0, 2), z(2), z(2),
                                pool, torch.tensor([2, 0, 1], device=dev), cu)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 64)
    assert torch.equal(pool, before)


def test_recurrent_verify_workload_sampled():
    """The benchmarked verification batch (512 requests x 4 tokens, H = 16, HV = 32,
    dk = dv = 128, bf16, 1 GiB of state) in one launch, as bench.py times it; 12 seeded
    requests, every head and token, against the oracle."""
    p = gdn_synth.verify_workload()
    out, pool_gpu, _ = run_recurrent(p, "verify workload")
    reqs = np.sort(gdn_synth.seeded_permutation(78, gdn_synth.TID_PERM, p.B)[:12])
    cu = p.cu_seqlens
    rows = np.concatenate([np.arange(cu[r], cu[r + 1]) for r in reqs])
    lengths = [int(cu[r + 1] - cu[r]) for r in reqs]
    sub = gdn_synth.make_problem(p.seed, lengths, p.H, p.HV, p.dk, p.dv, dtype=p.dtype,
                                 pool=len(reqs))
    sub.q, sub.k, sub.v, sub.a, sub.b = p.q[rows], p.k[rows], p.v[rows], p.a[rows], p.b[rows]
    sub.A_log, sub.dt_bias = p.A_log, p.dt_bias
    sub.state_pool = p.state_pool[p.cache_indices[reqs]]
    sub.cache_indices = np.arange(len(reqs), dtype=np.int64)
    rep = compare(sub, out[rows], pool_gpu[p.cache_indices[reqs]], oracle.prefill(sub))
    announce(f"verify workload sampled: {rep}")
    assert np.all(np.isfinite(out))
