"""Seeded random configurations through the C ABI against the oracles: the prefill at both
chunk sizes and both input dtypes, the decode step and the backward. Every draw varies the
request count (on both sides of the 64-request chunk-table switch), the lengths (empty
requests, partial chunks, short requests for the token recurrence), the head counts and
grouping ratios (1 to 4, not only powers of two), the head dims, the gates (gentle to strong
decay) and the initial states (entries up to 0.5: initial states much larger than the
outputs are the envelope test of test_gpu_range.py), so shapes the named tests do not list
are covered too.
Bars as elsewhere: bf16 2e-2 rms(o) plus the output's rounding and 1e-3 on the states, fp32
1e-4 and 1e-5; gradients 1e-4 rms."""
import numpy as np
import pytest

import gdn_synth
import oracle
from gpu_util import announce, compare, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_deltanet_prefill_gdn_amd as gdn
    gdn.load_library()
    yield


@pytest.mark.parametrize("case", range(64))
def test_prefill_random(case):
    import gated_deltanet_prefill_gdn_amd as gdn
    seed = 40000 + case
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 5, 13, 40, 66, 90]))
    top = int(rng.choice([20, 150, 600]))
    lengths = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, top, B)]
    H = int(rng.choice([1, 2, 3]))
    HV = H * int(rng.choice([1, 2, 3, 4]))
    dk = int(rng.choice([64, 128, 256]))
    dv = int(rng.choice([64, 128, 256]))
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    chunk = 128 if (dtype == "bf16" and dk >= 128 and rng.random() < 0.4) else 64
    flags = gdn.GDN_FLAG_CHUNK_ALL if rng.random() < 0.3 else 0
    pool = B + int(rng.integers(0, 4))
    p = gdn_synth.make_problem(seed, lengths, H, HV, dk, dv, dtype=dtype, pool=pool,
                               cache_indices=list(rng.permutation(pool)[:B]),
                               a_mean=float(rng.uniform(-4.0, 2.0)),
                               b_mean=float(rng.uniform(-2.0, 2.0)),
                               state_std=float(rng.choice([0.0, 0.1, 0.5])))
    out, pool_gpu, _ = run_gpu(p, f"random-prefill-{case} C={chunk} flags={flags}",
                               chunk_size=chunk, flags=flags)
    compare(p, out, pool_gpu, oracle.prefill(p))


@pytest.mark.parametrize("case", range(24))
def test_decode_random(case):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    seed = 41000 + case
    rng = np.random.default_rng(seed)
    H = int(rng.choice([1, 2, 3]))
    HV = H * int(rng.choice([1, 2, 3]))
    dk = int(rng.choice([64, 128, 256]))
    dv = int(rng.choice([64, 128, 256]))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    B = int(rng.integers(1, 70))
    pool = B + int(rng.integers(0, 5))
    p = gdn_synth.make_decode_problem(seed, B, H, HV, dk, dv, dtype=dtype, pool=pool,
                                      cache_indices=list(rng.permutation(pool)[:B]),
                                      state_std=float(rng.choice([0.0, 0.3])),
                                      a_mean=float(rng.uniform(-4.0, 2.0)),
                                      b_mean=float(rng.uniform(-2.0, 2.0)))
    d = to_device(p)
    announce(f"random-decode-{case} B={B} H={H} HV={HV} dk={dk} dv={dv} {dtype}")
    out = gdn.gdn_decode_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                             d["state_pool"], d["cache_indices"])
    torch.cuda.synchronize()
    compare(p, out.float().cpu().numpy().astype(np.float64), d["state_pool"].cpu().numpy(),
            oracle.decode(p))


@pytest.mark.parametrize("case", range(24))
def test_backward_random(case):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    from oracle import backward as bw
    seed = 42000 + case
    rng = np.random.default_rng(seed)
    H = int(rng.choice([1, 2, 3]))
    HV = H * int(rng.choice([1, 2, 3]))
    dk = int(rng.choice([64, 128, 256]))
    dv = int(rng.choice([64, 128, 256]))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    lengths = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 120, int(rng.integers(1, 4)))]
    p = gdn_synth.make_problem(seed, lengths, H, HV, dk, dv, dtype=dtype,
                               a_mean=float(rng.uniform(-3.0, 1.0)),
                               state_std=float(rng.choice([0.0, 0.3])))
    d = to_device(p)
    dout = rng.standard_normal((p.N, p.HV, p.dv)).astype(np.float32)
    if dtype == "bf16":
        bits = gdn_synth.f32_to_bf16_bits(dout).reshape(dout.shape)
        dval = gdn_synth.bf16_bits_to_f32(bits).reshape(dout.shape)
        dout_dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        dval, dout_dev = dout, torch.from_numpy(dout).to("cuda:0")
    dstate = rng.standard_normal((p.B, p.HV, p.dv, p.dk)).astype(np.float32)
    announce(f"random-backward-{case} lengths={lengths} H={H} HV={HV} dk={dk} dv={dv} {dtype}")
    g = gdn.gdn_prefill_bwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                            d["state_pool"], d["cache_indices"], d["cu_seqlens"], dout_dev,
                            torch.from_numpy(dstate).to("cuda:0"))
    torch.cuda.synchronize()
    ref = bw.prefill_backward(p, dval.astype(np.float64), dstate.astype(np.float64))
    for name in ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dstate0"):
        r = getattr(ref, name)
        if r.size == 0:
            continue
        x = g[name].cpu().numpy().astype(np.float64)
        e = float(np.max(np.abs(x - r))) / max(float(np.sqrt(np.mean(r * r))), 1e-30)
        assert e <= 1e-4, f"{name}: max|dg|/rms = {e:.2e}"
