"""GPU backward of the prefill (gdn_prefill_bwd, through the C ABI) against the fp64
backward oracle (oracle/backward.py, itself pinned by finite differences in
test_oracle_backward.py), element by element.

Bar: the kernels run in fp32 on exact inputs (bf16 widens exactly), so every gradient
tensor must satisfy max|g - g_ref| <= 1e-4 rms(g_ref): fp32 rounding through a few hundred
dependent token steps and sums over up to 256 rows stays orders of magnitude below that.
"""
import numpy as np
import pytest

import gdn_synth
from oracle import backward as bw
from gpu_util import announce, to_device

pytestmark = pytest.mark.gpu

BAR = 1e-4
NAMES = ("dq", "dk", "dv", "da", "db", "dA_log", "ddt_bias", "dstate0")


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_deltanet_prefill_gdn_amd as gdn
    gdn.load_library()
    yield


def _upstream(p, seed):
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((p.N, p.HV, p.dv)).astype(np.float32)
    if p.dtype == "bf16":
        dout_dev = gdn_synth.f32_to_bf16_bits(dout).reshape(dout.shape)
        dout_val = gdn_synth.bf16_bits_to_f32(dout_dev).reshape(dout.shape)
    else:
        dout_dev = dout_val = dout
    dstate = rng.standard_normal((p.B, p.HV, p.dv, p.dk)).astype(np.float32)
    return dout_dev, dout_val.astype(np.float64), dstate


def _run(p, seed, label):
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    d = to_device(p)
    dout_dev, dout_val, dstate = _upstream(p, seed)
    t = torch.from_numpy(np.ascontiguousarray(dout_dev))
    dout = (t.view(torch.bfloat16) if p.dtype == "bf16" else t).to("cuda:0")
    ds = torch.from_numpy(dstate).to("cuda:0")
    announce(f"{label} gdn_prefill_bwd N={p.N} B={p.B} H={p.H} HV={p.HV} dk={p.dk} dv={p.dv} "
             f"dtype={p.dtype}")
    g = gdn.gdn_prefill_bwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                            d["state_pool"], d["cache_indices"], d["cu_seqlens"], dout, ds)
    torch.cuda.synchronize()
    got = {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES}
    ref = bw.prefill_backward(p, dout_val, dstate.astype(np.float64))
    return got, ref


def _compare(got, ref, label):
    rep = {}
    for n in NAMES:
        r = getattr(ref, n)
        assert got[n].shape == r.shape, n
        assert np.all(np.isfinite(got[n])), n
        if r.size == 0:
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        err = float(np.max(np.abs(got[n] - r)))
        rep[n] = err / max(rms, 1e-30)
    announce(f"{label} max|dg|/rms: " + ", ".join(f"{k}={v:.1e}" for k, v in rep.items()))
    bad = {k: v for k, v in rep.items() if not v <= BAR}
    assert not bad, rep


CASES = {
    # ragged requests (one empty, one of one token) across checkpoint and sub-chunk edges,
    # grouped value heads, moderate decay, non-zero initial states
    "ragged-bf16": dict(seed=91, lengths=[130, 0, 65, 1, 200], H=2, HV=4, dk=128, dv=128,
                        dtype="bf16", a_mean=-2.0, state_std=0.3),
    "fp32-d64": dict(seed=92, lengths=[300, 17], H=1, HV=2, dk=64, dv=64, dtype="f32",
                     a_mean=-1.0, state_std=0.5),
    "dk256-dv128": dict(seed=93, lengths=[90, 40], H=1, HV=1, dk=256, dv=128, dtype="bf16",
                        a_mean=-3.0, state_std=0.2),
    "dk64-dv256": dict(seed=94, lengths=[70], H=1, HV=2, dk=64, dv=256, dtype="bf16",
                       b_mean=1.0, state_std=0.2),
    # three value heads per q/k head (dq, dk sum over them), strong decay
    "odd-groups-strong-decay": dict(seed=98, lengths=[100, 33, 257], H=3, HV=9, dk=128,
                                    dv=128, dtype="bf16", a_mean=2.0, state_std=0.3),
    "dk256-dv256": dict(seed=99, lengths=[50, 20], H=1, HV=2, dk=256, dv=256, dtype="f32",
                        a_mean=-2.0, state_std=0.2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_the_oracle(case):
    c = dict(CASES[case])
    seed, lengths = c.pop("seed"), c.pop("lengths")
    H, HV, dk, dv = c.pop("H"), c.pop("HV"), c.pop("dk"), c.pop("dv")
    pool = len(lengths) + 2
    p = gdn_synth.make_problem(seed, lengths, H, HV, dk, dv, pool=pool,
                               cache_indices=list(range(pool - 1, 1, -1))[:len(lengths)], **c)
    got, ref = _run(p, seed + 1, f"bwd-{case}")
    _compare(got, ref, f"bwd-{case}")


def test_backward_without_tokens():
    """N = 0: each initial state's gradient is the final state's; no gate gradient."""
    p = gdn_synth.make_problem(95, [0, 0], 1, 1, 64, 64, dtype="bf16", state_std=0.5)
    got, ref = _run(p, 96, "bwd-empty")
    np.testing.assert_array_equal(got["dstate0"], ref.dstate0)
    assert np.all(got["dA_log"] == 0) and np.all(got["ddt_bias"] == 0)


def test_backward_is_deterministic():
    p = gdn_synth.make_problem(97, [150, 70], 2, 4, 128, 128, dtype="bf16", state_std=0.3)
    g1, _ = _run(p, 98, "bwd-det-1")
    g2, _ = _run(p, 98, "bwd-det-2")
    for n in NAMES:
        np.testing.assert_array_equal(g1[n], g2[n])


def test_backward_workload1_sampled_head():
    """The dense-batch workload (4 x 4096 tokens, 16 heads) at full size on the GPU, the
    gradients of value head 0 (and of its q/k head: H = HV) against the oracle's backward of
    that head alone over every token; the heads are independent when H = HV."""
    import copy
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    p = gdn_synth.workload(1)
    d = to_device(p)
    dout_dev, dout_val, dstate = _upstream(p, 96)
    t = torch.from_numpy(np.ascontiguousarray(dout_dev))
    dout = t.view(torch.bfloat16).to("cuda:0")
    announce(f"workload1 gdn_prefill_bwd N={p.N} B={p.B} H={p.H} HV={p.HV}")
    g = gdn.gdn_prefill_bwd(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                            d["state_pool"], d["cache_indices"], d["cu_seqlens"], dout,
                            torch.from_numpy(dstate).to("cuda:0"))
    torch.cuda.synchronize()
    sub = copy.copy(p)
    sub.q, sub.k, sub.v = p.q[:, [0]], p.k[:, [0]], p.v[:, [0]]
    sub.a, sub.b = p.a[:, [0]], p.b[:, [0]]
    sub.A_log, sub.dt_bias = p.A_log[[0]], p.dt_bias[[0]]
    sub.state_pool = p.state_pool[:, [0]]
    sub.H, sub.HV = 1, 1
    ref = bw.prefill_backward(sub, dout_val[:, [0]], dstate[:, [0]].astype(np.float64))
    got = {"dq": g["dq"][:, [0]], "dk": g["dk"][:, [0]], "dv": g["dv"][:, [0]],
           "da": g["da"][:, [0]], "db": g["db"][:, [0]], "dA_log": g["dA_log"][[0]],
           "ddt_bias": g["ddt_bias"][[0]], "dstate0": g["dstate0"][:, [0]]}
    got = {n: x.cpu().numpy().astype(np.float64) for n, x in got.items()}
    _compare(got, ref, "workload1 head 0")
