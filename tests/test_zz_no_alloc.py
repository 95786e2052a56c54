"""The no-allocation prefill entry point (built-in device workspace) through the C ABI:
its outputs and states equal those of gdn_prefill_fwd with a caller workspace, on two calls
in a row (the second smaller, on the other state schedule); a problem whose workspace
exceeds the built-in array is refused before anything runs; and the call captured into a
HIP graph replays to the eager result."""
import numpy as np
import pytest

import gdn_synth
from gpu_util import announce, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import gated_deltanet_prefill_gdn_amd as gdn
    gdn.load_library()
    yield


def _both(p, label):
    """(out, pool) of gdn_prefill_fwd_noalloc and of gdn_prefill_fwd on the same inputs."""
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    res = []
    for noalloc in (True, False):
        d = to_device(p)
        out = torch.full((p.N, p.HV, p.dv), 3.0, dtype=d["v"].dtype, device="cuda:0")
        prob = gdn.problem_of(d["q"], d["k"], d["v"], d["state_pool"], d["cache_indices"])
        announce(f"{label} noalloc={noalloc} N={p.N} B={p.B} HV={p.HV} dk={p.dk} "
                 f"schedule={gdn.gdn_prefill_state_schedule(prob)} "
                 f"workspace={gdn.gdn_prefill_workspace_size(prob)}")
        args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                d["state_pool"], d["cache_indices"], d["cu_seqlens"])
        if noalloc:
            gdn.gdn_prefill_fwd_noalloc(*args, out)
        else:
            gdn.gdn_prefill_fwd(*args, out=out)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), d["state_pool"].cpu().numpy()))
    return res


def test_noalloc_matches_the_workspace_entry_point_twice():
    import gated_deltanet_prefill_gdn_amd as gdn
    big = gdn_synth.make_problem(81, [3000, 500, 0, 77], 2, 4, 128, 128, dtype="bf16", pool=6,
                                 cache_indices=[5, 0, 3, 1], a_mean=-3.0, state_std=0.3)
    small = gdn_synth.make_problem(82, [200, 65], 1, 1, 64, 64, dtype="bf16", pool=2,
                                   state_std=0.3)
    for p, label in ((big, "noalloc-1"), (small, "noalloc-2")):
        prob = gdn.make_problem(p.N, p.B, p.H, p.HV, p.dk, p.dv, p.pool, gdn.GDN_DTYPE_BF16)
        assert gdn.gdn_prefill_workspace_size(prob) <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        (o1, s1), (o2, s2) = _both(p, label)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(s1, s2)
        assert np.all(np.isfinite(o1))
    assert gdn.gdn_prefill_state_schedule(
        gdn.make_problem(big.N, big.B, 2, 4, 128, 128, 6, gdn.GDN_DTYPE_BF16)) == \
        gdn.GDN_SCHEDULE_SEGMENTS


def test_noalloc_refuses_problems_beyond_its_array():
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    p = gdn_synth.make_problem(83, [4096, 4096], 16, 16, 128, 128, dtype="bf16", state_std=0.3)
    prob = gdn.make_problem(p.N, p.B, p.H, p.HV, p.dk, p.dv, p.pool, gdn.GDN_DTYPE_BF16)
    assert gdn.gdn_prefill_workspace_size(prob) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    d = to_device(p)
    out = torch.full((p.N, p.HV, p.dv), 7.0, dtype=torch.bfloat16, device="cuda:0")
    announce("noalloc-refuse")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_prefill_fwd_noalloc(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"],
                                    d["dt_bias"], d["state_pool"], d["cache_indices"],
                                    d["cu_seqlens"], out)
    assert e.value.status == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    np.testing.assert_array_equal(d["state_pool"].cpu().numpy(), p.state_pool)


@pytest.mark.parametrize("lengths", [[300, 65, 7], [3, 70, 5, 9, 40]])
def test_noalloc_replayed_from_a_hip_graph(lengths):
    """The callers this entry point is for include code under graph capture: the call
    captured into a HIP graph (torch.cuda.graph) and replayed four times, with eager pool
    resets and synchronisations between the replays, gives the eager call's outputs and
    states bit for bit every time (the second case takes the short-request split, so the
    token recurrence is captured too)."""
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    p = gdn_synth.make_problem(990 + len(lengths), lengths, 2, 4, 128, 128, dtype="bf16",
                               state_std=0.2)
    d = to_device(p)
    pool0 = d["state_pool"].clone()
    out = torch.empty((p.N, p.HV, p.dv), dtype=d["v"].dtype, device="cuda:0")
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["state_pool"],
            d["cache_indices"], d["cu_seqlens"])
    s = torch.cuda.Stream()
    announce(f"graph lengths={lengths}: eager call")
    with torch.cuda.stream(s):
        gdn.gdn_prefill_fwd_noalloc(*args, out, stream=s)
    torch.cuda.synchronize()
    ref_out, ref_pool = out.clone(), d["state_pool"].clone()
    d["state_pool"].copy_(pool0)
    torch.cuda.synchronize()
    announce(f"graph lengths={lengths}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gdn.gdn_prefill_fwd_noalloc(*args, out, stream=s)
    torch.cuda.synchronize()
    for i in range(4):
        d["state_pool"].copy_(pool0)
        out.zero_()
        torch.cuda.synchronize()
        announce(f"graph lengths={lengths}: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: outputs differ"
        assert torch.equal(d["state_pool"], ref_pool), f"replay {i}: states differ"
