"""The C = 128 schedule (bf16 inputs, dk of 128 or 256) against the fp64 oracle through the
C ABI, at the bf16 bars: max|do| <= 2e-2 rms(o) plus the output's own rounding, state rel.
Frobenius <= 1e-3. The chunk size is a schedule parameter (pymllm gdn_chunkwise page,
Module Contents: the Torch function defaults to 128, the kernel entry point to 64), so
the oracle is the same token recurrence."""
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


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_workloads_at_c128(idx):
    p = gdn_synth.workload(idx)
    out, pool, _ = run_gpu(p, f"c128-workload{idx}", chunk_size=128)
    rep = compare(p, out, pool, oracle.prefill(p))
    announce(f"c128 workload{idx} {rep}")


def test_workload4_sampled_heads_at_c128():
    p = gdn_synth.workload(4)
    out, pool, _ = run_gpu(p, "c128-workload4", chunk_size=128)
    heads = [0, 1, 31]
    rep = compare(p, out, pool, oracle.prefill(p, heads=heads), heads=heads)
    announce(f"c128 workload4 sampled {rep}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (128, 256), (256, 64), (256, 128),
                                   (256, 256)])
def test_ragged_lengths_at_c128(dk, dv):
    """Every request chunked (GDN_FLAG_CHUNK_ALL): lengths on both sides of 64 and 128
    (one-row chunks, a chunk ending one row into the second half, whole chunks), an empty
    request, grouped value heads, a shuffled pool with a spare slot."""
    import gated_deltanet_prefill_gdn_amd as gdn
    lengths = [1, 63, 64, 65, 0, 127, 128, 129, 255, 256, 300, 2]
    p = gdn_synth.make_problem(1280 + dk + dv, lengths, 2, 4, dk, dv, dtype="bf16", pool=13,
                               cache_indices=[12, 3, 0, 7, 5, 2, 9, 1, 4, 11, 6, 8],
                               state_std=0.3)
    out, pool, _ = run_gpu(p, f"c128-ragged-{dk}x{dv}", chunk_size=128,
                           flags=gdn.GDN_FLAG_CHUNK_ALL)
    compare(p, out, pool, oracle.prefill(p))


@pytest.mark.parametrize("case", ["strong-decay", "beta-one", "gqa8-many"])
def test_gates_and_shapes_at_c128(case):
    """Strong decay (e^G underflows inside a 128-row chunk: every decay factor is an
    exponent difference, and the masked ones are selected away, not multiplied); beta near
    1; more than 64 requests with eight value heads per q/k head and enough pairs for
    the wide column blocks."""
    rng = np.random.default_rng(1290)
    if case == "strong-decay":
        p = gdn_synth.make_problem(1291, [1000, 300, 129], 2, 2, 128, 128, dtype="bf16",
                                   a_mean=3.0, state_std=0.5)
    elif case == "beta-one":
        p = gdn_synth.make_problem(1292, [700, 128, 57], 2, 4, 256, 128, dtype="bf16",
                                   a_mean=-4.0, b_mean=4.0, state_std=0.1)
    else:
        B = 80
        lengths = [int(x) for x in rng.integers(0, 400, B)]
        p = gdn_synth.make_problem(1293, lengths, 2, 16, 128, 128, dtype="bf16", pool=B + 4,
                                   cache_indices=list(rng.permutation(B + 4)[:B]),
                                   state_std=0.2)
    out, pool, _ = run_gpu(p, f"c128-{case}", chunk_size=128)
    compare(p, out, pool, oracle.prefill(p))


def test_split_invariance_at_c128():
    """One call over 777 tokens equals a call over the first 300 and a second over the rest
    through the same pool slot, all at C = 128 (the second call's chunks start at token
    300 of the request, so the chunk boundaries differ from the whole call's)."""
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    p = gdn_synth.make_problem(1294, [777], 2, 2, 128, 128, dtype="bf16", state_std=0.2)
    ref = oracle.prefill(p)
    out_full, pool_full, _ = run_gpu(p, "c128-whole", chunk_size=128)
    compare(p, out_full, pool_full, ref)
    d = to_device(p)
    sl = lambda x, a, b: x[a:b].contiguous()
    outs = []
    for (a, b) in ((0, 300), (300, 777)):
        announce(f"c128 split-part {a}:{b}")
        cu = torch.tensor([0, b - a], dtype=torch.int64, device="cuda:0")
        outs.append(gdn.gdn_prefill_fwd(sl(d["q"], a, b), sl(d["k"], a, b), sl(d["v"], a, b),
                                        sl(d["a"], a, b), sl(d["b"], a, b), d["A_log"],
                                        d["dt_bias"], d["state_pool"], d["cache_indices"], cu,
                                        chunk_size=128))
    torch.cuda.synchronize()
    out_split = torch.cat(outs).float().cpu().numpy()
    compare(p, out_split.astype(np.float64), d["state_pool"].cpu().numpy(), ref)


def test_c128_determinism_and_c64_agreement():
    """Ten C = 128 calls give bitwise equal results; C = 64 and C = 128 agree with each
    other within twice the bf16 bars (each is within the bar of the oracle)."""
    import torch
    p = gdn_synth.make_problem(1295, [1000, 513], 2, 4, 128, 128, dtype="bf16", state_std=0.2)
    d = to_device(p)
    pool0 = d["state_pool"].clone()
    outs = []
    for i in range(10):
        d["state_pool"].copy_(pool0)
        out, pool, _ = run_gpu(p, f"c128-rep{i}", dev_tensors=d, chunk_size=128)
        outs.append((out, pool))
    for out, pool in outs[1:]:
        np.testing.assert_array_equal(out, outs[0][0])
        np.testing.assert_array_equal(pool, outs[0][1])
    d["state_pool"].copy_(pool0)
    out64, pool64, _ = run_gpu(p, "c64-same", dev_tensors=d, chunk_size=64)
    # a different schedule rounds differently: equal bits would mean C = 64 ran twice
    announce(f"c64 vs c128: max|do| {np.abs(out64 - outs[0][0]).max():.3e}, differing "
             f"outputs {np.mean(out64 != outs[0][0]):.3f}, state max|dS| "
             f"{np.abs(pool64 - outs[0][1]).max():.3e}")
    assert not np.array_equal(out64, outs[0][0])
    rms = float(np.sqrt(np.mean(out64 ** 2)))
    assert np.all(np.abs(out64 - outs[0][0]) <= 4e-2 * rms + 2.0 ** -7 * np.abs(out64))
    rel = np.linalg.norm(pool64 - outs[0][1]) / np.linalg.norm(pool64)
    assert rel <= 2e-3, rel
    torch.cuda.synchronize()


def test_short_requests_split_at_c128():
    """A batch of short requests on average (N <= 64 B) at C = 128: the requests of at
    most GDN_SHORT_REQUEST tokens take the token recurrence, the others the C = 128 chunked
    kernels, in one call; against the oracle, and against the same call with every
    request chunked."""
    import gated_deltanet_prefill_gdn_amd as gdn
    lengths = [3, 70, 5, 130, 1, 9, 40, 10, 11, 0]
    assert sum(lengths) <= 64 * len(lengths)
    p = gdn_synth.make_problem(1296, lengths, 2, 4, 128, 128, dtype="bf16", pool=11,
                               cache_indices=[10, 0, 9, 1, 8, 2, 7, 3, 6, 4], state_std=0.2)
    ref = oracle.prefill(p)
    out, pool, _ = run_gpu(p, "c128-split", chunk_size=128)
    compare(p, out, pool, ref)
    out_all, pool_all, _ = run_gpu(p, "c128-chunk-all", chunk_size=128,
                                   flags=gdn.GDN_FLAG_CHUNK_ALL)
    compare(p, out_all, pool_all, ref)


@pytest.mark.parametrize("case", range(6))
def test_random_shapes_at_c128(case):
    """Seeded random configurations at C = 128: request counts on both sides of 64, lengths
    with empty and partial chunks on both sides of 64 and 128, grouped-head ratios up to 4,
    dk of 128 or 256 with every dv, a shuffled pool with spare slots, gates from gentle to
    strong decay, with and without the short-request split."""
    import gated_deltanet_prefill_gdn_amd as gdn
    rng = np.random.default_rng(1300 + case)
    B = int(rng.choice([1, 3, 17, 70]))
    lengths = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 400, B)]
    H = int(rng.choice([1, 2, 4]))
    HV = H * int(rng.choice([1, 2, 4]))
    dk = int(rng.choice([128, 256]))
    dv = int(rng.choice([64, 128, 256]))
    pool = B + int(rng.integers(0, 5))
    p = gdn_synth.make_problem(1300 + case, lengths, H, HV, dk, dv, dtype="bf16", pool=pool,
                               cache_indices=list(rng.permutation(pool)[:B]),
                               a_mean=float(rng.uniform(-3.0, 1.0)),
                               b_mean=float(rng.uniform(-1.0, 1.0)),
                               state_std=float(rng.choice([0.0, 0.1, 0.5])))
    flags = gdn.GDN_FLAG_CHUNK_ALL if case % 2 else 0
    out, pool_gpu, _ = run_gpu(p, f"c128-random-{case}", chunk_size=128, flags=flags)
    compare(p, out, pool_gpu, oracle.prefill(p))


def test_other_entry_points_at_c128():
    """At C = 128 the no-allocation entry point (built-in workspace) and the per-stage
    events entry point give the workspace entry point's result bit for bit."""
    import torch
    import gated_deltanet_prefill_gdn_amd as gdn
    p = gdn_synth.make_problem(1297, [700, 129, 64], 2, 4, 128, 128, dtype="bf16",
                               state_std=0.2)
    d = to_device(p)
    pool0 = d["state_pool"].clone()
    args = lambda: (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                    d["state_pool"], d["cache_indices"], d["cu_seqlens"])
    announce("c128 gdn_prefill_fwd (workspace)")
    ref = gdn.gdn_prefill_fwd(*args(), chunk_size=128)
    torch.cuda.synchronize()
    pool_ref = d["state_pool"].clone()
    d["state_pool"].copy_(pool0)
    announce("c128 gdn_prefill_fwd_noalloc")
    out = torch.empty_like(ref)
    gdn.gdn_prefill_fwd_noalloc(*args(), out, chunk_size=128)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(d["state_pool"], pool_ref)
    d["state_pool"].copy_(pool0)
    announce("c128 gdn_prefill_fwd_events")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(gdn.GDN_NUM_STAGES + 1)]
    for e in evs:
        e.record()  # creates the underlying event
    out2 = gdn.gdn_prefill_fwd_events(*args(), [e.cuda_event for e in evs], chunk_size=128)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref) and torch.equal(d["state_pool"], pool_ref)
    compare(p, ref.float().cpu().numpy().astype(np.float64), pool_ref.cpu().numpy(),
            oracle.prefill(p))
