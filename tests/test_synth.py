"""The seeded input generator: deterministic, distinct per tensor, correct rounding."""
import numpy as np

import gdn_synth


def test_deterministic_and_distinct_streams():
    a = gdn_synth.normal(123, gdn_synth.TID_Q, 1000)
    b = gdn_synth.normal(123, gdn_synth.TID_Q, 1000)
    c = gdn_synth.normal(123, gdn_synth.TID_K, 1000)
    np.testing.assert_array_equal(a, b)
    assert not np.allclose(a, c)


def test_moments():
    x = gdn_synth.normal(5, 1, 400000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = gdn_synth.uniform(5, 2, 400000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.005


def test_bf16_is_rounded_fp32_draw():
    p32 = gdn_synth.make_problem(9, [50], 1, 1, 64, 64, dtype="f32")
    pbf = gdn_synth.make_problem(9, [50], 1, 1, 64, 64, dtype="bf16")
    np.testing.assert_array_equal(gdn_synth.f32_to_bf16_bits(p32.q), pbf.q)
    back = gdn_synth.bf16_bits_to_f32(pbf.q)
    assert np.max(np.abs(back - p32.q) / np.maximum(np.abs(p32.q), 1e-30)) <= 2.0 ** -8


def test_threaded_draw_equals_serial_draw():
    big = gdn_synth._draw(3, 1, (300000,), "f32")
    ref = gdn_synth.normal(3, 1, 300000).astype(np.float32)
    np.testing.assert_array_equal(big, ref)


def test_workload_shapes():
    expect = {0: (256, 1, 1, 64, 64, "f32"), 1: (16384, 16, 16, 128, 128, "bf16"),
              3: (16384, 8, 8, 256, 256, "bf16")}
    for i, (N, H, HV, dk, dv, dt) in expect.items():
        p = gdn_synth.workload(i)
        assert (p.N, p.H, p.HV, p.dk, p.dv, p.dtype) == (N, H, HV, dk, dv, dt)
    p2 = gdn_synth.workload(2)
    assert p2.B == 8 and p2.H == 16 and p2.HV == 32 and p2.pool == 64
    assert len(set(p2.cache_indices.tolist())) == 8
    assert all(1 <= L <= 8192 for L in np.diff(p2.cu_seqlens))
