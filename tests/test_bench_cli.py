"""bench.py's command-line contract that can be checked without a GPU: more than one GPU
is refused with a message (the library has a one-GPU path only), and the byte accounting
of the three workloads matches the sizes stated for them."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_of_the_workloads():
    sys.path.insert(0, ROOT)
    import bench
    import gdn_synth
    # decode: 512 requests x 32 value heads of 128 x 128 fp32 state, read and written
    dec = gdn_synth.make_decode_problem(1, 512, 16, 32, 128, 128, pool=1)
    state = 2 * 512 * 32 * 128 * 128 * 4
    qk = 2 * 512 * 16 * 128 * 2
    vo = 2 * 512 * 32 * 128 * 2
    assert bench.decode_bytes(dec, 2) == state + qk + vo + 8 * 512 * 32 + 8 * 32 + 8 * 512
    # promote: K and V once, gates, memory in and out, one state per firing
    pr = gdn_synth.make_promote_problem(1, 4, 3, 16, 64, 128)
    expect = (4 * 3 * 16 * (64 + 128) * 2 + 4 * 3 * (2 * 16 + 64) * 4 + 2 * 4 * 64 * 128 * 4
              + 4 * 3 * 64 * 128 * 4)
    assert bench.promote_bytes(pr, 2) == expect
    assert bench.promote_bytes(gdn_synth.promote_workload(), 2) == 830472192
