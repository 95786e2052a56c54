"""Benchmark of the GDN chunkwise prefill forward on one MI355X.

A step is one gdn_prefill_fwd call (every stage of the path) over the dense-batch
bf16 workload: 4 requests x 4096 tokens, H = HV = 16, dk = dv = 128, C = 64, with
inputs resident in HBM. Prints one JSON line. Workloads 2-4 are timed as sub-results, and
every bf16 workload with dk >= 128 also at chunk size 128 on the same inputs
(``chunk_128``), the measured comparison of the two schedules.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

With ``--op decode`` a step is instead one gdn_decode_fwd call over the decode workload
(512 requests x 1 token, H = 16, HV = 32, dk = dv = 128, bf16, 1 GiB of state), and with
``--op promote`` one gdn_promote_scan call over the Promote workload (128 scans x 64
firings x 64 pairs, dk = dv = 128, bf16, every firing's state kept); with ``--op verify``
one gdn_recurrent_fwd call over a speculative-verification batch (512 requests x 4 tokens,
the decode workload's heads and pool), the chunked gdn_prefill_fwd on the same call timed
beside it; with ``--op backward`` one gdn_prefill_bwd call on the dense-batch workload. The
JSON line then reports that call. ``--op pipelined`` times successive prefill calls back to
back and pipelined over two streams (bench_pipelined).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
WORKLOAD_INDEX = 1
METRIC = "GDN prefill tokens/sec + effective TFLOPs (% MFMA/HBM roof), dk=dv=128 C=64"


def algorithmic_flops_per_token_vhead(dk: int, dv: int, C: int) -> float:
    """Three state contractions (6 dk dv), the triangular in-chunk products
    (C (3 dk + 2 dv)) and the inverse (C^2 / 3)."""
    return 6.0 * dk * dv + C * (3.0 * dk + 2.0 * dv) + C * C / 3.0


def path_bytes(p, s_qkv: int) -> float:
    """q, k, v read once, o written once, a and b (fp32), touched states read and written."""
    touched = int(sum(1 for L in (p.cu_seqlens[1:] - p.cu_seqlens[:-1]) if L > 0))
    return (p.N * (2 * p.H * p.dk * s_qkv + 2 * p.HV * p.dv * s_qkv + 8 * p.HV)
            + touched * p.HV * p.dv * p.dk * 8)


def stage_bytes(p, s_qkv: int, s_ws: int, n_chunks: int):
    """Algorithmic bytes each stage must move: its inputs read once, its outputs written
    once. Rows are chunk rows (n_chunks * C, padding included) for per-chunk data. The
    decayed keys K~ (fp16) exist once per (chunk, value head), since they carry that head's
    gates; the normalised q copy (fp16) once per (chunk, q/k head)."""
    C = p.chunk_size
    rows = n_chunks * C
    n_pairs = n_chunks * p.HV
    qk_frag = rows * p.HV * p.dk * 2 + rows * p.H * p.dk * 2   # K~ + normalised q
    touched = int(sum(1 for L in (p.cu_seqlens[1:] - p.cu_seqlens[:-1]) if L > 0))
    # A_qk is causal: of its (C / 32) x (C / 16) fragments (32-token step x 16-row tile)
    # those above the diagonal are zero and neither written nor read (2 of 8 at C = 64,
    # 12 of 32 at C = 128)
    nrt = C // 16
    aqk = n_pairs * C * C * s_ws * sum(w // 2 + 1 for w in range(nrt)) // (nrt * (C // 32))
    # stage 0 is the chunk table only: the bf16 chunk prep forms its own gates
    gate = (p.B + 1) * 8 + n_chunks * 4
    # prep: reads q, k, v and the raw gate inputs a, b (fp32); writes W<-, U~, the row
    # scale e^G, A_qk, K~ and the q copy
    prep = (2 * p.N * p.H * p.dk * s_qkv + p.N * p.HV * p.dv * s_qkv + p.N * p.HV * 8
            + rows * p.HV * (p.dk + p.dv) * s_ws + rows * p.HV * 4
            + aqk + qk_frag)
    # state: reads K~, the q copy, W<-, U~, e^G (its last row is e^{G_n}) and A_qk; writes
    # o; reads and writes the fp32 state of every touched slot
    state = (qk_frag + rows * p.HV * (p.dk + p.dv) * s_ws + rows * p.HV * 4
             + aqk + p.N * p.HV * p.dv * s_qkv
             + touched * p.HV * p.dv * p.dk * 8)
    return {"gate": gate, "chunk_prep": prep, "state": state}


DECODE_SOURCES = ("gdn_decode.hip", "gdn_internal.h")
PROMOTE_SOURCES = ("gdn_promote.hip", "gdn_internal.h", "gdn_mfma.h")
BACKWARD_SOURCES = ("gdn_backward.hip", "gdn_backward.h", "gdn_internal.h", "gdn_plan_gate.hip")
PREFILL_F32_SOURCES = ("gdn_ref.hip", "gdn_plan_gate.hip", "gdn_api.hip", "gdn_internal.h",
                       "gdn_mfma.h")


def kernel_source_hash(kind: str = "prefill") -> str:
    """sha256[:16] over the kernel sources a measurement depends on: for "prefill" (the
    bf16 path) every .hip / .h file of csrc except the decode, Promote, backward and fp32
    kernels' own files, for "prefill_f32" PREFILL_F32_SOURCES, for "decode" DECODE_SOURCES,
    for "promote" PROMOTE_SOURCES, for "backward" BACKWARD_SOURCES."""
    csrc = os.path.join(ROOT, "gated_deltanet_prefill_gdn_amd", "csrc")
    if kind == "decode":
        files = sorted(DECODE_SOURCES)
    elif kind == "promote":
        files = sorted(PROMOTE_SOURCES)
    elif kind == "backward":
        files = sorted(BACKWARD_SOURCES)
    elif kind == "prefill_f32":
        files = sorted(PREFILL_F32_SOURCES)
    else:
        files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))
                       and f not in ("gdn_decode.hip", "gdn_promote.hip", "gdn_backward.hip",
                                     "gdn_backward.h", "gdn_ref.hip"))
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, src_hash: str, launches_per_step: int = 1):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = d.get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


class Hip:
    """hipEvent helpers from the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        # Timing-only events: without the system-scope fence (cache write-back and
        # invalidate) that a default event record inserts between the kernels it separates.
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))

    def empty_pair_ms(self, stream, reps: int = 20) -> float:
        """Mean time between two events recorded back to back on `stream` with no work
        between them: the share of every event-timed stage that is event overhead."""
        import torch
        rec = self.lib.hipEventRecord
        rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        pairs = [(self.event(), self.event()) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in pairs:
            rec(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
            rec(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        ms = sum(self.elapsed_ms(e0, e1) for e0, e1 in pairs) / reps
        for e0, e1 in pairs:
            self.destroy(e0)
            self.destroy(e1)
        return ms


def cpu_baseline(p, reps: int = 3):
    """The oracle (fp64 token recurrence) as it stands, on this host's cores, over the
    whole workload (every request and value head), run `reps` times; the median wall
    time gives tokens/s. On 16 cores this is about 15 s of CPU time in total."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.prefill(p, nthreads=threads)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    return {"value": p.N / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({p.B} requests x {p.N // p.B} tokens, {p.HV} value heads), "
                      f"fp64 recurrence, median of {reps} runs, {dt:.2f} s wall each"}


DECODE_METRIC = "GDN decode step tokens/sec (one token per request), dk=dv=128"


def decode_bytes(p, s_qkv: int) -> int:
    """Algorithmic HBM bytes of one decode step: the fp32 state of every (request, value
    head) read and written once; q, k per q/k head, v and out per value head; a, b; the
    per-head gate parameters and the slot indices."""
    return (2 * p.B * p.HV * p.dv * p.dk * 4 + 2 * p.B * p.H * p.dk * s_qkv
            + 2 * p.B * p.HV * p.dv * s_qkv + 8 * p.B * p.HV + 8 * p.HV + 8 * p.B)


def decode_cpu_baseline(p, n_req: int = 64, reps: int = 3):
    """The oracle (fp64 recurrence, one step) as it stands, on this host's cores, over the
    first n_req requests of the decode workload with every value head; the median wall
    time gives tokens/s."""
    import numpy as np
    import oracle
    import gdn_synth
    reqs = np.arange(n_req)
    sub = gdn_synth.make_decode_problem(p.seed, 0, p.H, p.HV, p.dk, p.dv, dtype=p.dtype, pool=1)
    sub.q, sub.k, sub.v, sub.a, sub.b = p.q[reqs], p.k[reqs], p.v[reqs], p.a[reqs], p.b[reqs]
    sub.A_log, sub.dt_bias = p.A_log, p.dt_bias
    sub.state_pool = p.state_pool[p.cache_indices[reqs]]
    sub.cache_indices = np.arange(n_req, dtype=np.int64)
    sub.cu_seqlens = np.arange(n_req + 1, dtype=np.int64)
    threads = oracle.default_threads()
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.decode(sub, nthreads=threads)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    return {"value": n_req / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_req} of the {p.B} requests, all {p.HV} value heads, fp64 recurrence "
                      f"step, median of {reps} runs, {dt:.3f} s wall each"}


def bench_decode(args):
    import numpy as np
    import torch

    import gdn_synth
    import gated_deltanet_prefill_gdn_amd as gdn

    p = gdn_synth.decode_workload()
    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    q = t(p.q.view(np.int16), torch.bfloat16)
    k = t(p.k.view(np.int16), torch.bfloat16)
    v = t(p.v.view(np.int16), torch.bfloat16)
    a, b, A_log, dt_bias = t(p.a), t(p.b), t(p.A_log), t(p.dt_bias)
    pool = t(p.state_pool)
    idx = t(p.cache_indices)
    out = torch.empty((p.B, p.HV, p.dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_decode_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the same steps with HIP events on the launch stream around each launch
    hip = Hip()
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        rec(ctypes.c_void_p(e0), ctypes.c_void_p(stream.cuda_stream))
        step()
        rec(ctypes.c_void_p(e1), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    events_ms = float(np.mean([hip.elapsed_ms(e0, e1) for e0, e1 in evs]))
    for e0, e1 in evs:
        hip.destroy(e0)
        hip.destroy(e1)
    pair_ms = hip.empty_pair_ms(stream.cuda_stream)
    launch_ms = events_ms - pair_ms if events_ms > 2 * pair_ms else events_ms
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    nbytes = decode_bytes(p, 2)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash("decode")
    res = {
        "metric": DECODE_METRIC,
        "value": p.B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, seed 1100)",
        "config": {"workload": gdn_synth.DECODE_WORKLOAD, "global_batch": p.B, "seq_len": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic("decode_kernel", src_hash),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": launch_ms,
                     "avg_launch_ms_events": events_ms, "event_pair_ms": pair_ms},
        "kernel_source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = decode_cpu_baseline(p)
    print(json.dumps(res), flush=True)


VERIFY_METRIC = "GDN short-request (verification) tokens/sec, 4 tokens per request, dk=dv=128"


def verify_bytes(p, s_qkv: int) -> int:
    """Algorithmic HBM bytes of one recurrent call: the fp32 state of every (request, value
    head) read and written once; per token q, k per q/k head, v and out per value head, a
    and b; the gate parameters, the slot indices and the sequence offsets."""
    return (2 * p.B * p.HV * p.dv * p.dk * 4 + 2 * p.N * p.H * p.dk * s_qkv
            + 2 * p.N * p.HV * p.dv * s_qkv + 8 * p.N * p.HV + 8 * p.HV + 16 * p.B + 8)


def _time_launches(step, stream, steps: int, warmup: int):
    """Wall ms per step over `steps` back-to-back calls after `warmup`, then the average
    HIP-event time of one call on the launch stream less the empty event pair's."""
    import numpy as np
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    hip = Hip()
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    for e0, e1 in evs:
        rec(ctypes.c_void_p(e0), ctypes.c_void_p(stream.cuda_stream))
        step()
        rec(ctypes.c_void_p(e1), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    events_ms = float(np.mean([hip.elapsed_ms(e0, e1) for e0, e1 in evs]))
    for e0, e1 in evs:
        hip.destroy(e0)
        hip.destroy(e1)
    pair_ms = hip.empty_pair_ms(stream.cuda_stream)
    launch_ms = events_ms - pair_ms if events_ms > 2 * pair_ms else events_ms
    return ms_per_step, events_ms, pair_ms, launch_ms


def verify_cpu_baseline(p, n_req: int = 64, reps: int = 3):
    """The oracle's prefill as it stands, on this host's cores, over the first n_req
    requests of the verification workload with every value head; tokens/s."""
    import numpy as np
    import oracle
    import gdn_synth
    T = int(p.cu_seqlens[1] - p.cu_seqlens[0])
    sub = gdn_synth.make_problem(p.seed, [T] * n_req, p.H, p.HV, p.dk, p.dv, dtype=p.dtype,
                                 pool=n_req)
    rows = np.arange(n_req * T)
    sub.q, sub.k, sub.v, sub.a, sub.b = p.q[rows], p.k[rows], p.v[rows], p.a[rows], p.b[rows]
    sub.A_log, sub.dt_bias = p.A_log, p.dt_bias
    sub.state_pool = p.state_pool[p.cache_indices[:n_req]]
    sub.cache_indices = np.arange(n_req, dtype=np.int64)
    threads = oracle.default_threads()
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.prefill(sub, nthreads=threads)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    return {"value": n_req * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_req} of the {p.B} requests ({n_req * T} tokens), all {p.HV} value "
                      f"heads, fp64 token recurrence, median of {reps} runs, {dt:.3f} s wall each"}


def bench_verify(args):
    import numpy as np
    import torch

    import gdn_synth
    import gated_deltanet_prefill_gdn_amd as gdn

    p = gdn_synth.verify_workload()
    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    q = t(p.q.view(np.int16), torch.bfloat16)
    k = t(p.k.view(np.int16), torch.bfloat16)
    v = t(p.v.view(np.int16), torch.bfloat16)
    a, b, A_log, dt_bias = t(p.a), t(p.b), t(p.A_log), t(p.dt_bias)
    pool = t(p.state_pool)
    idx, cu = t(p.cache_indices), t(p.cu_seqlens)
    out = torch.empty((p.N, p.HV, p.dv), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(gdn.problem_of(q, k, v, pool, idx)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_recurrent_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx, cu, out=out,
                              stream=stream)

    def chunked():
        gdn.gdn_prefill_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx, cu, out=out,
                            workspace=ws, stream=stream)

    ms_per_step, events_ms, pair_ms, launch_ms = _time_launches(step, stream, args.steps,
                                                                args.warmup)
    chunked_ms = _time_launches(chunked, stream, args.steps, args.warmup)[0]
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    nbytes = verify_bytes(p, 2)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash("decode")
    res = {
        "metric": VERIFY_METRIC,
        "value": p.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, seed 1300)",
        "config": {"workload": gdn_synth.VERIFY_WORKLOAD, "global_batch": p.B,
                   "seq_len": int(p.cu_seqlens[1]), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "recurrent_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic("recurrent_kernel", src_hash),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": launch_ms,
                     "avg_launch_ms_events": events_ms, "event_pair_ms": pair_ms},
        # gdn_prefill_fwd on the same requests: it evaluates requests this short with the
        # same token recurrence (see --op crossover for the chunked path's cost)
        "prefill_fwd_ms_per_step": chunked_ms,
        "kernel_source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = verify_cpu_baseline(p)
    print(json.dumps(res), flush=True)


PROMOTE_METRIC = "Promote update scan pairs/sec (decay, erase, write per firing), dk=dv=128"


def promote_bytes(p, s_kv: int) -> int:
    """Algorithmic HBM bytes of one scan call: keys and values once, the gates and the
    log-decay, the memory in and out, and every firing's state written (fp32)."""
    BH, F, n, dk, dv = p.shape
    return (BH * F * n * (dk + dv) * s_kv + BH * F * (2 * n + dk) * 4
            + 2 * BH * dk * dv * 4 + BH * F * dk * dv * 4)


def promote_cpu_baseline(p, n_scans: int = 16, reps: int = 3):
    """The Promote oracle (fp64 numpy) as it stands on the first n_scans scans; the median
    wall time gives pairs/s."""
    import numpy as np
    from oracle.promote import promote_scan
    BH, F, n, dk, dv = p.shape
    sel = slice(0, n_scans)
    args = (p.M0[sel], p.values_f32("K")[sel], p.values_f32("V")[sel], p.beta[sel], p.w[sel],
            p.gamma[sel])
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        promote_scan(*args)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    return {"value": n_scans * F * n / dt, "unit": "pairs/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{n_scans} of the {BH} scans, all {F} firings, fp64 numpy (BLAS matrix "
                      f"products), median of {reps} runs, {dt:.3f} s wall each"}


def _blas_threads() -> int:
    """Threads numpy's BLAS may use here (OMP_NUM_THREADS if set, else the usable cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def bench_promote(args):
    import numpy as np
    import torch

    import gdn_synth
    import gated_deltanet_prefill_gdn_amd as gdn

    p = gdn_synth.promote_workload()
    BH, F, n, dk, dv = p.shape
    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    K = t(p.K.view(np.int16), torch.bfloat16)
    V = t(p.V.view(np.int16), torch.bfloat16)
    beta, w, gamma = t(p.beta), t(p.w), t(p.gamma)
    M = t(p.M0.copy())
    states = torch.empty((BH, F, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_promote_scan(K, V, beta, w, gamma, M, states=states, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    hip = Hip()
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    evs = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        rec(ctypes.c_void_p(e0), ctypes.c_void_p(stream.cuda_stream))
        step()
        rec(ctypes.c_void_p(e1), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    events_ms = float(np.mean([hip.elapsed_ms(e0, e1) for e0, e1 in evs]))
    for e0, e1 in evs:
        hip.destroy(e0)
        hip.destroy(e1)
    pair_ms = hip.empty_pair_ms(stream.cuda_stream)
    launch_ms = events_ms - pair_ms if events_ms > 2 * pair_ms else events_ms
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    nbytes = promote_bytes(p, 2)
    flops = 4.0 * BH * F * n * dk * dv
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash("promote")
    res = {
        "metric": PROMOTE_METRIC,
        "value": BH * F * n / (ms_per_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller, seed 1200)",
        "config": {"workload": gdn_synth.PROMOTE_WORKLOAD, "global_batch": BH, "seq_len": F,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "promote_scan_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic("promote_scan_kernel", src_hash),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": launch_ms,
                     "avg_launch_ms_events": events_ms, "event_pair_ms": pair_ms},
        "effective": {"tflops": flops / (launch_ms * 1e-3) / 1e12,
                      "frac_mfma_bf16": flops / (launch_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                      "algorithmic_flops": flops},
        "kernel_source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = promote_cpu_baseline(p)
    print(json.dumps(res), flush=True)



SUB_WORKLOADS = (2, 3, 4)   # reported beside the headline workload in the same line
FLUSH_BYTES = 512 << 20     # more than the 256 MiB Infinity Cache


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def stored_counters(kernel: str, workload: str, src_hash: str):
    """Per-launch counter figures (HBM bytes, MFMA busy, executed MFMA flops) of `kernel`
    on `workload` from the committed rocprofv3 summaries, if they were taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = d.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent


def workload_tag(p) -> str:
    """Short name of a workload: dtype, requests, tokens, heads and head dims."""
    if p.B == 1 or len(set(int(x) for x in (p.cu_seqlens[1:] - p.cu_seqlens[:-1]))) == 1:
        t = f"b{p.B}_t{p.N // max(p.B, 1)}"
    else:
        t = f"b{p.B}_n{p.N}"
    hv = f"_hv{p.HV}" if p.HV != p.H else ""
    c = f"_c{p.chunk_size}" if p.chunk_size != 64 else ""
    return f"{p.name}_{t}_h{p.H}{hv}_d{p.dk}{c}"


def prefill_cpu_baseline(p, heads=None, reps: int = 3):
    """The oracle (fp64 token recurrence) as it stands, threaded over this host's cores, on
    every request of the workload and the value heads in `heads` (all if None); the median
    wall time of `reps` runs, scaled to the whole workload by HV / len(heads), gives
    tokens/s."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    hs = list(range(p.HV)) if heads is None else list(heads)
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.prefill(p, heads=hs, nthreads=threads)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls))
    per_tok = dt * p.HV / len(hs)   # seconds for every head
    which = ("every value head" if len(hs) == p.HV
             else f"value heads {hs} of {p.HV} (time scaled by {p.HV}/{len(hs)})")
    return {"value": p.N / per_tok, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"all {p.B} requests ({p.N} tokens), {which}, fp64 recurrence, "
                      f"median of {reps} runs, {dt:.2f} s wall each"}


def measure_prefill(p, steps: int, warmup: int, cold_steps: int, copy_calibration=False):
    """Times gdn_prefill_fwd on the workload `p` (inputs resident in HBM, workspace
    preallocated). Returns a dict of the wall time per call over `steps` back-to-back
    calls, per-call HIP-event times (warm and after a cache flush: median, p10, p90), the
    per-stage launch times and the roofline of the dominant kernel."""
    import numpy as np
    import torch

    import gated_deltanet_prefill_gdn_amd as gdn

    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    if p.dtype == "bf16":
        q = t(p.q.view(np.int16), torch.bfloat16)
        k = t(p.k.view(np.int16), torch.bfloat16)
        v = t(p.v.view(np.int16), torch.bfloat16)
        s_qkv = 2
    else:
        q, k, v = t(p.q), t(p.k), t(p.v)
        s_qkv = 4
    a, b, A_log, dt_bias = t(p.a), t(p.b), t(p.A_log), t(p.dt_bias)
    pool = t(p.state_pool.copy())
    idx, cu = t(p.cache_indices), t(p.cu_seqlens)
    out = torch.empty((p.N, p.HV, p.dv), dtype=v.dtype, device=dev)
    prob = gdn.problem_of(q, k, v, pool, idx)
    C = p.chunk_size
    ws = torch.empty(gdn.gdn_prefill_workspace_size(prob, C), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    hip = Hip()
    rec = hip.lib.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(events=None):
        if events is None:
            gdn.gdn_prefill_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx, cu, chunk_size=C,
                                out=out, workspace=ws, stream=stream)
        else:
            gdn.gdn_prefill_fwd_events(q, k, v, a, b, A_log, dt_bias, pool, idx, cu, events,
                                       chunk_size=C, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The K timed steps: plain calls, nothing recorded between them.
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps

    # Per-call event times: one event pair around each call (none inside it).
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for e0, e1 in evs:
        rec(ctypes.c_void_p(e0), sp)
        step()
        rec(ctypes.c_void_p(e1), sp)
    torch.cuda.synchronize()
    warm = [hip.elapsed_ms(e0, e1) for e0, e1 in evs]
    for e0, e1 in evs:
        hip.destroy(e0)
        hip.destroy(e1)

    # The same calls with HIP events on the launch stream around every stage: per-kernel
    # launch durations for the roofline.
    nst = gdn.GDN_NUM_STAGES
    sev = [[hip.event() for _ in range(nst + 1)] for _ in range(steps)]
    for i in range(steps):
        step(sev[i])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([hip.elapsed_ms(e[j], e[j + 1]) for e in sev]))
                for j, name in enumerate(gdn.STAGE_NAMES)}
    for e in sev:
        for x in e:
            hip.destroy(x)
    pair_ms = hip.empty_pair_ms(stream.cuda_stream)

    # Calls timed one by one after a 512 MiB write has evicted the Infinity Cache.
    cold = []
    if cold_steps > 0:
        scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        e0, e1 = hip.event(), hip.event()
        for _ in range(cold_steps):
            scratch.fill_(1)
            torch.cuda.synchronize()
            rec(ctypes.c_void_p(e0), sp)
            step()
            rec(ctypes.c_void_p(e1), sp)
            torch.cuda.synchronize()
            cold.append(hip.elapsed_ms(e0, e1))
        hip.destroy(e0)
        hip.destroy(e1)
        del scratch

    # The same inputs at chunk size 128, where the call takes it (bf16, dk >= 128): the
    # measured comparison of the two schedules, timed like the sub-results.
    c128 = None
    if C == 64 and p.dtype == "bf16" and p.dk >= 128:
        ws128 = torch.empty(gdn.gdn_prefill_workspace_size(prob, 128), dtype=torch.uint8,
                            device=dev)
        step128 = lambda: gdn.gdn_prefill_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx, cu,
                                              chunk_size=128, out=out, workspace=ws128,
                                              stream=stream)
        ms128, ev128, _, _ = _time_launches(step128, stream, max(3, steps // 2),
                                            max(3, warmup // 2))
        c128 = {"chunk_size": 128, "ms_per_step": ms128, "tokens_per_s": p.N / (ms128 * 1e-3),
                "call_ms_events": ev128, "vs_chunk_64": ms_per_step / ms128}
        del ws128

    if copy_calibration:
        src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del q, k, v, a, b, pool, out, ws
    torch.cuda.empty_cache()

    n_chunks = int(sum((int(L) + p.chunk_size - 1) // p.chunk_size
                       for L in (p.cu_seqlens[1:] - p.cu_seqlens[:-1])))
    # launch durations: each event-timed stage less the overhead of an empty event pair
    launch = {n: (ms - pair_ms if ms > 2 * pair_ms else ms) for n, ms in stage_ms.items()}
    dom = max(launch, key=launch.get)
    sched = gdn.gdn_prefill_state_schedule(gdn.make_problem(
        p.N, p.B, p.H, p.HV, p.dk, p.dv, p.pool,
        gdn.GDN_DTYPE_BF16 if p.dtype == "bf16" else gdn.GDN_DTYPE_F32), C)
    kernels = dict(gdn.STAGE_KERNELS[sched])
    if C == 128:
        kernels["chunk_prep"] = "mfma_prep128_kernel"
    kernel_name = kernels[dom]
    pbytes = path_bytes(p, s_qkv)
    flops = algorithmic_flops_per_token_vhead(p.dk, p.dv, p.chunk_size) * p.N * p.HV
    src_hash = kernel_source_hash("prefill" if p.dtype == "bf16" else "prefill_f32")
    io = stage_bytes(p, s_qkv, 2, n_chunks) if p.dtype == "bf16" else {}
    tag = workload_tag(p)
    ctr = stored_counters(kernel_name, tag, src_hash)
    sec = launch[dom] * 1e-3
    achieved = pbytes / sec / 1e9
    roof = {"bound": "hbm", "kernel": kernel_name, "stage": dom,
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": ctr.get("hbm_bytes_per_launch") if ctr else None,
            "algorithmic_bytes_per_launch": pbytes,
            "algorithmic_bytes_basis": "the whole path's minimum HBM traffic: q, k, v read "
                                       "once, out written once, a and b (fp32), every "
                                       "touched fp32 state read and written once",
            "avg_launch_ms": launch[dom], "avg_launch_ms_events": stage_ms[dom],
            "event_pair_ms": pair_ms}
    if dom in io:
        roof["kernel_io_bytes_per_launch"] = io[dom]
        roof["kernel_io_frac"] = io[dom] / sec / 1e9 / HBM_PEAK_GBS
    if ctr:
        roof["counters"] = {kk: ctr[kk] for kk in ("mfma_busy_frac", "mfma_tflops_executed",
                                                   "read_bytes", "write_bytes") if kk in ctr}
    stages = {}
    for n in launch:
        kn = kernels[n]
        c = stored_counters(kn, tag, src_hash)
        ent = {"kernel": kn, "launch_ms": launch[n], "events_ms": stage_ms[n]}
        if n in io:
            ent["kernel_io_bytes"] = io[n]
            ent["kernel_io_gbs"] = io[n] / max(launch[n], 1e-9) / 1e-3 / 1e9
        if c:
            ent["hbm_bytes_counted"] = c.get("hbm_bytes_per_launch")
            ent["mfma_busy_frac"] = c.get("mfma_busy_frac")
            ent["mfma_tflops_executed"] = c.get("mfma_tflops_executed")
        stages[n] = ent
    call = {"warm": {"p10": _pct(warm, 10), "median": _pct(warm, 50), "p90": _pct(warm, 90),
                     "n": len(warm)}}
    if cold:
        call["flushed"] = {"p10": _pct(cold, 10), "median": _pct(cold, 50),
                           "p90": _pct(cold, 90), "n": len(cold)}
    return {
        "tag": tag, "N": p.N, "B": p.B, "n_chunks": n_chunks,
        "ms_per_step": ms_per_step,
        "tokens_per_s": p.N / (ms_per_step * 1e-3),
        "call_ms_events": call,
        "roofline": roof,
        "effective": {"tflops": flops / (ms_per_step * 1e-3) / 1e12,
                      "frac_mfma_bf16": flops / (ms_per_step * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                      "path_gbs": pbytes / (ms_per_step * 1e-3) / 1e9,
                      "frac_hbm": pbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "algorithmic_flops": flops, "algorithmic_bytes": pbytes},
        "stages": stages,
        "state_schedule": sched,
        "chunk_size": C,
        "chunk_128": c128,
        "kernel_source_hash": src_hash,
    }


def bench_prefill(args):
    import gdn_synth

    import dataclasses

    def load(i):
        w = gdn_synth.workload(i, args.dtype)
        return w if args.chunk == 64 else dataclasses.replace(w, chunk_size=args.chunk)

    main_idx = args.workload if args.workload is not None else WORKLOAD_INDEX
    p = load(main_idx)
    m = measure_prefill(p, args.steps, args.warmup, args.cold_steps, args.copy_calibration)
    res = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": f"synthetic (seeded SplitMix64/Box-Muller, seed {p.seed})",
        "config": {"workload": gdn_synth.WORKLOADS[main_idx]
                   + (f" [q, k, v, out drawn in {p.dtype}]" if args.dtype else "")
                   + (f" [chunk size {args.chunk}]" if args.chunk != 64 else ""),
                   "global_batch": p.B,
                   "seq_len": int(p.N // max(p.B, 1)), "parallelism": "none (1 GPU)"},
        "roofline": m["roofline"],
        "effective": m["effective"],
        "call_ms_events": m["call_ms_events"],
        "stages": m["stages"],
        "chunk_128": m["chunk_128"],
        "kernel_source_hash": m["kernel_source_hash"],
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(p)
    subs = []
    if args.workload is None and not args.no_sub:
        del p
        for wi in SUB_WORKLOADS:
            sp_ = load(wi)
            sm = measure_prefill(sp_, max(3, args.steps // 2), max(3, args.warmup // 2),
                                 args.cold_steps)
            ent = {"workload": gdn_synth.WORKLOADS[wi]
                   + (f" [q, k, v, out drawn in {sp_.dtype}]" if args.dtype else "")
                   + (f" [chunk size {args.chunk}]" if args.chunk != 64 else ""),
                   "index": wi,
                   "tokens_per_s": sm["tokens_per_s"], "ms_per_step": sm["ms_per_step"],
                   "call_ms_events": sm["call_ms_events"],
                   "path_frac_hbm": sm["effective"]["frac_hbm"],
                   "effective_tflops": sm["effective"]["tflops"],
                   "dominant_kernel": sm["roofline"]["kernel"],
                   "dominant_kernel_frac": sm["roofline"]["frac"],
                   "roofline": sm["roofline"], "stages": sm["stages"],
                   "chunk_128": sm["chunk_128"]}
            if not args.no_cpu_baseline:
                # the long request's 32 heads: two sampled heads bound the oracle's time
                heads = [0, sp_.HV - 1] if sp_.N * sp_.HV > (1 << 21) else None
                ent["cpu_baseline"] = prefill_cpu_baseline(sp_, heads=heads, reps=1)
            subs.append(ent)
            del sp_
        res["workloads"] = subs
    print(json.dumps(res), flush=True)


BACKWARD_METRIC = "GDN prefill backward tokens/sec (every input's gradient), dk=dv=128 C=64"


def backward_bytes(p, s_qkv: int) -> int:
    """Algorithmic HBM bytes of one backward call: q, k, v, dout read and dq, dk, dv written
    (fp32); a, b read and da, db written; the initial and final-state gradients and the
    initial states read, the initial-state gradients written (fp32)."""
    return (p.N * (2 * p.H * p.dk * s_qkv + 2 * p.HV * p.dv * s_qkv + 8 * p.HV)
            + p.N * (2 * p.H * p.dk + p.HV * p.dv + 2 * p.HV) * 4
            + 3 * p.B * p.HV * p.dv * p.dk * 4)


def backward_flops(p) -> float:
    """Algorithmic flops of one backward call: per token and value head the forward step
    (S k and the rank-one update: 4 dv dk) and the reverse step of the recurrence (D += do
    q^T, S^T do, D k, S_{t-1} k, <D, S_{t-1}>, the three products of dk, and the update of D:
    19 dv dk), 23 dv dk in all; the per-token gates and norms are left out."""
    return 23.0 * p.N * p.HV * p.dv * p.dk


FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X published vector fp32 (with packed math)


def backward_cpu_baseline(p, heads, reps: int = 1):
    """The backward oracle (fp64 numpy reverse mode) as it stands, on a sample of value
    heads; tokens/s scaled to every head."""
    import numpy as np
    from oracle import backward as bw
    sub = dataclasses_replace_heads(p, heads)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal((sub.N, sub.HV, sub.dv))
    dstate = rng.standard_normal((sub.B, sub.HV, sub.dv, sub.dk))
    walls = []
    for _ in range(reps):
        t0 = time.perf_counter()
        bw.prefill_backward(sub, dout, dstate)
        walls.append(time.perf_counter() - t0)
    dt = float(np.median(walls)) * p.HV / len(heads)
    return {"value": p.N / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"value heads {list(heads)} of {p.HV} over all {p.N} tokens (time scaled "
                      f"by {p.HV}/{len(heads)}), fp64 numpy reverse mode, one thread"}


def dataclasses_replace_heads(p, heads):
    """The workload restricted to the given value heads (with their q/k heads kept whole)."""
    import copy
    import numpy as np
    q = copy.copy(p)
    hv = np.asarray(heads)
    grp = p.HV // p.H
    hs = sorted(set(int(h) // grp for h in hv))
    assert len(hs) == 1 and len(hv) <= grp, "sample the value heads of one q/k head"
    q.q, q.k = p.q[:, hs], p.k[:, hs]
    q.v, q.a, q.b = p.v[:, hv], p.a[:, hv], p.b[:, hv]
    q.A_log, q.dt_bias = p.A_log[hv], p.dt_bias[hv]
    q.state_pool = p.state_pool[:, hv]
    q.H, q.HV = 1, len(hv)
    return q


def bench_backward(args):
    import numpy as np
    import torch

    import gdn_synth
    import gated_deltanet_prefill_gdn_amd as gdn

    p = gdn_synth.workload(WORKLOAD_INDEX)
    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    q = t(p.q.view(np.int16), torch.bfloat16)
    k = t(p.k.view(np.int16), torch.bfloat16)
    v = t(p.v.view(np.int16), torch.bfloat16)
    a, b, A_log, dt_bias = t(p.a), t(p.b), t(p.A_log), t(p.dt_bias)
    pool = t(p.state_pool)
    idx, cu = t(p.cache_indices), t(p.cu_seqlens)
    g = torch.Generator(device="cpu").manual_seed(5)
    dout = torch.randn((p.N, p.HV, p.dv), generator=g).to(torch.bfloat16).to(dev)
    dstate = torch.randn((p.B, p.HV, p.dv, p.dk), generator=g).to(dev)
    prob = gdn.problem_of(q, k, v, pool, idx)
    ws = torch.empty(gdn.gdn_prefill_bwd_workspace_size(prob), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        gdn.gdn_prefill_bwd(q, k, v, a, b, A_log, dt_bias, pool, idx, cu, dout, dstate,
                            workspace=ws, stream=stream)

    ms_per_step, events_ms, pair_ms, launch_ms = _time_launches(step, stream, args.steps,
                                                                args.warmup)
    if args.copy_calibration:
        src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    nbytes = backward_bytes(p, 2)
    flops = backward_flops(p)
    src_hash = kernel_source_hash("backward")
    ctr = stored_counters("bwd_rows_kernel", "backward_" + workload_tag(p), src_hash)
    res = {
        "metric": BACKWARD_METRIC,
        "value": p.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, fp32 arithmetic and gradients",
        "data": f"synthetic (seeded SplitMix64/Box-Muller, seed {p.seed}; upstream gradients "
                "torch.randn seed 5)",
        "config": {"workload": gdn_synth.WORKLOADS[WORKLOAD_INDEX], "global_batch": p.B,
                   "seq_len": int(p.N // p.B), "parallelism": "none (1 GPU)"},
        # The call is bound by the fp32 vector arithmetic of its token recurrence (the row
        # kernel is about 95% of it); its time is the whole call's, on the launch stream.
        "roofline": {"bound": "alu", "kernel": "gdn_prefill_bwd (bwd_rows_kernel and the "
                                               "small token, finish and gate kernels)",
                     "achieved": flops / (launch_ms * 1e-3) / 1e12,
                     "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (launch_ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                     "traffic": ctr.get("hbm_bytes_per_launch") if ctr else None,
                     "traffic_kernel": "bwd_rows_kernel",
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes,
                     "hbm_frac": nbytes / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "avg_launch_ms": launch_ms, "avg_launch_ms_events": events_ms,
                     "event_pair_ms": pair_ms},
        "kernel_source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = backward_cpu_baseline(p, heads=[0])
    print(json.dumps(res), flush=True)


CROSSOVER_LENGTHS = (1, 2, 4, 8, 9, 10, 11, 12, 16, 20, 24, 32, 48, 64)


def bench_crossover(args):
    """Short requests: gdn_prefill_fwd as shipped (requests of at most GDN_SHORT_REQUEST
    tokens through the token recurrence), the same call with GDN_FLAG_CHUNK_ALL (every
    request chunked) and gdn_recurrent_fwd, on 512 requests of equal length L, bf16,
    H = 16, HV = 32, dk = dv = 128 (seeded torch.randn inputs). Prints one JSON line with
    the per-call wall time of each at every L: the measurement behind the threshold."""
    import torch

    import gated_deltanet_prefill_gdn_amd as gdn

    dev = torch.device("cuda:0")
    B, H, HV, D = 512, 16, 32, 128
    g = torch.Generator(device="cpu").manual_seed(7)
    rows = []
    for L in CROSSOVER_LENGTHS:
        N = B * L
        q = torch.randn((N, H, D), generator=g).to(torch.bfloat16).to(dev)
        k = torch.randn((N, H, D), generator=g).to(torch.bfloat16).to(dev)
        v = torch.randn((N, HV, D), generator=g).to(torch.bfloat16).to(dev)
        a = (torch.randn((N, HV), generator=g) - 2.0).to(dev)
        b = torch.randn((N, HV), generator=g).to(dev)
        A_log = torch.rand((HV,), generator=g).to(dev)
        dt_bias = (0.1 * torch.randn((HV,), generator=g)).to(dev)
        pool = (0.05 * torch.randn((B, HV, D, D), generator=g)).to(dev)
        idx = torch.arange(B, dtype=torch.int64, device=dev)
        cu = torch.arange(0, N + 1, L, dtype=torch.int64, device=dev)
        out = torch.empty((N, HV, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(gdn.gdn_prefill_workspace_size(gdn.problem_of(q, k, v, pool, idx)),
                         dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)
        calls = {
            "prefill_fwd": lambda: gdn.gdn_prefill_fwd(q, k, v, a, b, A_log, dt_bias, pool, idx,
                                                       cu, out=out, workspace=ws, stream=stream),
            "prefill_fwd_chunk_all": lambda: gdn.gdn_prefill_fwd(
                q, k, v, a, b, A_log, dt_bias, pool, idx, cu, out=out, workspace=ws,
                stream=stream, flags=gdn.GDN_FLAG_CHUNK_ALL),
            "recurrent_fwd": lambda: gdn.gdn_recurrent_fwd(q, k, v, a, b, A_log, dt_bias, pool,
                                                           idx, cu, out=out, stream=stream),
        }
        row = {"L": L, "N": N}
        for name, f in calls.items():
            row[name + "_ms"] = _time_launches(f, stream, args.steps, args.warmup)[0]
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del q, k, v, a, b, pool, out, ws
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "short-request dispatch: per-call ms of gdn_prefill_fwd, of the same call "
                  "with every request chunked, and of gdn_recurrent_fwd",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic (torch.randn, seed 7)",
        "config": {"workload": f"B={B} requests of L tokens, H={H} HV={HV} dk=dv={D}",
                   "short_request_threshold": gdn.GDN_SHORT_REQUEST},
        "rows": rows, "kernel_source_hash": kernel_source_hash()}), flush=True)


def bench_pipelined(args):
    """Successive prefill calls as a serving loop issues them: back to back on one stream,
    and pipelined over two streams, where each call starts once the previous call's chunk
    prep has ended (gdn_prefill_fwd_events marks it), so that its prep overlaps the previous
    call's state pass; the calls alternate between two sets of workspace, output and pool.
    Prints one JSON line with the wall ms per call of each on workloads 1-4 (or the one
    named by --workload): where a single call leaves compute units idle (one long request
    at d = 256 fills half of the device in its state pass), the second stream fills them."""
    import numpy as np
    import torch

    import gated_deltanet_prefill_gdn_amd as gdn
    import gdn_synth

    dev = torch.device("cuda:0")

    def t(x, dt=None):
        x = torch.from_numpy(np.ascontiguousarray(x))
        return (x.view(dt) if dt is not None else x).to(dev)

    rows = []
    for wi in ([args.workload] if args.workload is not None else [1] + list(SUB_WORKLOADS)):
        p = gdn_synth.workload(wi)
        q, k, v = (t(getattr(p, n).view(np.int16), torch.bfloat16) for n in "qkv")
        a, b, A_log, dt_bias = t(p.a), t(p.b), t(p.A_log), t(p.dt_bias)
        idx, cu = t(p.cache_indices), t(p.cu_seqlens)
        sets = []
        for _ in range(2):
            pool = t(p.state_pool.copy())
            ws_bytes = gdn.gdn_prefill_workspace_size(gdn.problem_of(q, k, v, pool, idx))
            evs = [torch.cuda.Event() for _ in range(gdn.GDN_NUM_STAGES + 1)]
            for e in evs:
                e.record()  # creates the event
            sets.append({"pool": pool, "evs": evs,
                         "out": torch.empty((p.N, p.HV, p.dv), dtype=v.dtype, device=dev),
                         "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev)})
        streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
        torch.cuda.synchronize()

        def call(st, stream):
            gdn.gdn_prefill_fwd_events(q, k, v, a, b, A_log, dt_bias, st["pool"], idx, cu,
                                       [e.cuda_event for e in st["evs"]], out=st["out"],
                                       workspace=st["ws"], stream=stream)

        def serial(n):
            for i in range(n):
                call(sets[i % 2], streams[0])

        def pipelined(n):
            for i in range(n):
                if i > 0:  # event 2 is recorded when the previous call's prep has ended
                    streams[i % 2].wait_event(sets[(i - 1) % 2]["evs"][2])
                call(sets[i % 2], streams[i % 2])

        def per_call_ms(f):
            f(max(2, args.warmup))
            torch.cuda.synchronize()
            best = float("inf")
            for _ in range(3):
                t0 = time.perf_counter()
                f(args.steps)
                torch.cuda.synchronize()
                best = min(best, (time.perf_counter() - t0) * 1e3 / args.steps)
            return best

        ms_s, ms_p = per_call_ms(serial), per_call_ms(pipelined)
        row = {"workload": gdn_synth.WORKLOADS[wi], "index": wi, "tokens": int(p.N),
               "serial_ms_per_call": round(ms_s, 4), "pipelined_ms_per_call": round(ms_p, 4),
               "pipelined_tokens_per_s": p.N / (ms_p * 1e-3),
               "pipelined_over_serial_rate": round(ms_s / ms_p, 3)}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del q, k, v, a, b, sets
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "successive gdn_prefill_fwd calls: wall ms per call back to back on one "
                  "stream and pipelined over two streams (each call after the previous "
                  "call's chunk prep)",
        "value": None, "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller)", "rows": rows,
        "kernel_source_hash": kernel_source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--op", choices=("prefill", "decode", "promote", "verify", "backward",
                                     "crossover", "pipelined"),
                    default="prefill",
                    help="the call a step times (default: the prefill forward)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra calls timed one by one after a 512 MiB cache flush")
    ap.add_argument("--workload", type=int, choices=(0, 1, 2, 3, 4), default=None,
                    help="time only this named workload (default: workload 1, with "
                         "workloads 2-4 as sub-results)")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the sub-results for workloads 2-4")
    ap.add_argument("--dtype", choices=("bf16", "f32"), default=None,
                    help="draw the prefill workloads with q, k, v in this dtype instead of "
                         "their own (f32 runs the fp32-arithmetic kernels)")
    ap.add_argument("--chunk", type=int, choices=(64, 128), default=64,
                    help="chunk size of the prefill (128: bf16 inputs with dk of 128 or 256; "
                         "the measured comparison of the two schedules)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    if args.op == "decode":
        bench_decode(args)
        return
    if args.op == "promote":
        bench_promote(args)
        return
    if args.op == "verify":
        bench_verify(args)
        return
    if args.op == "backward":
        bench_backward(args)
        return
    if args.op == "crossover":
        bench_crossover(args)
        return
    if args.op == "pipelined":
        bench_pipelined(args)
        return

    bench_prefill(args)


if __name__ == "__main__":
    main()
