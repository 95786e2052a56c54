"""Python binding of libgdn (Gated DeltaNet chunkwise prefill forward and decode step on
MI355X).

The names match the C ABI in include/gdn.h. This module only marshals
arguments: it checks tensor shapes, dtypes, devices and contiguity, allocates
``out`` and the workspace with torch when the caller does not pass them, and
hands raw device pointers to the library. Every step of the computation runs in
the library's HIP kernels; there is no fallback. If libgdn.so is not built the
import of the library fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same sources (the CPU sanitizer runs use it).
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(PKG, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE = 3
GDN_ERR_HIP = 4
GDN_ERR_BAD_INPUT = 5
GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1

GDN_NUM_STAGES = 5
STAGE_NAMES = ("gate", "chunk_prep", "state_operator", "state_combine", "state")
# The kernel each stage of a bf16 prefill launches (the profilers' names), by the state
# schedule gdn_prefill_state_schedule reports.
STAGE_KERNELS = {
    0: {"gate": "plan_kernel", "chunk_prep": "mfma_prep_kernel", "state_operator": "-",
        "state_combine": "-", "state": "mfma_state_kernel"},
    1: {"gate": "plan_kernel", "chunk_prep": "mfma_prep_kernel",
        "state_operator": "chain_kernel<operator>", "state_combine": "combine_kernel",
        "state": "chain_kernel<out>"},
    2: {"gate": "gate_kernel", "chunk_prep": "ref_prep_kernel", "state_operator": "-",
        "state_combine": "-", "state": "ref_state_kernel"},
}

GDN_NOALLOC_SCRATCH_BYTES = 64 << 20

GDN_SCHEDULE_COLUMN_SLICES = 0
GDN_SCHEDULE_SEGMENTS = 1
GDN_SCHEDULE_FP32 = 2

GDN_FLAG_CHUNK_ALL = 1   # gdn_problem_t.flags: chunk every request
GDN_SHORT_REQUEST = 10   # requests of at most this many tokens take the token recurrence
GDN_SPLIT_MEAN_LENGTH = 64  # ... in batches whose mean request length is at most this

EXPORTED = ("gdn_prefill_workspace_size", "gdn_prefill_state_schedule", "gdn_prefill_fwd",
            "gdn_prefill_fwd_events", "gdn_prefill_fwd_noalloc", "gdn_prefill_nonfinite",
            "gdn_prefill_bwd_workspace_size", "gdn_prefill_bwd",
            "gdn_decode_fwd", "gdn_recurrent_fwd", "gdn_promote_scan", "gdn_validate_inputs",
            "gdn_status_str", "gdn_version")


class GdnProblem(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("pool_size", ctypes.c_int64),
        ("qkv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class GdnPromoteProblem(ctypes.Structure):
    _fields_ = [
        ("scans", ctypes.c_int64),
        ("firings", ctypes.c_int32),
        ("pairs", ctypes.c_int32),
        ("head_k", ctypes.c_int32),
        ("head_v", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_str(status)})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Open libgdn.so and declare the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    import torch  # noqa: F401  (load torch's HIP runtime first so libgdn shares it)
    if not os.path.exists(path):
        raise ImportError(f"libgdn.so is not built at {path}; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(GdnProblem)
    L.gdn_prefill_workspace_size.restype = ctypes.c_size_t
    L.gdn_prefill_workspace_size.argtypes = [PP, ctypes.c_int32]
    L.gdn_prefill_bwd_workspace_size.restype = ctypes.c_size_t
    L.gdn_prefill_bwd_workspace_size.argtypes = [PP, ctypes.c_int32]
    L.gdn_prefill_bwd.restype = ctypes.c_int
    L.gdn_prefill_bwd.argtypes = [P] * 10 + [ctypes.c_int32] + [P] * 10 + [PP, P, ctypes.c_size_t,
                                                                          P]
    L.gdn_prefill_nonfinite.restype = ctypes.c_int
    L.gdn_prefill_nonfinite.argtypes = [P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32), P]
    L.gdn_prefill_state_schedule.restype = ctypes.c_int32
    L.gdn_prefill_state_schedule.argtypes = [PP, ctypes.c_int32]
    L.gdn_prefill_fwd.restype = ctypes.c_int
    L.gdn_prefill_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, PP, P,
                                  ctypes.c_size_t, P]
    L.gdn_prefill_fwd_noalloc.restype = ctypes.c_int
    L.gdn_prefill_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, PP, P]
    L.gdn_prefill_fwd_events.restype = ctypes.c_int
    L.gdn_prefill_fwd_events.argtypes = L.gdn_prefill_fwd.argtypes + [P]
    L.gdn_decode_fwd.restype = ctypes.c_int
    L.gdn_decode_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, PP, P]
    L.gdn_recurrent_fwd.restype = ctypes.c_int
    L.gdn_recurrent_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, PP, P]
    L.gdn_promote_scan.restype = ctypes.c_int
    L.gdn_promote_scan.argtypes = [P, P, P, P, P, P, P, ctypes.POINTER(GdnPromoteProblem), P]
    L.gdn_validate_inputs.restype = ctypes.c_int
    L.gdn_validate_inputs.argtypes = [P, P, PP, P]
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_status_str.argtypes = [ctypes.c_int]
    L.gdn_version.restype = ctypes.c_int32
    L.gdn_version.argtypes = []
    if path == LIB_PATH:
        _lib = L
    return L


def status_str(status: int) -> str:
    return load_library().gdn_status_str(int(status)).decode()


def gdn_version() -> int:
    return int(load_library().gdn_version())


def make_problem(N: int, B: int, H: int, HV: int, dk: int, dv: int, pool: int,
                 dtype: int, flags: int = 0) -> GdnProblem:
    return GdnProblem(int(N), int(B), int(H), int(HV), int(dk), int(dv), int(pool), int(dtype),
                      int(flags))


def gdn_prefill_workspace_size(prob: GdnProblem, chunk_size: int = 64) -> int:
    return int(load_library().gdn_prefill_workspace_size(ctypes.byref(prob), int(chunk_size)))


def gdn_prefill_state_schedule(prob: GdnProblem, chunk_size: int = 64) -> int:
    """GDN_SCHEDULE_* of the kernels that run a call's state pass (-1 if invalid)."""
    return int(load_library().gdn_prefill_state_schedule(ctypes.byref(prob), int(chunk_size)))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype=None, ndim=None, device=None):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def problem_of(q, k, v, state_pool, cache_indices, flags: int = 0) -> GdnProblem:
    N, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    return make_problem(N, cache_indices.shape[0], H, HV, dk, dv, state_pool.shape[0],
                        _dtype_code(q), flags)


def gdn_recurrent_fwd(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                      out=None, stream=None):
    """The prefill's operation evaluated token by token (no chunks, no workspace), for short
    requests; same arguments and result as gdn_prefill_fwd."""
    import torch
    prob, out = _check_prefill_args(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                                    cu_seqlens, out)
    st = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    rc = load_library().gdn_recurrent_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(cache_indices), _ptr(cu_seqlens), _ptr(out), ctypes.byref(prob),
        ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_recurrent_fwd")
    return out


def gdn_prefill_fwd(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                    chunk_size: int = 64, out=None, workspace=None, stream=None, flags: int = 0):
    """``chunk_size``: 64, or 128 for bf16 inputs with dk of 128 or 256 (the same result
    within rounding; 64 is the faster schedule). ``flags``: GDN_FLAG_* bits of the problem
    descriptor (GDN_FLAG_CHUNK_ALL: chunk every request, none through the token
    recurrence)."""
    return _prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                    chunk_size, out, workspace, stream, None, flags)


def gdn_prefill_fwd_noalloc(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                            cu_seqlens, out, chunk_size: int = 64, stream=None, flags: int = 0):
    """gdn_prefill_fwd on the library's built-in device workspace: allocates nothing, so
    ``out`` must be given. Problems whose workspace exceeds GDN_NOALLOC_SCRATCH_BYTES raise
    GdnError(GDN_ERR_WORKSPACE); calls that may overlap on one GPU must be serialised."""
    import torch
    prob, out = _check_prefill_args(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                                    cu_seqlens, out, flags=flags)
    st = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    rc = load_library().gdn_prefill_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(cache_indices), _ptr(cu_seqlens), int(chunk_size), _ptr(out),
        ctypes.byref(prob), ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_fwd_noalloc")
    return out


def gdn_prefill_fwd_events(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                           cu_seqlens, stage_events, chunk_size: int = 64, out=None,
                           workspace=None, stream=None, flags: int = 0):
    """gdn_prefill_fwd that records the GDN_NUM_STAGES + 1 caller-created hipEvent_t
    handles in ``stage_events`` (ints) on the stream around the stages."""
    if len(stage_events) != GDN_NUM_STAGES + 1:
        raise ValueError("need GDN_NUM_STAGES + 1 events")
    arr = (ctypes.c_void_p * len(stage_events))(*[int(e) for e in stage_events])
    return _prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                    chunk_size, out, workspace, stream, arr, flags)


def _check_prefill_args(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                        out, want_out: bool = True, flags: int = 0):
    """Shapes, dtypes, devices and contiguity of a prefill call's tensors; allocates ``out``
    if it is None. Returns (problem descriptor, out)."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_prefill_fwd runs on a HIP device; tensors are on " + str(dev))
    _need(q, "q", ndim=3, device=dev)
    _need(k, "k", dtype=q.dtype, ndim=3, device=dev)
    _need(v, "v", dtype=q.dtype, ndim=3, device=dev)
    N, H, dk = q.shape
    if tuple(k.shape) != (N, H, dk):
        raise ValueError(f"k shape {tuple(k.shape)} != q shape {tuple(q.shape)}")
    HV, dv = v.shape[1], v.shape[2]
    if v.shape[0] != N:
        raise ValueError("v must have N rows")
    for t, name in ((a, "a"), (b, "b")):
        _need(t, name, dtype=torch.float32, ndim=2, device=dev)
        if tuple(t.shape) != (N, HV):
            raise ValueError(f"{name} must be [N, HV] = {(N, HV)}, got {tuple(t.shape)}")
    for t, name in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, name, dtype=torch.float32, ndim=1, device=dev)
        if t.shape[0] != HV:
            raise ValueError(f"{name} must be [HV]")
    _need(state_pool, "state_pool", dtype=torch.float32, ndim=4, device=dev)
    if tuple(state_pool.shape[1:]) != (HV, dv, dk):
        raise ValueError(f"state_pool must be [pool, {HV}, {dv}, {dk}], got {tuple(state_pool.shape)}")
    _need(cache_indices, "cache_indices", dtype=torch.int64, ndim=1, device=dev)
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int64, ndim=1, device=dev)
    if cu_seqlens.shape[0] != cache_indices.shape[0] + 1:
        raise ValueError("cu_seqlens must have B + 1 entries")
    prob = problem_of(q, k, v, state_pool, cache_indices, flags)
    if not want_out:
        return prob, None
    if out is None:
        out = torch.empty((N, HV, dv), dtype=v.dtype, device=dev)
    else:
        _need(out, "out", dtype=v.dtype, ndim=3, device=dev)
        if tuple(out.shape) != (N, HV, dv):
            raise ValueError("out must be [N, HV, dv]")
    return prob, out


def _prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
             chunk_size, out, workspace, stream, events, flags=0):
    """GDN prefill forward on device tensors; returns ``out`` [N, HV, dv] in v's dtype.

    q, k [N, H, dk] and v [N, HV, dv] bf16/fp32; a, b [N, HV] fp32; A_log, dt_bias [HV]
    fp32; state_pool [pool, HV, dv, dk] fp32 (updated in place); cache_indices [B]
    int64; cu_seqlens [B+1] int64. ``workspace`` is an optional uint8 device tensor of at
    least gdn_prefill_workspace_size bytes. ``stream``: a torch stream (default: current).
    """
    import torch
    dev = q.device
    N, HV = q.shape[0], v.shape[1]
    prob, out = _check_prefill_args(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                                    cu_seqlens, out, flags=flags)
    need = gdn_prefill_workspace_size(prob, chunk_size)
    if need == 0 and (N > 0 and cache_indices.shape[0] > 0):
        raise GdnError(GDN_ERR_UNSUPPORTED, "gdn_prefill_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
            _ptr(state_pool), _ptr(cache_indices), _ptr(cu_seqlens), int(chunk_size), _ptr(out),
            ctypes.byref(prob), _ptr(workspace), workspace.numel(), ctypes.c_void_p(st))
    L = load_library()
    rc = L.gdn_prefill_fwd(*args) if events is None else L.gdn_prefill_fwd_events(*args, events)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_fwd")
    return out


def gdn_prefill_bwd_workspace_size(prob: GdnProblem, chunk_size: int = 64) -> int:
    return int(load_library().gdn_prefill_bwd_workspace_size(ctypes.byref(prob),
                                                              int(chunk_size)))


def gdn_prefill_bwd(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                    dout, dstate, chunk_size: int = 64, workspace=None, stream=None):
    """Gradients of a prefill call's inputs (see gdn_prefill_bwd in include/gdn.h).
    state_pool: the pool as it was BEFORE the forward call; dout [N, HV, dv] in v's dtype;
    dstate [B, HV, dv, dk] fp32. Returns a dict of fp32 tensors dq, dk, dv, da, db, dA_log,
    ddt_bias, dstate0."""
    import torch
    dev = q.device
    prob, _ = _check_prefill_args(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices,
                                  cu_seqlens, None, want_out=False)
    N, H, dk_ = q.shape
    HV, dv_ = v.shape[1], v.shape[2]
    B = cache_indices.shape[0]
    _need(dout, "dout", dtype=v.dtype, ndim=3, device=dev)
    if tuple(dout.shape) != (N, HV, dv_):
        raise ValueError("dout must be [N, HV, dv]")
    _need(dstate, "dstate", dtype=torch.float32, ndim=4, device=dev)
    if tuple(dstate.shape) != (B, HV, dv_, dk_):
        raise ValueError("dstate must be [B, HV, dv, dk]")
    f = dict(device=dev, dtype=torch.float32)
    g = {"dq": torch.empty((N, H, dk_), **f), "dk": torch.empty((N, H, dk_), **f),
         "dv": torch.empty((N, HV, dv_), **f), "da": torch.empty((N, HV), **f),
         "db": torch.empty((N, HV), **f), "dA_log": torch.empty((HV,), **f),
         "ddt_bias": torch.empty((HV,), **f), "dstate0": torch.empty((B, HV, dv_, dk_), **f)}
    need = gdn_prefill_bwd_workspace_size(prob, chunk_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    rc = load_library().gdn_prefill_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(cache_indices), _ptr(cu_seqlens), int(chunk_size), _ptr(dout),
        _ptr(dstate), *[_ptr(g[n]) for n in ("dq", "dk", "dv", "da", "db", "dA_log",
                                             "ddt_bias", "dstate0")],
        ctypes.byref(prob), _ptr(workspace), workspace.numel(), ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_bwd")
    return g


def gdn_prefill_nonfinite(workspace, stream=None) -> bool:
    """Whether the last prefill call that ran with this workspace left a non-finite final
    state (synchronises the stream)."""
    import torch
    _need(workspace, "workspace", dtype=torch.uint8, ndim=1)
    st = (stream or torch.cuda.current_stream(workspace.device)).cuda_stream
    flag = ctypes.c_int32(0)
    rc = load_library().gdn_prefill_nonfinite(_ptr(workspace), workspace.numel(),
                                              ctypes.byref(flag), ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_prefill_nonfinite")
    return bool(flag.value)


def gdn_decode_fwd(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, out=None,
                   stream=None):
    """One decode step on device tensors (one token per request); returns ``out``
    [B, HV, dv] in v's dtype.

    q, k [B, H, dk] and v [B, HV, dv] bf16/fp32; a, b [B, HV] fp32; A_log, dt_bias [HV]
    fp32; state_pool [pool, HV, dv, dk] fp32 (updated in place); cache_indices [B] int64.
    ``stream``: a torch stream (default: current)."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn_decode_fwd runs on a HIP device; tensors are on " + str(dev))
    _need(q, "q", ndim=3, device=dev)
    _need(k, "k", dtype=q.dtype, ndim=3, device=dev)
    _need(v, "v", dtype=q.dtype, ndim=3, device=dev)
    B, H, dk = q.shape
    if tuple(k.shape) != (B, H, dk):
        raise ValueError(f"k shape {tuple(k.shape)} != q shape {tuple(q.shape)}")
    HV, dv = v.shape[1], v.shape[2]
    if v.shape[0] != B:
        raise ValueError("v must have B rows")
    for t, name in ((a, "a"), (b, "b")):
        _need(t, name, dtype=torch.float32, ndim=2, device=dev)
        if tuple(t.shape) != (B, HV):
            raise ValueError(f"{name} must be [B, HV] = {(B, HV)}, got {tuple(t.shape)}")
    for t, name in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, name, dtype=torch.float32, ndim=1, device=dev)
        if t.shape[0] != HV:
            raise ValueError(f"{name} must be [HV]")
    _need(state_pool, "state_pool", dtype=torch.float32, ndim=4, device=dev)
    if tuple(state_pool.shape[1:]) != (HV, dv, dk):
        raise ValueError(f"state_pool must be [pool, {HV}, {dv}, {dk}], got {tuple(state_pool.shape)}")
    _need(cache_indices, "cache_indices", dtype=torch.int64, ndim=1, device=dev)
    if cache_indices.shape[0] != B:
        raise ValueError("cache_indices must have B entries")
    prob = problem_of(q, k, v, state_pool, cache_indices)
    if out is None:
        out = torch.empty((B, HV, dv), dtype=v.dtype, device=dev)
    else:
        _need(out, "out", dtype=v.dtype, ndim=3, device=dev)
        if tuple(out.shape) != (B, HV, dv):
            raise ValueError("out must be [B, HV, dv]")
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    rc = load_library().gdn_decode_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state_pool), _ptr(cache_indices), _ptr(out), ctypes.byref(prob),
        ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_fwd")
    return out


def gdn_promote_scan(K, V, beta, w, gamma, M, keep_states: bool = True, states=None,
                     stream=None):
    """The Promote update scan on device tensors; updates ``M`` in place and returns the
    per-firing states [scans, F, dk, dv] fp32 (or None when keep_states is False).

    K [scans, F, n, dk] and V [scans, F, n, dv] bf16; beta, w [scans, F, n] fp32;
    gamma [scans, F, dk] fp32; M [scans, dk, dv] fp32."""
    import torch
    dev = K.device
    if dev.type != "cuda":
        raise ValueError("gdn_promote_scan runs on a HIP device; tensors are on " + str(dev))
    _need(K, "K", ndim=4, device=dev)
    _need(V, "V", dtype=K.dtype, ndim=4, device=dev)
    BH, F, n, dk = K.shape
    dv = V.shape[3]
    if tuple(V.shape[:3]) != (BH, F, n):
        raise ValueError(f"V must be [{BH}, {F}, {n}, dv], got {tuple(V.shape)}")
    for t, name in ((beta, "beta"), (w, "w")):
        _need(t, name, dtype=torch.float32, ndim=3, device=dev)
        if tuple(t.shape) != (BH, F, n):
            raise ValueError(f"{name} must be [{BH}, {F}, {n}]")
    _need(gamma, "gamma", dtype=torch.float32, ndim=3, device=dev)
    if tuple(gamma.shape) != (BH, F, dk):
        raise ValueError(f"gamma must be [{BH}, {F}, {dk}]")
    _need(M, "M", dtype=torch.float32, ndim=3, device=dev)
    if tuple(M.shape) != (BH, dk, dv):
        raise ValueError(f"M must be [{BH}, {dk}, {dv}]")
    if keep_states and states is None:
        states = torch.empty((BH, F, dk, dv), dtype=torch.float32, device=dev)
    if states is not None:
        _need(states, "states", dtype=torch.float32, ndim=4, device=dev)
        if tuple(states.shape) != (BH, F, dk, dv):
            raise ValueError(f"states must be [{BH}, {F}, {dk}, {dv}]")
    prob = GdnPromoteProblem(int(BH), int(F), int(n), int(dk), int(dv), _dtype_code(K), 0)
    st = (stream or torch.cuda.current_stream(dev)).cuda_stream
    rc = load_library().gdn_promote_scan(_ptr(K), _ptr(V), _ptr(beta), _ptr(w), _ptr(gamma),
                                         _ptr(M), _ptr(states), ctypes.byref(prob),
                                         ctypes.c_void_p(st))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_promote_scan")
    return states


def gdn_validate_inputs(cu_seqlens, cache_indices, prob: GdnProblem, stream=None) -> int:
    """Debug check of cu_seqlens / cache_indices contents (synchronises). Returns a status."""
    import torch
    st = (stream or torch.cuda.current_stream(cu_seqlens.device)).cuda_stream
    return int(load_library().gdn_validate_inputs(_ptr(cu_seqlens), _ptr(cache_indices),
                                                  ctypes.byref(prob), ctypes.c_void_p(st)))
