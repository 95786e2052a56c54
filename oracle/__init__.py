"""CPU oracle for the Gated DeltaNet prefill forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library and
the HIP library never imports it.

Contents
--------
* ``prefill``: the token-by-token recurrence (C, fp64 or fp32 arithmetic) with the
  state-pool semantics of the pymllm ``gdn_extend_chunkwise`` page (Module
  Contents: ``state_pool [pool, HV, V, K]`` updated in place at the slot
  ``cache_indices[b]`` of each request; packed tokens split by ``cu_seqlens``).
* ``decode``: one token per request, i.e. one step of the same recurrence from each
  request's slot (the same page: the pool and indices carry the state into the
  decoding that follows the prefill). It is ``prefill`` with ``cu_seqlens`` = 0..B.
* ``chunked``: the chunkwise forms of the pages in fp64 (self-checks only).
* ``bruteforce``: dense products of the per-token transition matrices.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, a hand-worked example, brute force, invariants). Conventions the
pages leave open (q/k head for value head hv is hv // (HV/H); no query scale;
eps = 1e-6 inside the L2 norm) are not pinned by the pages.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library at ``path`` and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.gdn_oracle_recurrence.restype = ctypes.c_int
    L.gdn_oracle_recurrence.argtypes = [
        ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, P, P, ctypes.c_double, ctypes.c_int, ctypes.c_int]
    L.gdn_oracle_gates.restype = None
    L.gdn_oracle_gates.argtypes = [ctypes.c_double] * 4 + [ctypes.POINTER(ctypes.c_double)] * 3
    return L


def lib():
    global _lib
    if _lib is None:
        override = os.environ.get("GDN_ORACLE_LIB")   # a planted-mistake build (tests only)
        if override:
            _lib = load_library(override)
        else:
            if not os.path.exists(_LIB):
                build()
            _lib = load_library(_LIB)
    return _lib


def set_library(L):
    """Swap the library every call here uses (the tests plant mistakes this way);
    returns the previous one."""
    global _lib
    prev, _lib = _lib, L
    return prev


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def gates(a: float, b: float, A_log: float, dt_bias: float):
    """(alpha, beta, g) for one token/head, from the C oracle."""
    al, be, g = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    lib().gdn_oracle_gates(float(a), float(b), float(A_log), float(dt_bias),
                           ctypes.byref(al), ctypes.byref(be), ctypes.byref(g))
    return al.value, be.value, g.value


@dataclasses.dataclass
class OracleResult:
    out: np.ndarray          # [N, n_heads, n_rows] fp64
    state_pool: np.ndarray   # [pool, HV, dv, dk] fp64: the pool after the call
    heads: np.ndarray        # selected value heads
    rows: tuple              # (row_lo, row_hi)


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def recurrence_raw(in_dtype: str, q, k, v, a, b, A_log, dt_bias, cu_seqlens, H, HV, dk, dv,
                   S0: np.ndarray, heads: Sequence[int], rows=None, eps: float = EPS,
                   fp32_arith: bool = False, nthreads: Optional[int] = None):
    """Run the recurrence for every sequence from explicit initial states.

    S0: [B, n_heads, n_rows, dk] fp64 initial states. Returns (out, S_final)."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    N = int(cu[-1]) if B >= 0 else 0
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    r0, r1 = (0, dv) if rows is None else rows
    nr = r1 - r0
    S = np.ascontiguousarray(S0, dtype=np.float64).copy()
    assert S.shape == (B, heads.shape[0], nr, dk), S.shape
    out = np.zeros((N, heads.shape[0], nr), dtype=np.float64)
    dt = {"f32": 0, "bf16": 1}[in_dtype]
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    if N == 0:
        # empty inputs: give the C code valid (dummy) pointers
        q = q if q.size else np.zeros(1, q.dtype)
        k = k if k.size else np.zeros(1, k.dtype)
        v = v if v.size else np.zeros(1, v.dtype)
        a = a if a.size else np.zeros(1, np.float32)
        b = b if b.size else np.zeros(1, np.float32)
        out = np.zeros((0, heads.shape[0], nr), dtype=np.float64)
        outbuf = np.zeros(1, dtype=np.float64)
    else:
        outbuf = out
    rc = lib().gdn_oracle_recurrence(
        dt, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(cu),
        B, H, HV, dk, dv, _ptr(heads), heads.shape[0], r0, r1,
        _ptr(S) if S.size else _ptr(np.zeros(1)), _ptr(outbuf), float(eps), int(fp32_arith),
        int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, S


def prefill(p, heads: Optional[Sequence[int]] = None, rows=None, eps: float = EPS,
            fp32_arith: bool = False, nthreads: Optional[int] = None) -> OracleResult:
    """The prefill call on a ``gdn_synth.Problem``: every sequence b starts from
    ``state_pool[cache_indices[b]]``, runs the recurrence over its tokens and writes
    its final state back to the same slot; ``out`` holds o_t for every token."""
    if heads is None:
        heads = list(range(p.HV))
    heads = np.asarray(heads, dtype=np.int32)
    r0, r1 = (0, p.dv) if rows is None else rows
    pool64 = p.state_pool.astype(np.float64)
    idx = np.asarray(p.cache_indices, dtype=np.int64)
    S0 = pool64[idx][:, heads, r0:r1, :]            # [B, n_heads, rows, dk]
    out, S = recurrence_raw(p.dtype, p.q, p.k, p.v, p.a, p.b, p.A_log, p.dt_bias, p.cu_seqlens,
                            p.H, p.HV, p.dk, p.dv, S0, heads, (r0, r1), eps, fp32_arith, nthreads)
    new_pool = pool64.copy()
    for bi, slot in enumerate(idx):
        for j, hv in enumerate(heads):
            new_pool[slot, hv, r0:r1, :] = S[bi, j]
    return OracleResult(out=out, state_pool=new_pool, heads=heads, rows=(r0, r1))


def decode(p, heads: Optional[Sequence[int]] = None, rows=None, eps: float = EPS,
           fp32_arith: bool = False, nthreads: Optional[int] = None) -> OracleResult:
    """The decode step on a ``gdn_synth.Problem`` whose requests hold one token each
    (row b of q, k, v, a, b is request b's token): one step of the recurrence from
    ``state_pool[cache_indices[b]]``, the state written back to that slot, and
    ``out[b] = S_new q`` (state-transition equation of "Simple math to speed up GDN
    prefill", section Reminder). Same arithmetic as ``prefill``."""
    cu = np.asarray(p.cu_seqlens, dtype=np.int64)
    if not np.array_equal(cu, np.arange(p.B + 1, dtype=np.int64)):
        raise ValueError("a decode problem has exactly one token per request")
    return prefill(p, heads, rows, eps, fp32_arith, nthreads)
