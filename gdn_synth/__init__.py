"""Seeded synthetic inputs for the Gated DeltaNet prefill forward.

This module only draws numbers. It holds none of the method's arithmetic, so both
the CPU oracle side and the HIP side can take their inputs from it.

Generator
---------
* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014) in counter form: value ``i`` of a stream is the
  SplitMix64 finaliser applied to ``stream_seed + (i + 1) * 0x9E3779B97F4A7C15``.
* Uniforms take the top 53 bits: ``u = (z >> 11) * 2**-53`` in [0, 1).
* Normals come from the Box-Muller transform (Box and Muller, 1958) on pairs of
  uniforms, evaluated in fp64.
* Every tensor has its own stream: ``stream_seed = mix(seed ^ tensor_id)``.
* bf16 tensors are the fp64 draw rounded to fp32 (round to nearest even), then
  to bf16 (round to nearest even). They are returned as raw uint16 bit patterns;
  the exact value of each is ``float32(bits << 16)``.

Workloads
---------
The five named workloads follow the problem statement of the pymllm
``gdn_extend_chunkwise`` page (packed varlen tokens, H q/k heads, HV value heads,
fp32 state pool indexed per request) at the sizes listed in ``WORKLOADS``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libgdn_synth.so")
_lib = None

# tensor ids for per-tensor streams
TID_Q, TID_K, TID_V, TID_A, TID_B, TID_ALOG, TID_DTB, TID_STATE, TID_LEN, TID_PERM = range(1, 11)


def build(force: bool = True) -> str:
    """Compile the generator with gcc (IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _c():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, dbl, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_stream_seed.restype = u64
        L.synth_stream_seed.argtypes = [u64, u64]
        L.synth_uniform.restype = None
        L.synth_uniform.argtypes = [u64, u64, i64, i64, P]
        L.synth_normal.restype = None
        L.synth_normal.argtypes = [u64, u64, i64, dbl, dbl, ctypes.c_int, P, ctypes.c_int]
        L.synth_normal_f64.restype = None
        L.synth_normal_f64.argtypes = [u64, u64, i64, dbl, dbl, P]
        _lib = L
    return _lib


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


def stream_seed(seed: int, tensor_id: int) -> int:
    return int(_c().synth_stream_seed(seed & 0xFFFFFFFFFFFFFFFF, tensor_id))


def uniform(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _c().synth_uniform(seed, tensor_id, start, n, out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """n standard normals in fp64 (Box-Muller on uniform pairs)."""
    out = np.empty(n, dtype=np.float64)
    if n:
        _c().synth_normal_f64(seed, tensor_id, n, 0.0, 1.0, out.ctypes.data_as(ctypes.c_void_p))
    return out


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Problem:
    """One prefill call's inputs, host side, exactly as the boundary receives them.

    q, k: [N, H, dk]; v: [N, HV, dv]. For dtype "bf16" they are uint16 bit
    patterns, for "f32" float32. a, b: [N, HV] fp32. A_log, dt_bias: [HV] fp32.
    state_pool: [pool, HV, dv, dk] fp32. cache_indices: [B] int64.
    cu_seqlens: [B+1] int64.
    """
    name: str
    dtype: str
    H: int
    HV: int
    dk: int
    dv: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    state_pool: np.ndarray
    cache_indices: np.ndarray
    cu_seqlens: np.ndarray
    chunk_size: int = 64
    seed: int = 0

    @property
    def N(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def B(self) -> int:
        return int(self.cache_indices.shape[0])

    @property
    def pool(self) -> int:
        return int(self.state_pool.shape[0])

    def values_f32(self, name: str) -> np.ndarray:
        """q, k or v as exact fp32 values (bf16 widens exactly)."""
        x = getattr(self, name)
        return bf16_bits_to_f32(x) if self.dtype == "bf16" else x


def _draw(seed: int, tid: int, shape: Sequence[int], dtype: str, mean: float = 0.0, std: float = 1.0):
    """Normals * std + mean, rounded to fp32 (and then bf16 bit patterns for "bf16")."""
    n = int(np.prod(shape)) if len(shape) else 1
    bf = dtype == "bf16"
    out = np.empty(n, dtype=np.uint16 if bf else np.float32)
    if n:
        _c().synth_normal(seed, tid, n, float(mean), float(std), int(bf),
                          out.ctypes.data_as(ctypes.c_void_p), _threads())
    return out.reshape(shape)


def make_problem(
    seed: int,
    lengths: Sequence[int],
    H: int,
    HV: int,
    dk: int,
    dv: int,
    dtype: str = "bf16",
    pool: Optional[int] = None,
    cache_indices: Optional[Sequence[int]] = None,
    a_mean: float = 0.0,
    b_mean: float = 0.0,
    state_std: float = 0.0,
    dt_bias_std: float = 0.1,
    chunk_size: int = 64,
    name: str = "custom",
) -> Problem:
    """Generic seeded problem: q, k, v ~ N(0,1) raw (not normalised), a ~ N(a_mean,1),
    b ~ N(b_mean,1), A_log = log(1 + 15u) (so exp(A_log) ~ U[1,16]),
    dt_bias ~ N(0, dt_bias_std^2), state_pool ~ N(0, state_std^2) (zeros if 0)."""
    assert dtype in ("bf16", "f32")
    lengths = [int(x) for x in lengths]
    B = len(lengths)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    N = int(cu[-1])
    if pool is None:
        pool = B
    if cache_indices is None:
        cache_indices = list(range(B))
    idx = np.asarray(cache_indices, dtype=np.int64)
    q = _draw(seed, TID_Q, (N, H, dk), dtype)
    k = _draw(seed, TID_K, (N, H, dk), dtype)
    v = _draw(seed, TID_V, (N, HV, dv), dtype)
    a = _draw(seed, TID_A, (N, HV), "f32", mean=a_mean)
    b = _draw(seed, TID_B, (N, HV), "f32", mean=b_mean)
    A_log = np.log1p(15.0 * uniform(seed, TID_ALOG, HV)).astype(np.float32)
    dt_bias = _draw(seed, TID_DTB, (HV,), "f32", std=dt_bias_std)
    if state_std > 0:
        state = _draw(seed, TID_STATE, (pool, HV, dv, dk), "f32", std=state_std)
    else:
        state = np.zeros((pool, HV, dv, dk), dtype=np.float32)
    return Problem(name=name, dtype=dtype, H=H, HV=HV, dk=dk, dv=dv, q=q, k=k, v=v, a=a, b=b,
                   A_log=A_log, dt_bias=dt_bias, state_pool=state, cache_indices=idx,
                   cu_seqlens=cu, chunk_size=chunk_size, seed=seed)


def seeded_permutation(seed: int, tid: int, n: int) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the uniform stream."""
    u = uniform(seed, tid, n)
    perm = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(u[n - 1 - i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


# Named workloads. Seeds are 1000 + index.
WORKLOADS = {
    0: "tiny fp32: B=1 T=256 H=HV=1 dk=dv=64 C=64, zero state",
    1: "dense batch bf16: B=4 x T=4096 H=HV=16 dk=dv=128 C=64, zero state",
    2: "varlen GQA bf16: B=8 lengths U[1,8192] H=16 HV=32 dk=dv=128 C=64, pool 64 ~N(0,0.01)",
    3: "wide head bf16: B=1 T=16384 H=HV=8 dk=dv=256 C=64, zero state",
    4: "long prefill decay stress bf16: B=1 T=131072 H=16 HV=32 dk=dv=128 C=64, a~N(-4,1) b~N(2,1)",
}


def workload_lengths(idx: int) -> list:
    seed = 1000 + idx
    if idx == 0:
        return [256]
    if idx == 1:
        return [4096] * 4
    if idx == 2:
        u = uniform(seed, TID_LEN, 8)
        return [1 + int(8192 * x) for x in u]
    if idx == 3:
        return [16384]
    if idx == 4:
        return [131072]
    raise ValueError(idx)


def workload(idx: int, dtype: Optional[str] = None) -> Problem:
    """The five named workloads (see WORKLOADS). ``dtype`` ("bf16" or "f32") draws the same
    workload with q, k, v (and out) in that dtype instead of its own; its name then ends in
    that dtype."""
    if dtype is None:
        return _workload(idx)
    p = _workload(idx, dtype)
    p.name = p.name.rsplit("_", 1)[0] + "_" + dtype
    return p


def _workload(idx: int, dtype: Optional[str] = None) -> Problem:
    seed = 1000 + idx
    L = workload_lengths(idx)
    kw = {} if dtype is None else {"dtype": dtype}
    if idx == 0:
        return make_problem(seed, L, 1, 1, 64, 64, **{"dtype": "f32", **kw}, name="tiny_f32")
    if idx == 1:
        return make_problem(seed, L, 16, 16, 128, 128, **kw, name="dense_batch_bf16")
    if idx == 2:
        perm = seeded_permutation(seed, TID_PERM, 64)
        return make_problem(seed, L, 16, 32, 128, 128, pool=64, cache_indices=perm[:8],
                            state_std=0.1, **kw, name="varlen_gqa_bf16")
    if idx == 3:
        return make_problem(seed, L, 8, 8, 256, 256, **kw, name="wide_head_bf16")
    if idx == 4:
        return make_problem(seed, L, 16, 32, 128, 128, a_mean=-4.0, b_mean=2.0, state_std=0.1,
                            **kw, name="long_decay_bf16")
    raise ValueError(idx)


# The decode workload: one new token for each of 512 requests, the head layout of the
# varlen GQA workload (H = 16 q/k heads, HV = 32 value heads, dk = dv = 128, bf16), a pool of
# 512 slots ~N(0, 0.1^2) (the states a prefill left behind) taken in a seeded order.
DECODE_WORKLOAD = ("decode batch bf16: B=512 requests x 1 token, H=16 HV=32 dk=dv=128, "
                   "pool 512 ~N(0,0.01) in seeded order")


def make_decode_problem(seed: int, B: int, H: int, HV: int, dk: int, dv: int,
                        dtype: str = "bf16", pool: Optional[int] = None,
                        cache_indices: Optional[Sequence[int]] = None, state_std: float = 0.1,
                        a_mean: float = 0.0, b_mean: float = 0.0,
                        name: str = "decode") -> Problem:
    """A decode step's inputs: B requests of one token each (cu_seqlens = 0, 1, .., B),
    otherwise drawn as by make_problem."""
    return make_problem(seed, [1] * B, H, HV, dk, dv, dtype=dtype, pool=pool,
                        cache_indices=cache_indices, a_mean=a_mean, b_mean=b_mean,
                        state_std=state_std, name=name)


def decode_workload() -> Problem:
    seed = 1100
    perm = seeded_permutation(seed, TID_PERM, 512)
    return make_decode_problem(seed, 512, 16, 32, 128, 128, pool=512, cache_indices=perm,
                               state_std=0.1, name="decode_batch_bf16")


# Speculative-decoding verification: 512 requests, each bringing 4 tokens (3 drafted + 1),
# with the decode workload's heads and pool.
VERIFY_WORKLOAD = ("verify batch bf16: B=512 requests x 4 tokens, H=16 HV=32 dk=dv=128, "
                   "pool 512 ~N(0,0.01) in seeded order")


def verify_workload(tokens: int = 4) -> Problem:
    seed = 1300
    perm = seeded_permutation(seed, TID_PERM, 512)
    return make_problem(seed, [tokens] * 512, 16, 32, 128, 128, dtype="bf16", pool=512,
                        cache_indices=perm, state_std=0.1, name="verify_batch_bf16")


# ---------------------------------------------------------------- Promote update scan
TID_PK, TID_PV, TID_PBETA, TID_PW, TID_PGAMMA, TID_PM = range(21, 27)

# The Promote workload: batch 8 x 16 heads, dk = dv = 128, 64 pairs per firing (a level's
# query count), 64 firings (a level firing every second 64-token chunk of an 8192-token
# sequence), bf16 keys and values, every firing's state kept.
PROMOTE_WORKLOAD = ("promote scan bf16: BH=8x16, F=64 firings x n=64 pairs, dk=dv=128, "
                    "states kept")


@dataclasses.dataclass
class PromoteProblem:
    """One Promote update scan's inputs. K [BH, F, n, dk] (rows of unit length before
    rounding), V [BH, F, n, dv]: uint16 bf16 bit patterns for "bf16", float32 for "f32".
    beta, w [BH, F, n] in (0, 1); gamma [BH, F, dk] <= 0; M0 [BH, dk, dv] fp32."""
    dtype: str
    K: np.ndarray
    V: np.ndarray
    beta: np.ndarray
    w: np.ndarray
    gamma: np.ndarray
    M0: np.ndarray
    seed: int = 0

    @property
    def shape(self):
        BH, F, n, dk = self.K.shape
        return BH, F, n, dk, self.V.shape[3]

    def values_f32(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        return bf16_bits_to_f32(x) if self.dtype == "bf16" else x


def make_promote_problem(seed: int, BH: int, F: int, n: int, dk: int, dv: int,
                         dtype: str = "bf16", gamma_max: float = 0.5,
                         m_std: float = 0.5) -> PromoteProblem:
    """Keys: normal rows scaled to unit length in fp64, then rounded; values N(0, 1);
    beta, w ~ U(0, 1); gamma ~ -U(0, gamma_max) (decay factors in [e^-gamma_max, 1]);
    M0 ~ N(0, m_std^2)."""
    assert dtype in ("bf16", "f32")
    kr = normal(seed, TID_PK, BH * F * n * dk).reshape(BH, F, n, dk)
    kr /= np.sqrt((kr * kr).sum(axis=-1, keepdims=True))
    k32 = kr.astype(np.float32)
    K = f32_to_bf16_bits(k32).reshape(k32.shape) if dtype == "bf16" else k32
    V = _draw(seed, TID_PV, (BH, F, n, dv), dtype)
    beta = uniform(seed, TID_PBETA, BH * F * n).astype(np.float32).reshape(BH, F, n)
    w = uniform(seed, TID_PW, BH * F * n).astype(np.float32).reshape(BH, F, n)
    gamma = (-gamma_max * uniform(seed, TID_PGAMMA, BH * F * dk)).astype(np.float32)
    M0 = _draw(seed, TID_PM, (BH, dk, dv), "f32", std=m_std)
    return PromoteProblem(dtype=dtype, K=K, V=V, beta=beta, w=w,
                          gamma=gamma.reshape(BH, F, dk), M0=M0, seed=seed)


def promote_workload() -> PromoteProblem:
    return make_promote_problem(1200, 128, 64, 64, 128, 128, dtype="bf16")
