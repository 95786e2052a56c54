// One decode step on the state pool: every request brings exactly one new token.
//
// For request b (row b of q, k, v, a, b), value head hv, q/k head h = hv / (HV / H) and
// slot s = cache_indices[b], the token's step of the recurrence ("Simple math to speed up
// GDN prefill" (veitner), section Reminder, state transition; gates and shapes from the
// pymllm gdn_chunkwise page, Module Contents) is
//   S   <- alpha S (I - beta kh kh^T) + beta v kh^T  =  alpha S + u kh^T,
//   u    = beta (v - alpha S kh),
//   out  = S_new qh = alpha (S qh) + (kh . qh) u,
// with kh, qh the L2-normalised k and q (S is dv x dk, fp32, updated in place). Row i of
// S (value index i) enters only through (S kh)_i and (S qh)_i, so the rows are
// independent: a group of dk / 8 lanes holds one row, 8 fp32 per lane, forms
// both dot products with cross-lane (DPP) sums over the group, and writes the new row. Each
// workgroup covers kRowsPerThread rows per lane group of one (request, value head), so
// a wave keeps kRowsPerThread x 2 KiB of state loads in flight, all issued before the
// first wait. The state is read once and written once: the kernel is bound by HBM
// bandwidth. Both the state loads and the state stores are non-temporal (the rows are
// touched once per call): with both, the decode workload's step takes 0.376 ms instead of
// 0.415 (5.8 instead of 5.2 TB/s); either alone changes nothing (measured).
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;
// Rows per lane group: a workgroup then covers 64 rows at dk = 64 and 128 and 32 at
// dk = 256, which divides every supported dv (64, 128, 256), so no row is out of range.
template <int DK>
constexpr int kRowsPerThread = DK == 64 ? 2 : 4;
template <int DK>
constexpr int kRowsPerBlock = (64 / (DK / 8)) * kRowsPerThread<DK> * (kDecodeThreads / 64);
static_assert(kRowsPerBlock<64> == 64 && kRowsPerBlock<128> == 64 && kRowsPerBlock<256> == 32,
              "a workgroup's rows divide dv");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += ((u >> 16) & 1u) + 0x7FFFu;
  return (uint16_t)(u >> 16);
}

// This lane's eight elements of a q or k row as fp32: 4 gl .. 4 gl + 3 and
// DK / 2 + 4 gl .. DK / 2 + 4 gl + 3 (the same split as its state columns).
template <int DK, bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t row0, int gl, float (&x)[8]) {
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + row0 + 4 * gl;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + DK / 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      x[2 * i] = bf16_to_f32(lo[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(lo[i] >> 16);
      x[4 + 2 * i] = bf16_to_f32(hi[i] & 0xFFFFu);
      x[4 + 2 * i + 1] = bf16_to_f32(hi[i] >> 16);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + row0 + 4 * gl;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + DK / 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = lo[i];
      x[4 + i] = hi[i];
    }
  }
}

// x from another lane of the same 16-lane row, chosen by a DPP control code.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes of a row group (aligned groups of LPR consecutive lanes, LPR >= 8),
// left in every lane of the group: lane ^ 1 and lane ^ 2 inside each quad, then the mirror
// images inside the half-row (the other quad) and the row (the other half), all as DPP
// moves; a 32-lane group adds the other row with a lane shuffle.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "8 to 32 lanes per row");
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

template <int DK, bool BF16>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ ga, const float* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int64_t* __restrict__ cache_indices, int H, int HV,
    int DV, int nrb, float* __restrict__ state_pool, void* __restrict__ out) {
  constexpr int LPR = DK / 8;                    // lanes per state row
  constexpr int RPW = 64 / LPR;                  // rows per wave and load
  constexpr int NR = kRowsPerThread<DK>;         // rows per lane group
  constexpr int RWV = RPW * NR;                  // rows per wave
  constexpr int RWG = kRowsPerBlock<DK>;         // rows per workgroup (divides dv)
  // The host keeps the grid below 2^31 blocks, so 32-bit index arithmetic suffices.
  const uint32_t x = blockIdx.x;
  const uint32_t pair32 = x / (uint32_t)nrb;
  const int rb = (int)(x - pair32 * (uint32_t)nrb);
  const uint32_t b32 = pair32 / (uint32_t)HV;
  const int hv = (int)(pair32 - b32 * (uint32_t)HV);
  const int h = hv / (HV / H);
  const int64_t pair = pair32;  // request * HV + value head
  const int64_t bi = b32;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int gl = l % LPR;  // this lane's columns: 4 gl .. 4 gl + 3 and DK/2 + 4 gl ..
  const int rg = l / LPR;  // row group inside the wave
  const int64_t slot = cache_indices[bi];
  const float a_t = ga[pair], b_t = gb[pair], alog = A_log[hv], dtb = dt_bias[hv];

  // This lane's rows: r0 + j RPW for j < NR. Its 8 columns are two runs of 4, one in
  // each half of the row, so that one load instruction of a wave covers the first (or
  // second) halves of RPW rows as RPW contiguous 2 DK-byte pieces with no gaps. The
  // state and v loads are issued first, so that their latency overlaps the loads and
  // reductions of q and k and the gates.
  const int r0 = rb * RWG + wv * RWV + rg;
  float vr[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int64_t vi = pair * DV + r0 + j * RPW;
    vr[j] = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(v)[vi])
                 : reinterpret_cast<const float*>(v)[vi];
  }
  float* Sp = state_pool + ((slot * HV + hv) * (int64_t)DV + r0) * DK + 4 * gl;
  f32x4 s[NR][2];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    s[j][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + j * RPW * DK));
    s[j][1] =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + j * RPW * DK + DK / 2));
  }

  // Normalised k and q slices, and kh . qh.
  float kk[8], qq[8];
  load8<DK, BF16>(k, (bi * H + h) * DK, gl, kk);
  load8<DK, BF16>(q, (bi * H + h) * DK, gl, qq);
  // Keep every load above this point: the scheduler would otherwise move some state
  // loads below the first row's stores to save registers, a second memory round trip.
  __builtin_amdgcn_sched_barrier(0);
  float ssk = 0.f, ssq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ssk = __builtin_fmaf(kk[e], kk[e], ssk);
    ssq = __builtin_fmaf(qq[e], qq[e], ssq);
  }
  ssk = group_sum<LPR>(ssk);
  ssq = group_sum<LPR>(ssq);
  const float rk = 1.0f / sqrtf(ssk + kNormEps), rq = 1.0f / sqrtf(ssq + kNormEps);
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kk[e] *= rk;
    qq[e] *= rq;
    kq = __builtin_fmaf(kk[e], qq[e], kq);
  }
  kq = group_sum<LPR>(kq);

  // Gates: g = log(alpha) = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b).
  const float xg = a_t + dtb;
  const float sp = fmaxf(xg, 0.f) + log1pf(expf(-fabsf(xg)));
  const float alpha = expf(-expf(alog) * sp);
  const float beta = 1.f / (1.f + expf(-b_t));

  float pk[NR], pq[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a0 = __builtin_fmaf(s[j][0][e], kk[e], a0);
      a0 = __builtin_fmaf(s[j][1][e], kk[4 + e], a0);
      a1 = __builtin_fmaf(s[j][0][e], qq[e], a1);
      a1 = __builtin_fmaf(s[j][1][e], qq[4 + e], a1);
    }
    pk[j] = a0;
    pq[j] = a1;
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    pk[j] = group_sum<LPR>(pk[j]);
    pq[j] = group_sum<LPR>(pq[j]);
  }

#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int r = r0 + j * RPW;
    const float u = beta * (vr[j] - alpha * pk[j]);
    f32x4 n0, n1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      n0[e] = __builtin_fmaf(alpha, s[j][0][e], u * kk[e]);
      n1[e] = __builtin_fmaf(alpha, s[j][1][e], u * kk[4 + e]);
    }
    __builtin_nontemporal_store(n0, reinterpret_cast<f32x4*>(Sp + j * RPW * DK));
    __builtin_nontemporal_store(n1, reinterpret_cast<f32x4*>(Sp + j * RPW * DK + DK / 2));
    if (gl == 0) {
      const float o = __builtin_fmaf(alpha, pq[j], kq * u);
      const int64_t oi = pair * DV + r;
      if constexpr (BF16)
        reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(out)[oi] = o;
    }
  }
}

// The same row split applied to every token of a request in turn (the recurrence itself,
// with no chunks): the state rows stay in registers from the request's first token to its
// last, so the state is read and written once per call whatever the number of tokens.
// For short requests (speculative-decoding verification, a few tokens each) this replaces
// the chunked path, whose 64-row chunks would be mostly padding; it is correct for any
// length but runs each request's tokens one after another.
template <int DK, bool BF16>
__global__ __launch_bounds__(kDecodeThreads) void recurrent_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ ga, const float* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int64_t* __restrict__ cache_indices,
    const int64_t* __restrict__ cu, int H, int HV, int DV, int nrb, int64_t max_len,
    float* __restrict__ state_pool, void* __restrict__ out) {
  constexpr int LPR = DK / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int NR = kRowsPerThread<DK>;
  constexpr int RWV = RPW * NR;
  constexpr int RWG = kRowsPerBlock<DK>;
  const uint32_t x = blockIdx.x;
  const uint32_t pair32 = x / (uint32_t)nrb;
  const int rb = (int)(x - pair32 * (uint32_t)nrb);
  const uint32_t b32 = pair32 / (uint32_t)HV;
  const int hv = (int)(pair32 - b32 * (uint32_t)HV);
  const int h = hv / (HV / H);
  const int64_t bi = b32;
  const int64_t t_begin = cu[bi], t_end = cu[bi + 1];
  if (t_begin >= t_end) return;  // an empty request leaves its slot untouched
  if (t_end - t_begin > max_len) return;  // left to the chunked kernels
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int gl = l % LPR, rg = l / LPR;
  const int64_t slot = cache_indices[bi];
  const float alog = A_log[hv], dtb = dt_bias[hv];
  const float decay = expf(alog);

  const int r0 = rb * RWG + wv * RWV + rg;
  float* Sp = state_pool + ((slot * HV + hv) * (int64_t)DV + r0) * DK + 4 * gl;
  f32x4 s[NR][2];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    s[j][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + j * RPW * DK));
    s[j][1] =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + j * RPW * DK + DK / 2));
  }

  // One token's inputs; the next token's are loaded while the current one is applied
  // (the last token loads itself again, so every load stays in the request).
  struct TokenIn {
    float vr[NR], kk[8], qq[8], a_t, b_t;
  };
  auto load_token = [&](int64_t t, TokenIn& x) {
    const int64_t th = t * HV + hv;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int64_t vi = th * DV + r0 + j * RPW;
      x.vr[j] = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(v)[vi])
                     : reinterpret_cast<const float*>(v)[vi];
    }
    load8<DK, BF16>(k, (t * H + h) * DK, gl, x.kk);
    load8<DK, BF16>(q, (t * H + h) * DK, gl, x.qq);
    x.a_t = ga[th];
    x.b_t = gb[th];
  };
  TokenIn nxt;
  load_token(t_begin, nxt);
  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t th = t * HV + hv;
    const TokenIn cur = nxt;
    load_token(t + 1 < t_end ? t + 1 : t, nxt);
    float vr[NR], kk[8], qq[8];
#pragma unroll
    for (int j = 0; j < NR; ++j) vr[j] = cur.vr[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kk[e] = cur.kk[e];
      qq[e] = cur.qq[e];
    }
    const float a_t = cur.a_t, b_t = cur.b_t;
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssk = __builtin_fmaf(kk[e], kk[e], ssk);
      ssq = __builtin_fmaf(qq[e], qq[e], ssq);
    }
    ssk = group_sum<LPR>(ssk);
    ssq = group_sum<LPR>(ssq);
    const float rk = 1.0f / sqrtf(ssk + kNormEps), rq = 1.0f / sqrtf(ssq + kNormEps);
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kk[e] *= rk;
      qq[e] *= rq;
      kq = __builtin_fmaf(kk[e], qq[e], kq);
    }
    kq = group_sum<LPR>(kq);
    const float xg = a_t + dtb;
    const float sp = fmaxf(xg, 0.f) + log1pf(expf(-fabsf(xg)));
    const float alpha = expf(-decay * sp);
    const float beta = 1.f / (1.f + expf(-b_t));

    float pk[NR], pq[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0 = __builtin_fmaf(s[j][0][e], kk[e], a0);
        a0 = __builtin_fmaf(s[j][1][e], kk[4 + e], a0);
        a1 = __builtin_fmaf(s[j][0][e], qq[e], a1);
        a1 = __builtin_fmaf(s[j][1][e], qq[4 + e], a1);
      }
      pk[j] = group_sum<LPR>(a0);
      pq[j] = group_sum<LPR>(a1);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const float u = beta * (vr[j] - alpha * pk[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[j][0][e] = __builtin_fmaf(alpha, s[j][0][e], u * kk[e]);
        s[j][1][e] = __builtin_fmaf(alpha, s[j][1][e], u * kk[4 + e]);
      }
      if (gl == 0) {
        const float o = __builtin_fmaf(alpha, pq[j], kq * u);
        const int64_t oi = th * DV + r0 + j * RPW;
        if constexpr (BF16)
          reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16(o);
        else
          reinterpret_cast<float*>(out)[oi] = o;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    __builtin_nontemporal_store(s[j][0], reinterpret_cast<f32x4*>(Sp + j * RPW * DK));
    __builtin_nontemporal_store(s[j][1], reinterpret_cast<f32x4*>(Sp + j * RPW * DK + DK / 2));
  }
}

template <int DK, bool BF16>
hipError_t launch_recurrent_t(const void* q, const void* k, const void* v, const float* a,
                              const float* b, const float* A_log, const float* dt_bias,
                              const int64_t* idx, const int64_t* cu, const Shape& s,
                              int64_t max_len, float* pool, void* out, hipStream_t st) {
  if (s.dv % kRowsPerBlock<DK> != 0) return hipErrorInvalidValue;
  const int nrb = s.dv / kRowsPerBlock<DK>;
  const int64_t blocks = s.B * (int64_t)s.HV * nrb;
  hipLaunchKernelGGL((recurrent_kernel<DK, BF16>), dim3((unsigned)blocks), dim3(kDecodeThreads),
                     0, st, q, k, v, a, b, A_log, dt_bias, idx, cu, s.H, s.HV, s.dv, nrb, max_len,
                     pool, out);
  return hipGetLastError();
}

template <int DK, bool BF16>
hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* a,
                           const float* b, const float* A_log, const float* dt_bias,
                           const int64_t* idx, const Shape& s, float* pool, void* out,
                           hipStream_t st) {
  if (s.dv % kRowsPerBlock<DK> != 0) return hipErrorInvalidValue;
  const int nrb = s.dv / kRowsPerBlock<DK>;
  const int64_t blocks = s.B * (int64_t)s.HV * nrb;
  hipLaunchKernelGGL((decode_kernel<DK, BF16>), dim3((unsigned)blocks), dim3(kDecodeThreads), 0,
                     st, q, k, v, a, b, A_log, dt_bias, idx, s.H, s.HV, s.dv, nrb, pool, out);
  return hipGetLastError();
}

}  // namespace

int64_t decode_blocks(const Shape& s) {
  const int rwg = s.dk == 64 ? kRowsPerBlock<64> : s.dk == 128 ? kRowsPerBlock<128>
                                                                : kRowsPerBlock<256>;
  return s.B * (int64_t)s.HV * ((s.dv + rwg - 1) / rwg);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* A_log, const float* dt_bias,
                         const int64_t* cache_indices, const Shape& s, float* state_pool,
                         void* out, hipStream_t st) {
#define GDN_DECODE_CASE(DKv)                                                                    \
  if (s.dk == DKv)                                                                              \
    return s.bf16 ? launch_decode_t<DKv, true>(q, k, v, a, b, A_log, dt_bias, cache_indices, s, \
                                               state_pool, out, st)                             \
                  : launch_decode_t<DKv, false>(q, k, v, a, b, A_log, dt_bias, cache_indices,  \
                                                s, state_pool, out, st);
  GDN_DECODE_CASE(64)
  GDN_DECODE_CASE(128)
  GDN_DECODE_CASE(256)
#undef GDN_DECODE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_recurrent(const void* q, const void* k, const void* v, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            const int64_t* cache_indices, const int64_t* cu_seqlens,
                            const Shape& s, int64_t max_len, float* state_pool, void* out,
                            hipStream_t st) {
#define GDN_RECURRENT_CASE(DKv)                                                              \
  if (s.dk == DKv)                                                                           \
    return s.bf16 ? launch_recurrent_t<DKv, true>(q, k, v, a, b, A_log, dt_bias,             \
                                                  cache_indices, cu_seqlens, s, max_len,     \
                                                  state_pool, out, st)                       \
                  : launch_recurrent_t<DKv, false>(q, k, v, a, b, A_log, dt_bias,            \
                                                   cache_indices, cu_seqlens, s, max_len,    \
                                                   state_pool, out, st);
  GDN_RECURRENT_CASE(64)
  GDN_RECURRENT_CASE(128)
  GDN_RECURRENT_CASE(256)
#undef GDN_RECURRENT_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
