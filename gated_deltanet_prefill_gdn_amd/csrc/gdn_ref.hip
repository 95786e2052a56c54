// Chunkwise GDN forward in plain fp32 arithmetic (no matrix cores).
//
// This family serves fp32 inputs, where every operand must stay in fp32. It
// computes, per chunk of n <= C rows (row convention: S is dv x dk, K and Q are
// n x dk, V is n x dv; G is the chunk-local inclusive log cumulative gate):
//   A   = tril(diag(beta) Kh Kh^T, -1)            Kh = diag(r_k) K, r_k = 1/|k|
//   T   = (I + A)^-1                               the one inverse, M^-1
//   W<- = diag(e^G) T diag(beta) Kh                W up to the decay (veitner page,
//                                                  Reminder, equation for W)
//   U~  = (Gamma o T) diag(beta) V,  Gamma_ri = exp(G_r - G_i) for i <= r
//         This is N^-1 B V with N^-1 = G M^-1 G^-1 (veitner page, Save one invert),
//         applied entry by entry so no 1/gamma is formed.
// and then, sequentially over the chunks of a request (pymllm gdn_chunkwise page,
// Algorithm, steps 2 and 3, in row convention):
//   U     = U~ - W<- S^T
//   O     = diag(e^G) Qh S^T + (Gamma o tril0(Qh Kh^T)) U
//   S_new = e^{G_n} S + U^T diag(e^{G_n - G}) Kh
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = 64;

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<__hip_bfloat16>(const __hip_bfloat16* p, int64_t i) {
  return __bfloat162float(p[i]);
}
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(__hip_bfloat16* p, int64_t i, float x) {
  p[i] = __float2bfloat16(x);  // round to nearest even
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Inverse L2 norms of rows [0, n) of a chunk: s_r[r] = 1 / sqrt(|x_r|^2 + eps).
template <typename Tin>
__device__ void row_inv_norms(const Tin* x, int64_t t0, int n, int heads, int h, int d,
                              float* s_r) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = wave; r < C; r += 4) {
    float acc = 0.f;
    if (r < n) {
      const int64_t base = ((t0 + r) * heads + h) * (int64_t)d;
      for (int j = lane; j < d; j += 64) {
        const float e = ld(x, base + j);
        acc += e * e;
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) s_r[r] = r < n ? (float)(1.0 / sqrt((double)acc + (double)kNormEps)) : 0.f;
  }
}

// One workgroup per (global chunk, value head).
template <typename Tin>
__global__ __launch_bounds__(256) void ref_prep_kernel(
    const Tin* __restrict__ k, const Tin* __restrict__ v, const int64_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_seq,
    const double* __restrict__ gcum, const float* __restrict__ beta, int H, int HV, int dk,
    int dv, float* __restrict__ W, float* __restrict__ U) {
  __shared__ float s_rk[C], s_bt[C];
  __shared__ double s_G[C];
  __shared__ float s_A[C][C + 1];
  __shared__ float s_T[C][C + 1];
  const int64_t c = blockIdx.x;
  const int hv = blockIdx.y;
  const int32_t seq = chunk_seq[c];
  if (seq < 0) return;
  const int h = hv / (HV / H);
  const int64_t t0 = cu[seq] + (int64_t)(c - chunk_off[seq]) * C;
  const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
  const int64_t pair = c * HV + hv;
  const int tid = threadIdx.x;
  if (tid < C) {
    s_G[tid] = gcum[pair * C + tid];
    s_bt[tid] = beta[pair * C + tid];
  }
  row_inv_norms(k, t0, n, H, h, dk, s_rk);
  __syncthreads();
  // A = tril(diag(beta) Kh Kh^T, -1)
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    float val = 0.f;
    if (i < r && r < n) {
      const int64_t br = ((t0 + r) * H + h) * (int64_t)dk, bi = ((t0 + i) * H + h) * (int64_t)dk;
      float acc = 0.f;
      for (int j = 0; j < dk; ++j) acc += ld(k, br + j) * ld(k, bi + j);
      val = s_bt[r] * s_rk[r] * s_rk[i] * acc;
    }
    s_A[r][i] = val;
  }
  __syncthreads();
  // T = (I + A)^-1 by forward substitution; thread `col` owns column col, so the
  // column it reads back is the one it wrote.
  if (tid < C) {
    const int col = tid;
    for (int r = 0; r < C; ++r) {
      float val;
      if (r < col) {
        val = 0.f;
      } else if (r == col) {
        val = 1.f;
      } else {
        float acc = 0.f;
        for (int i = col; i < r; ++i) acc += s_A[r][i] * s_T[i][col];
        val = -acc;
      }
      s_T[r][col] = val;
    }
  }
  __syncthreads();
  // W<- = diag(e^G) T diag(beta r_k) K
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    s_A[r][i] = (i <= r && r < n) ? expf((float)s_G[r]) * s_T[r][i] * s_bt[i] * s_rk[i] : 0.f;
  }
  __syncthreads();
  float* Wp = W + pair * C * (int64_t)dk;
  for (int idx = tid; idx < C * dk; idx += 256) {
    const int r = idx / dk, j = idx % dk;
    float acc = 0.f;
    for (int i = 0; i <= r && i < n; ++i) acc += s_A[r][i] * ld(k, ((t0 + i) * H + h) * (int64_t)dk + j);
    Wp[idx] = acc;
  }
  __syncthreads();
  // U~ = (Gamma o T) diag(beta) V
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    s_A[r][i] = (i <= r && r < n) ? expf((float)(s_G[r] - s_G[i])) * s_T[r][i] * s_bt[i] : 0.f;
  }
  __syncthreads();
  float* Up = U + pair * C * (int64_t)dv;
  for (int idx = tid; idx < C * dv; idx += 256) {
    const int r = idx / dv, j = idx % dv;
    float acc = 0.f;
    for (int i = 0; i <= r && i < n; ++i) acc += s_A[r][i] * ld(v, ((t0 + i) * HV + hv) * (int64_t)dv + j);
    Up[idx] = acc;
  }
}

constexpr int kBV = 16;      // state rows (dv index) per workgroup
constexpr int kMaxDk = 256;

// One workgroup per (request, value head, block of kBV state rows); walks the
// request's chunks in order with its rows of S resident in LDS.
template <typename Tin>
__global__ __launch_bounds__(256) void ref_state_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const int64_t* __restrict__ cu,
    const int64_t* __restrict__ cache_indices, const int32_t* __restrict__ chunk_off,
    const double* __restrict__ gcum, const float* __restrict__ W, const float* __restrict__ U,
    int H, int HV, int dk, int dv, int64_t short_len, float* __restrict__ state_pool,
    Tin* __restrict__ out, int32_t* __restrict__ nonfinite) {
  __shared__ float s_S[kBV][kMaxDk + 1];
  __shared__ float s_U[C][kBV + 1];
  __shared__ float s_Aqk[C][C + 1];
  __shared__ float s_rq[C], s_rk[C], s_kd[C], s_eg[C];
  __shared__ double s_G[C];
  const int seq = blockIdx.x, hv = blockIdx.y, v0 = blockIdx.z * kBV;
  const int64_t L = cu[seq + 1] - cu[seq];
  const int64_t nchunks = path_chunks(L, C, short_len);
  if (nchunks == 0) return;  // empty (slot untouched) or evaluated by the token recurrence
  const int64_t slot = cache_indices[seq];
  const int h = hv / (HV / H);
  const int tid = threadIdx.x;
  float* Sg = state_pool + ((slot * HV + hv) * (int64_t)dv + v0) * dk;
  for (int idx = tid; idx < kBV * dk; idx += 256) s_S[idx / dk][idx % dk] = Sg[idx];
  for (int64_t cl = 0; cl < nchunks; ++cl) {
    const int64_t c = chunk_off[seq] + cl;
    const int64_t t0 = cu[seq] + cl * C;
    const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
    const int64_t pair = c * HV + hv;
    __syncthreads();  // previous chunk's S update is complete
    if (tid < C) s_G[tid] = gcum[pair * C + tid];
    row_inv_norms(q, t0, n, H, h, dk, s_rq);
    row_inv_norms(k, t0, n, H, h, dk, s_rk);
    __syncthreads();
    if (tid < C) {
      const double Gn = s_G[n - 1];
      s_eg[tid] = tid < n ? expf((float)s_G[tid]) : 0.f;
      s_kd[tid] = tid < n ? expf((float)(Gn - s_G[tid])) * s_rk[tid] : 0.f;
    }
    // A_qk = Gamma o tril0(Qh Kh^T)
    for (int idx = tid; idx < C * C; idx += 256) {
      const int r = idx / C, i = idx % C;
      float val = 0.f;
      if (i <= r && r < n) {
        const int64_t br = ((t0 + r) * H + h) * (int64_t)dk, bi = ((t0 + i) * H + h) * (int64_t)dk;
        float acc = 0.f;
        for (int j = 0; j < dk; ++j) acc += ld(q, br + j) * ld(k, bi + j);
        val = expf((float)(s_G[r] - s_G[i])) * s_rq[r] * s_rk[i] * acc;
      }
      s_Aqk[r][i] = val;
    }
    // U = U~ - W<- S^T (rows of this block only)
    const float* Wp = W + pair * C * (int64_t)dk;
    const float* Up = U + pair * C * (int64_t)dv;
    for (int idx = tid; idx < C * kBV; idx += 256) {
      const int r = idx / kBV, cc = idx % kBV;
      float val = 0.f;
      if (r < n) {
        float acc = 0.f;
        for (int j = 0; j < dk; ++j) acc += Wp[r * (int64_t)dk + j] * s_S[cc][j];
        val = Up[r * (int64_t)dv + v0 + cc] - acc;
      }
      s_U[r][cc] = val;
    }
    __syncthreads();
    // O = diag(e^G r_q) Q S^T + A_qk U
    for (int idx = tid; idx < C * kBV; idx += 256) {
      const int r = idx / kBV, cc = idx % kBV;
      if (r < n) {
        const int64_t br = ((t0 + r) * H + h) * (int64_t)dk;
        float acc = 0.f;
        for (int j = 0; j < dk; ++j) acc += ld(q, br + j) * s_S[cc][j];
        float o = s_eg[r] * s_rq[r] * acc;
        for (int i = 0; i <= r; ++i) o += s_Aqk[r][i] * s_U[i][cc];
        st(out, ((t0 + r) * HV + hv) * (int64_t)dv + v0 + cc, o);
      }
    }
    __syncthreads();
    // S <- e^{G_n} S + U^T diag(e^{G_n - G} r_k) K
    const float egn = expf((float)s_G[n - 1]);
    for (int idx = tid; idx < kBV * dk; idx += 256) {
      const int cc = idx / dk, j = idx % dk;
      float acc = 0.f;
      for (int r = 0; r < n; ++r) acc += s_U[r][cc] * s_kd[r] * ld(k, ((t0 + r) * H + h) * (int64_t)dk + j);
      s_S[cc][j] = egn * s_S[cc][j] + acc;
    }
  }
  __syncthreads();
  bool finite = true;
  for (int idx = tid; idx < kBV * dk; idx += 256) {
    const float x = s_S[idx / dk][idx % dk];
    Sg[idx] = x;
    finite = finite && __builtin_isfinite(x);
  }
  if (!finite) *nonfinite = 1;
}

}  // namespace

hipError_t launch_ref_prep(const void* k, const void* v, const int64_t* cu_seqlens,
                           const int32_t* chunk_off, const int32_t* chunk_seq, const double* gcum,
                           const float* beta, const Shape& s, int64_t max_chunks, float* w,
                           float* u, hipStream_t st) {
  const dim3 grid((unsigned)max_chunks, (unsigned)s.HV);
  if (s.bf16) {
    hipLaunchKernelGGL(ref_prep_kernel<__hip_bfloat16>, grid, dim3(256), 0, st,
                       (const __hip_bfloat16*)k, (const __hip_bfloat16*)v, cu_seqlens, chunk_off,
                       chunk_seq, gcum, beta, s.H, s.HV, s.dk, s.dv, w, u);
  } else {
    hipLaunchKernelGGL(ref_prep_kernel<float>, grid, dim3(256), 0, st, (const float*)k,
                       (const float*)v, cu_seqlens, chunk_off, chunk_seq, gcum, beta, s.H, s.HV,
                       s.dk, s.dv, w, u);
  }
  return hipGetLastError();
}

hipError_t launch_ref_state(const void* q, const void* k, const int64_t* cu_seqlens,
                            const int64_t* cache_indices, const int32_t* chunk_off,
                            const double* gcum, const float* w, const float* u, const Shape& s,
                            float* state_pool, void* out, int32_t* nonfinite, hipStream_t st) {
  const dim3 grid((unsigned)s.B, (unsigned)s.HV, (unsigned)(s.dv / kBV));
  if (s.bf16) {
    hipLaunchKernelGGL(ref_state_kernel<__hip_bfloat16>, grid, dim3(256), 0, st,
                       (const __hip_bfloat16*)q, (const __hip_bfloat16*)k, cu_seqlens,
                       cache_indices, chunk_off, gcum, w, u, s.H, s.HV, s.dk, s.dv, s.short_len,
                       state_pool, (__hip_bfloat16*)out, nonfinite);
  } else {
    hipLaunchKernelGGL(ref_state_kernel<float>, grid, dim3(256), 0, st, (const float*)q,
                       (const float*)k, cu_seqlens, cache_indices, chunk_off, gcum, w, u, s.H,
                       s.HV, s.dk, s.dv, s.short_len, state_pool, (float*)out, nonfinite);
  }
  return hipGetLastError();
}

}  // namespace gdn
