// Varlen chunk table and the gate / log-space cumulative-decay kernel.
//
// Chunks of C tokens restart at every request (a request's last chunk may be
// partial). The gate of token t at value head hv is
//   g_t = log(alpha_t) = -exp(A_log[hv]) * softplus(a[t,hv] + dt_bias[hv]),
//   beta_t = sigmoid(b[t,hv])
// (pymllm gdn_chunkwise page, Module Contents: a and b are the raw gate inputs
// before softplus/exp and sigmoid). The cumulative gate of "Simple math to speed
// up GDN prefill" (veitner), section Reminder, gamma^r = prod_{j<=r} alpha^j, is
// kept in log space: G_r = sum_{j<=r} g_j, chunk-local and inclusive, summed in
// fp64 so that differences G_r - G_i keep their relative accuracy even when G
// reaches hundreds inside a chunk. Padding rows of a partial chunk get g = 0
// (alpha = 1) and beta = 0, so G stays at the last real token's value.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanLds = 4096;  // chunk_off entries kept in LDS for the request search

// One workgroup: chunk_off[b] = sum_{b' < b} ceil(L_b' / C), chunk_off[B] = total,
// then chunk_seq[c] = the request that owns global chunk c (or -1 past the total).
// The scan runs per wavefront with shuffles, then across the 16 wavefronts; the search
// for each chunk's request reads an LDS copy of chunk_off when it fits.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int64_t* __restrict__ cu,
                                                            int64_t B, int C,
                                                            int64_t short_len,
                                                            int32_t* __restrict__ chunk_off,
                                                            int32_t* __restrict__ chunk_seq,
                                                            int64_t max_chunks) {
  constexpr int NW = kPlanThreads / 64;
  __shared__ int32_t s_wsum[NW];
  __shared__ int32_t s_off[kPlanLds];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool in_lds = B + 1 <= kPlanLds;
  int32_t carry = 0;
  for (int64_t base = 0; base < B; base += kPlanThreads) {
    const int64_t bi = base + tid;
    int32_t n = 0;
    if (bi < B) {
      const int64_t L = cu[bi + 1] - cu[bi];
      n = (int32_t)path_chunks(L, C, short_len);
    }
    int32_t x = n;  // inclusive scan within the wavefront
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wv] = x;
    __syncthreads();
    if (wv == 0) {  // inclusive scan of the wavefront totals
      int32_t ws = lane < NW ? s_wsum[lane] : 0;
      for (int off = 1; off < NW; off <<= 1) {
        const int32_t y = __shfl_up(ws, off, 64);
        if (lane >= off) ws += y;
      }
      if (lane < NW) s_wsum[lane] = ws;
    }
    __syncthreads();
    const int32_t excl = carry + (wv > 0 ? s_wsum[wv - 1] : 0) + x - n;
    if (bi < B) {
      chunk_off[bi] = excl;
      if (in_lds) s_off[bi] = excl;
    }
    carry += s_wsum[NW - 1];
    __syncthreads();  // s_wsum is rewritten by the next block of requests
  }
  const int32_t total = carry;
  if (tid == 0) {
    chunk_off[B] = total;
    if (in_lds) s_off[B] = total;
  }
  __threadfence_block();
  __syncthreads();
  for (int64_t c = tid; c < max_chunks; c += kPlanThreads) {
    int32_t seq = -1;
    if (c < total) {
      int64_t lo = 0, hi = B;  // chunk_off[lo] <= c < chunk_off[hi]
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        const int32_t om = in_lds ? s_off[mid] : chunk_off[mid];
        if (om <= c) lo = mid; else hi = mid;
      }
      seq = (int32_t)lo;
    }
    chunk_seq[c] = seq;
  }
}

// One wavefront per (global chunk, value head); lane r is row r of the chunk (C == 64).
__global__ __launch_bounds__(256) void gate_kernel(
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int64_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_seq, int HV,
    int64_t max_chunks, double* __restrict__ gcum, float* __restrict__ beta,
    int32_t* __restrict__ nonfinite) {
  constexpr int C = 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) *nonfinite = 0;  // the state pass raises it
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= max_chunks * HV) return;
  const int64_t c = pair / HV;
  const int hv = (int)(pair - c * HV);
  const int32_t seq = chunk_seq[c];
  if (seq < 0) return;  // unused chunk slot: never read downstream
  const int64_t t0 = cu[seq] + (int64_t)(c - chunk_off[seq]) * C;
  const int64_t n = min((int64_t)C, cu[seq + 1] - t0);
  float g = 0.f, bt = 0.f;
  if (lane < n) {
    const int64_t t = t0 + lane;
    const float x = a[t * HV + hv] + dt_bias[hv];
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    g = -expf(A_log[hv]) * sp;
    bt = 1.f / (1.f + expf(-b[t * HV + hv]));
  }
  double s = (double)g;
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(s, off, 64);
    if (lane >= off) s += y;
  }
  gcum[pair * C + lane] = s;
  beta[pair * C + lane] = bt;
}

}  // namespace

hipError_t launch_plan(const int64_t* cu_seqlens, const Shape& s, int32_t* chunk_off,
                       int32_t* chunk_seq, int64_t max_chunks, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, cu_seqlens, s.B, s.C,
                     s.short_len, chunk_off, chunk_seq, max_chunks);
  return hipGetLastError();
}

hipError_t launch_gate(const float* a, const float* b, const float* A_log, const float* dt_bias,
                       const int64_t* cu_seqlens, const int32_t* chunk_off,
                       const int32_t* chunk_seq, const Shape& s, int64_t max_chunks,
                       double* gcum, float* beta, int32_t* nonfinite, hipStream_t st) {
  const int64_t pairs = max_chunks * s.HV;
  const int64_t blocks = (pairs + 3) / 4;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, b, A_log, dt_bias,
                     cu_seqlens, chunk_off, chunk_seq, s.HV, max_chunks, gcum, beta, nonfinite);
  return hipGetLastError();
}

}  // namespace gdn
