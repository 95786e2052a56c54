// Sequential state pass on matrix cores (bf16 inputs).
//
// One workgroup (4 wavefronts) per (request, value head, block of 16 state rows);
// the block's rows of S stay resident as fp32 matrix-core accumulators for the
// whole request. Per chunk, in row convention (pymllm gdn_chunkwise page,
// Algorithm steps 2-3; "Simple math to speed up GDN prefill", Reminder,
// chunkwise transition with decorated S->, W<-, K->):
//   U     = U~ - W<- S^T                                  (n x 16)
//   O     = diag(e^G) Qh S^T + (Gamma o tril0(Qh Kh^T)) U  (written to out)
//   S^T  <- e^{G_n} S^T + Kh^T diag(e^{G_n - G}) U
// with Qh, Kh the L2-normalised rows and Gamma_ri = e^{G_r - G_i}. The inter-chunk
// loop is sequential (pymllm page: the propagation between chunks remains
// sequential over ceil(T/C) steps).
//
// Work split: wave w computes the rows 16w..16w+15 of P = W<- S^T, U and O, and owns
// the 32-wide dk steps w, w+4, ... of S^T for the update. S^T (fp16) and U (fp16)
// cross waves through LDS once per chunk. Matrix-core operands: Qh, Kh, W<-, U~, U
// and S in fp16 with fp32 accumulation; Qh Kh^T on the raw bf16 values (exact
// products), scaled afterwards.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;
constexpr int SA = C + 16;  // row stride of the A_qk tile (fp16)

template <int DK>
struct StateSmem {
  static constexpr int SK = DK + 16;
  uint16_t k[C * SK];          // raw bf16 k rows of the chunk
  half8 S[DK / 32][64];        // S^T B-fragments, one per 32-wide dk step
  half4 U[4][64];              // U tiles (D layout)
  half4 Uk[4][64];             // diag(e^{G_n - G}) U tiles
  uint16_t Aqk[C * SA];        // Gamma o tril0(Qh Kh^T), fp16 bits
  float rk[C], rq[C], eg[C], kd[C];
  double G[C];
};

__device__ __forceinline__ u32x2 ld_u32x2(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ u32x4 row_frag(const uint16_t* base, int stride, int row, int col0,
                                          int g) {
  const uint16_t* p = base + row * stride + col0 + 4 * g;
  const u32x2 lo = ld_u32x2(p), hi = ld_u32x2(p + 16);
  u32x4 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

template <int DK>
__global__ __launch_bounds__(256) void mfma_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const double* __restrict__ gcum,
    const _Float16* __restrict__ W, const _Float16* __restrict__ Ut, int B, int H, int HV,
    int DV, float* __restrict__ state_pool, uint16_t* __restrict__ out) {
  using Sm = StateSmem<DK>;
  constexpr int SK = Sm::SK;
  constexpr int NKS = DK / 32;             // 32-wide dk steps
  constexpr int NOWN = (NKS + 3) / 4;      // dk steps owned per wave (upper bound)
  constexpr int KP = C * DK / 8 / 256;     // 16-byte pieces of the k tile per thread
  __shared__ Sm sm;

  // Blocks of the same (request, head) share blockIdx.x mod 8, so they run on one
  // XCD and re-read q, k and W<- from its L2.
  const int nvb = DV / 16;
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int vb = (int)(rest % nvb);
  const int64_t p = (rest / nvb) * 8 + (x & 7);
  if (p >= (int64_t)B * HV) return;
  const int seq = (int)(p / HV), hv = (int)(p % HV);
  const int64_t L = cu[seq + 1] - cu[seq];
  if (L <= 0) return;
  const int h = hv / (HV / H);
  const int v0 = 16 * vb;
  const int64_t slot = cache_indices[seq];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int64_t nch = (L + C - 1) / C;
  const int64_t cbase = chunk_off[seq];

  // ---- resident state: S^T tiles of the owned dk steps
  float* Sg = state_pool + ((slot * HV + hv) * (int64_t)DV + v0 + m) * DK;
  f32x4 Sacc[NOWN][2];
#pragma unroll
  for (int i = 0; i < NOWN; ++i) {
    const int sp = w + 4 * i;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (sp < NKS) z = *reinterpret_cast<const f32x4*>(Sg + 32 * sp + 16 * tt + 4 * g);
      Sacc[i][tt] = z;
    }
    if (sp < NKS) sm.S[sp][l] = cat(to_half4(Sacc[i][0]), to_half4(Sacc[i][1]));
  }

  // ---- prefetch registers for one chunk
  u32x4 kreg[KP], qreg[NKS], wreg[NKS];
  u32x2 ureg;
  double greg = 0.0;
  auto load_chunk = [&](int64_t cl) {
    const int64_t cg = cbase + cl;
    const int64_t t0 = cu[seq] + cl * C;
    const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
    const int64_t pr = cg * HV + hv;
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int e = tid + 256 * u, row = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (row < n) z = *reinterpret_cast<const u32x4*>(k + ((t0 + row) * H + h) * (int64_t)DK + c8);
      kreg[u] = z;
    }
    const int qrow = 16 * w + m;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qrow < n) {
        const uint16_t* pq = q + ((t0 + qrow) * H + h) * (int64_t)DK + 32 * s + 4 * g;
        const u32x2 a = ld_u32x2(pq), b2 = ld_u32x2(pq + 16);
        z[0] = a[0]; z[1] = a[1]; z[2] = b2[0]; z[3] = b2[1];
      }
      qreg[s] = z;
      wreg[s] = *reinterpret_cast<const u32x4*>(W + pr * C * DK + ((w * NKS + s) * 64 + l) * 8);
    }
    ureg = *reinterpret_cast<const u32x2*>(Ut + pr * C * DV + ((vb * 4 + w) * 64 + l) * 4);
    if (tid < C) greg = gcum[pr * C + tid];
  };
  load_chunk(0);
  __syncthreads();  // initial S fragments visible

  for (int64_t cl = 0; cl < nch; ++cl) {
    const int64_t t0 = cu[seq] + cl * C;
    const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
    // 1. stage the k tile and the gates; keep this chunk's fragments
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int e = tid + 256 * u, row = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[row * SK + c8]) = kreg[u];
    }
    if (tid < C) {
      sm.G[tid] = greg;
      sm.eg[tid] = expf((float)greg);
    }
    u32x4 qc[NKS], wc[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qc[s] = qreg[s];
      wc[s] = wreg[s];
    }
    const u32x2 uc = ureg;
    if (cl + 1 < nch) load_chunk(cl + 1);
    __syncthreads();  // (A)

    // 2. norms: r_k for rows 16w.. from LDS; r_q of this lane's row from its fragments
    {
      const int row = 16 * w + m;
      float acc = 0.f;
#pragma unroll
      for (int cc = g * (DK / 4); cc < (g + 1) * (DK / 4); cc += 8) {
        const u32x4 xk = *reinterpret_cast<const u32x4*>(&sm.k[row * SK + cc]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += bf_lo(xk[j]) * bf_lo(xk[j]) + bf_hi(xk[j]) * bf_hi(xk[j]);
      }
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      if (g == 0) sm.rk[row] = 1.0f / sqrtf(acc + kNormEps);
    }
    float rq_lane;
    {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc += bf_lo(qc[s][j]) * bf_lo(qc[s][j]) + bf_hi(qc[s][j]) * bf_hi(qc[s][j]);
      acc += __shfl_xor(acc, 16, 64);
      acc += __shfl_xor(acc, 32, 64);
      rq_lane = 1.0f / sqrtf(acc + kNormEps);
      if (g == 0) sm.rq[16 * w + m] = rq_lane;
    }
    if (tid < C) sm.kd[tid] = expf((float)(sm.G[C - 1] - sm.G[tid]));
    __syncthreads();  // (B)

    // 3. A_qk rows 16w..16w+15 = Gamma o tril0(Qh Kh^T), from raw bf16 q, k
    {
      const int jmax = w | 1;  // token tiles read by the A_qk U product of this row tile
      for (int J = 0; J <= jmax; ++J) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (J <= w) {
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            acc = mma_bf16(bf16x8_from_u32x4(qc[s]),
                           bf16x8_from_u32x4(row_frag(sm.k, SK, 16 * J + m, 32 * s, g)), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * g + i, cc = 16 * J + m;
          float val = 0.f;
          if (cc <= r)
            val = expf((float)(sm.G[r] - sm.G[cc])) * sm.rq[r] * sm.rk[cc] * acc[i];
          sm.Aqk[r * SA + cc] = __builtin_bit_cast(uint16_t, (_Float16)val);
        }
      }
    }

    // 4. P = W<- S^T and Qh S^T for rows 16w..; U = U~ - P
    f32x4 P = {0.f, 0.f, 0.f, 0.f}, O1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const half8 sf = sm.S[s][l];
      P = mma_f16(half8_from_u32x4(wc[s]), sf, P);
      half8 qh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qh[2 * j] = (_Float16)(bf_lo(qc[s][j]) * rq_lane);
        qh[2 * j + 1] = (_Float16)(bf_hi(qc[s][j]) * rq_lane);
      }
      O1 = mma_f16(qh, sf, O1);
    }
    const half4 ut = __builtin_bit_cast(half4, uc);
    f32x4 U;
#pragma unroll
    for (int i = 0; i < 4; ++i) U[i] = (float)ut[i] - P[i];
    sm.U[w][l] = to_half4(U);
    {
      f32x4 Uk;
#pragma unroll
      for (int i = 0; i < 4; ++i) Uk[i] = U[i] * sm.kd[16 * w + 4 * g + i];
      sm.Uk[w][l] = to_half4(Uk);
    }
    __syncthreads();  // (C)

    // 5. O = diag(e^G) Qh S^T + A_qk U, rows 16w..16w+15
    {
      f32x4 AU = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s <= (w >> 1); ++s) {
        const half8 a = half8_from_u32x4(row_frag(sm.Aqk, SA, 16 * w + m, 32 * s, g));
        const half8 b = cat(sm.U[2 * s][l], sm.U[2 * s + 1][l]);
        AU = mma_f16(a, b, AU);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i;
        if (r < n) {
          const float o = sm.eg[r] * O1[i] + AU[i];
          out[((t0 + r) * HV + hv) * (int64_t)DV + v0 + m] = f32_to_bf16_bits(o);
        }
      }
    }
    // 6. S^T <- e^{G_n} S^T + Kh^T diag(e^{G_n - G}) U on the owned dk steps
    {
      float rkv[2][8];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) rkv[s][j] = sm.rk[32 * s + kperm(g, j)];
      half8 ub[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) ub[s] = cat(sm.Uk[2 * s][l], sm.Uk[2 * s + 1][l]);
      const float egn = sm.eg[C - 1];
#pragma unroll
      for (int i = 0; i < NOWN; ++i) {
        const int sp = w + 4 * i;
        if (sp < NKS) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = Sacc[i][tt] * egn;
            const int col = 32 * sp + 16 * tt + m;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              half8 a;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const uint16_t kb = sm.k[(32 * s + kperm(g, j)) * SK + col];
                a[j] = (_Float16)(bf16_bits_to_f32(kb) * rkv[s][j]);
              }
              acc = mma_f16(a, ub[s], acc);
            }
            Sacc[i][tt] = acc;
          }
          sm.S[sp][l] = cat(to_half4(Sacc[i][0]), to_half4(Sacc[i][1]));
        }
      }
    }
    __syncthreads();  // (D)
  }

  // ---- write the state back in place
#pragma unroll
  for (int i = 0; i < NOWN; ++i) {
    const int sp = w + 4 * i;
    if (sp < NKS) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        *reinterpret_cast<f32x4*>(Sg + 32 * sp + 16 * tt + 4 * g) = Sacc[i][tt];
    }
  }
}

template <int DK>
hipError_t launch_state_t(const void* q, const void* k, const int64_t* cu, const int64_t* idx,
                          const int32_t* off, const double* gcum, const _Float16* w,
                          const _Float16* u, const Shape& s, float* pool, void* out,
                          hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8;
  const int64_t blocks = pairs8 * 8 * (s.dv / 16);
  hipLaunchKernelGGL((mfma_state_kernel<DK>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, cu, idx, off, gcum, w, u, (int)s.B,
                     s.H, s.HV, s.dv, pool, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_state(const void* q, const void* k, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const double* gcum, const void* w, const void* u, const Shape& s,
                             float* state_pool, void* out, hipStream_t st) {
  const _Float16* W = (const _Float16*)w;
  const _Float16* U = (const _Float16*)u;
  switch (s.dk) {
    case 64: return launch_state_t<64>(q, k, cu_seqlens, cache_indices, chunk_off, gcum, W, U, s, state_pool, out, st);
    case 128: return launch_state_t<128>(q, k, cu_seqlens, cache_indices, chunk_off, gcum, W, U, s, state_pool, out, st);
    case 256: return launch_state_t<256>(q, k, cu_seqlens, cache_indices, chunk_off, gcum, W, U, s, state_pool, out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
