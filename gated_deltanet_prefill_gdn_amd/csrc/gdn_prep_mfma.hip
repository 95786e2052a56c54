// Chunk preparation on matrix cores (bf16 inputs): one workgroup per (chunk, value head).
//
// Row convention (S is dv x dk; K, V are the chunk's n <= 64 rows; G the chunk-local
// inclusive log cumulative gate; r_k = 1/|k|):
//   A   = tril(diag(beta r_k) K K^T diag(r_k), -1)          Gram of raw bf16 keys, exact
//                                                           products, fp32 accumulation
//   T   = (I + A)^-1                                        the single inverse, M^-1
//   W<- = diag(e^G) T diag(beta r_k) K                      ("Simple math to speed up GDN
//                                                           prefill", Reminder: W up to a
//                                                           decay factor, arrow decoration)
//   U~  = (Gamma o T) diag(beta) V,  Gamma_ri = e^{G_r - G_i}   the decayed inverse
//        N^-1 = G M^-1 G^-1 of the Save-one-invert section, taken entry by entry.
//   A_qk = Gamma o tril0(Qh Kh^T)                          the intra-chunk read mask of the
//        pymllm page's output step ("triu is the causal mask, j <= r"), Qh = diag(r_q) Q.
// The inverse is blocked in 16 x 16 tiles: diagonal tiles by forward substitution
// (one lane per column), off-diagonal tiles T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ on
// fp32 matrix cores. The factors T1 = diag(e^G) T diag(beta r_k) and
// T2 = (Gamma o T) diag(beta) are split into bf16 hi + lo, so the bf16 products
// with the exact raw K and V keep fp32 accuracy. W<- and U~ are stored as fp16 in
// the fragment layouts the state kernel reads directly into registers.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;

template <int DK, int DV>
struct PrepSmem {
  static constexpr int SK = (DK > DV ? DK : DV) + 16;  // row stride of the K/V staging tile
  static constexpr int ST = C + 16;                    // row stride of the T1/T2 bf16 tiles
  static constexpr int SQ = DK + 8;                    // row stride of the Q tile
  uint16_t kv[C * SK];                                 // K rows, later V rows (bf16 bits)
  uint16_t q[C * SQ];                                  // Q rows (bf16 bits)
  union {
    float A[C][C + 1];            // strictly lower Gram part (until T is complete)
    uint16_t Ts[2][C * ST];       // bf16 hi / lo of T1, later of T2
  } u;
  float T[C][C + 1];
  float rk[C], rq[C], bt[C], eg[C];
  double G[C];
};

__device__ __forceinline__ u32x2 lds_u32x2(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Fragment of a row-major bf16 tile: row `row`, 32-wide k step starting at col0,
// elements kperm(g, 0..7).
__device__ __forceinline__ u32x4 row_frag(const uint16_t* base, int stride, int row, int col0,
                                          int g) {
  const uint16_t* p = base + row * stride + col0 + 4 * g;
  const u32x2 lo = lds_u32x2(p), hi = lds_u32x2(p + 16);
  u32x4 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

// Fragment along the row index (a column of a row-major bf16 tile): column `col`,
// rows row0 + kperm(g, 0..7).
__device__ __forceinline__ u32x4 col_frag(const uint16_t* base, int stride, int col, int row0,
                                          int g) {
  uint16_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = base[(row0 + kperm(g, j)) * stride + col];
  u32x4 r;
  r[0] = e[0] | ((uint32_t)e[1] << 16);
  r[1] = e[2] | ((uint32_t)e[3] << 16);
  r[2] = e[4] | ((uint32_t)e[5] << 16);
  r[3] = e[6] | ((uint32_t)e[7] << 16);
  return r;
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void mfma_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ chunk_seq, const double* __restrict__ gcum,
    const float* __restrict__ beta, int H, int HV, _Float16* __restrict__ Wout,
    _Float16* __restrict__ Uout, float* __restrict__ kd_out, _Float16* __restrict__ Aout,
    float* __restrict__ erq_out) {
  using Sm = PrepSmem<DK, DV>;
  constexpr int SK = Sm::SK, ST = Sm::ST, SQ = Sm::SQ;
  __shared__ Sm sm;
  const int64_t c = blockIdx.x;
  const int hv = blockIdx.y;
  const int32_t seq = chunk_seq[c];
  if (seq < 0) return;
  const int h = hv / (HV / H);
  const int64_t t0 = cu[seq] + (int64_t)(c - chunk_off[seq]) * C;
  const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
  const int64_t pair = c * HV + hv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;

  // ---- stage K (LDS) and V (registers, written to LDS once K is no longer needed)
  constexpr int KP = C * DK / 8 / 256;  // 16-byte pieces per thread
  constexpr int VP = C * DV / 8 / 256;
  u32x4 vreg[VP];
#pragma unroll
  for (int u = 0; u < VP; ++u) {
    const int e = tid + 256 * u, row = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < n) x = *reinterpret_cast<const u32x4*>(v + ((t0 + row) * HV + hv) * (int64_t)DV + c8);
    vreg[u] = x;
  }
#pragma unroll
  for (int u = 0; u < KP; ++u) {
    const int e = tid + 256 * u, row = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    u32x4 y = {0u, 0u, 0u, 0u};
    if (row < n) {
      x = *reinterpret_cast<const u32x4*>(k + ((t0 + row) * H + h) * (int64_t)DK + c8);
      y = *reinterpret_cast<const u32x4*>(q + ((t0 + row) * H + h) * (int64_t)DK + c8);
    }
    *reinterpret_cast<u32x4*>(&sm.kv[row * SK + c8]) = x;
    *reinterpret_cast<u32x4*>(&sm.q[row * SQ + c8]) = y;
  }
  if (tid < C) {
    const double Gv = gcum[pair * C + tid];
    sm.G[tid] = Gv;
    sm.eg[tid] = expf((float)Gv);
    sm.bt[tid] = beta[pair * C + tid];
  }
  lds_barrier();

  // ---- r_k and r_q: wave w, rows 16w..16w+15; lane group g sums a quarter of a row
  {
    const int row = 16 * w + m;
    float acck = 0.f, accq = 0.f;
#pragma unroll
    for (int cc = g * (DK / 4); cc < (g + 1) * (DK / 4); cc += 8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.kv[row * SK + cc]);
      const u32x4 y = *reinterpret_cast<const u32x4*>(&sm.q[row * SQ + cc]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = __uint_as_float(x[j] << 16), a1 = __uint_as_float(x[j] & 0xFFFF0000u);
        const float b0 = __uint_as_float(y[j] << 16), b1 = __uint_as_float(y[j] & 0xFFFF0000u);
        acck += a0 * a0 + a1 * a1;
        accq += b0 * b0 + b1 * b1;
      }
    }
    acck += __shfl_xor(acck, 16, 64);
    acck += __shfl_xor(acck, 32, 64);
    accq += __shfl_xor(accq, 16, 64);
    accq += __shfl_xor(accq, 32, 64);
    if (g == 0) {
      const float r = 1.0f / sqrtf(acck + kNormEps);
      const float rq = 1.0f / sqrtf(accq + kNormEps);
      sm.rk[row] = r;
      sm.rq[row] = rq;
      kd_out[pair * C + row] = expf((float)(sm.G[C - 1] - sm.G[row])) * r;
      erq_out[pair * C + row] = sm.eg[row] * rq;
    }
  }
  lds_barrier();

  // ---- Gram tiles (I >= J) of raw K K^T -> A (strictly lower, scaled)
  {
    constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    for (int idx = w; idx < 10; idx += 4) {
      const int I = TI[idx], J = TJ[idx];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        const bf16x8 a = bf16x8_from_u32x4(row_frag(sm.kv, SK, 16 * I + m, 32 * s, g));
        const bf16x8 b = bf16x8_from_u32x4(row_frag(sm.kv, SK, 16 * J + m, 32 * s, g));
        acc = mma_bf16(a, b, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * g + i, cc = 16 * J + m;
        sm.u.A[r][cc] = (cc < r) ? sm.bt[r] * sm.rk[r] * sm.rk[cc] * acc[i] : 0.f;
      }
    }
  }
  // ---- A_qk = Gamma o tril0(Qh Kh^T), rows 16w..16w+15, computed transposed
  // (D[i][r] = (K Q^T)[16J+4g+ii][16w+m] on the raw bf16 values, then scaled by
  // e^{G_r - G_i} r_k[i] r_q[r], i <= r). Stored as the A fragments of A_qk U in the
  // state kernel: k step s holds token tiles 2s and 2s + 1.
  {
    const int r = 16 * w + m;
    const double Gr = sm.G[r];
    const float rq = sm.rq[r];
    half4 t4[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          acc = mma_bf16(bf16x8_from_u32x4(row_frag(sm.kv, SK, 16 * J + m, 32 * s, g)),
                         bf16x8_from_u32x4(row_frag(sm.q, SQ, r, 32 * s, g)), acc);
      }
      f32x4 val;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * J + 4 * g + ii;
        val[ii] = (i <= r) ? expf((float)(Gr - sm.G[i])) * sm.rk[i] * rq * acc[ii] : 0.f;
      }
      t4[J] = to_half4(val);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      *reinterpret_cast<half8*>(Aout + pair * C * C + ((w * 2 + s) * 64 + l) * 8) =
          cat(t4[2 * s], t4[2 * s + 1]);
  }
  lds_barrier();

  // ---- T = (I + A)^-1, diagonal 16x16 blocks: wave w, lane = column
  if (l < 16) {
    const int b0 = 16 * w, col = l;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc += sm.u.A[b0 + r][b0 + i] * t[i];
      t[r] = (r < col) ? 0.f : ((r == col) ? 1.f : -acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.T[b0 + r][b0 + col] = t[r];
  }
  lds_barrier();
  // off-diagonal blocks by distance d = I - J; X = sum_K A_IK T_KJ, then T_IJ = -T_II X
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int J = w, I = w + d;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          X = mma_f32(sm.u.A[16 * I + m][16 * K + 4 * s + g], sm.T[16 * K + 4 * s + g][16 * J + m], X);
      }
      // Y = T_II X with contraction index 4g + s, so lane (g, m) feeds X[4g + s][m] = X[s]
      f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) Y = mma_f32(sm.T[16 * I + m][16 * I + 4 * g + s], X[s], Y);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.T[16 * I + 4 * g + i][16 * J + m] = -Y[i];
    }
    lds_barrier();
  }

  // ---- T1 = diag(e^G) T diag(beta r_k) as bf16 hi + lo (overwrites A)
  for (int e = tid; e < C * C; e += 256) {
    const int r = e >> 6, i = e & 63;
    const float x = (i <= r) ? sm.eg[r] * sm.T[r][i] * sm.bt[i] * sm.rk[i] : 0.f;
    const uint16_t hi = f32_to_bf16_bits(x);
    sm.u.Ts[0][r * ST + i] = hi;
    sm.u.Ts[1][r * ST + i] = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
  }
  lds_barrier();

  // ---- W<-^T = K^T T1^T: wave w owns 32-wide dk steps s' = w, w + 4, ...; the two
  // 16-row D tiles of a step form exactly the state kernel's A fragment of W<-.
  for (int sp = w; sp < DK / 32; sp += 4) {
    f32x4 acc[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int I = 0; I < 4; ++I) acc[tt][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // token k steps
      bf16x8 a[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        a[tt] = bf16x8_from_u32x4(col_frag(sm.kv, SK, 32 * sp + 16 * tt + m, 32 * s, g));
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x8 bh = bf16x8_from_u32x4(row_frag(sm.u.Ts[0], ST, 16 * I + m, 32 * s, g));
        const bf16x8 bl = bf16x8_from_u32x4(row_frag(sm.u.Ts[1], ST, 16 * I + m, 32 * s, g));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          acc[tt][I] = mma_bf16(a[tt], bh, acc[tt][I]);
          acc[tt][I] = mma_bf16(a[tt], bl, acc[tt][I]);
        }
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const half8 hv8 = cat(to_half4(acc[0][I]), to_half4(acc[1][I]));
      *reinterpret_cast<half8*>(Wout + pair * C * DK + ((I * (DK / 32) + sp) * 64 + l) * 8) = hv8;
    }
  }
  lds_barrier();

  // ---- V into LDS; T2 = (Gamma o T) diag(beta) as bf16 hi + lo
#pragma unroll
  for (int u = 0; u < VP; ++u) {
    const int e = tid + 256 * u, row = e / (DV / 8), c8 = (e % (DV / 8)) * 8;
    *reinterpret_cast<u32x4*>(&sm.kv[row * SK + c8]) = vreg[u];
  }
  for (int e = tid; e < C * C; e += 256) {
    const int r = e >> 6, i = e & 63;
    const float x = (i <= r) ? expf((float)(sm.G[r] - sm.G[i])) * sm.T[r][i] * sm.bt[i] : 0.f;
    const uint16_t hi = f32_to_bf16_bits(x);
    sm.u.Ts[0][r * ST + i] = hi;
    sm.u.Ts[1][r * ST + i] = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
  }
  lds_barrier();

  // ---- U~ = T2 V: wave w owns dv column tiles u = w, w + 4, ...; D tiles are stored as
  // they are, which is the layout the state kernel adds them in.
  for (int ut = w; ut < DV / 16; ut += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) acc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 b = bf16x8_from_u32x4(col_frag(sm.kv, SK, 16 * ut + m, 32 * s, g));
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x8 ah = bf16x8_from_u32x4(row_frag(sm.u.Ts[0], ST, 16 * I + m, 32 * s, g));
        const bf16x8 al = bf16x8_from_u32x4(row_frag(sm.u.Ts[1], ST, 16 * I + m, 32 * s, g));
        acc[I] = mma_bf16(ah, b, acc[I]);
        acc[I] = mma_bf16(al, b, acc[I]);
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
      *reinterpret_cast<half4*>(Uout + pair * C * DV + ((ut * 4 + I) * 64 + l) * 4) = to_half4(acc[I]);
  }
}

template <int DK, int DV>
hipError_t launch_prep_t(const void* q, const void* k, const void* v, const int64_t* cu,
                         const int32_t* off, const int32_t* cseq, const double* gcum,
                         const float* beta, const Shape& s, int64_t max_chunks, _Float16* w,
                         _Float16* u, float* kd, _Float16* aqk, float* erq, hipStream_t st) {
  hipLaunchKernelGGL((mfma_prep_kernel<DK, DV>), dim3((unsigned)max_chunks, (unsigned)s.HV),
                     dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     cu, off, cseq, gcum, beta, s.H, s.HV, w, u, kd, aqk, erq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_prep(const void* q, const void* k, const void* v,
                            const int64_t* cu_seqlens, const int32_t* chunk_off,
                            const int32_t* chunk_seq, const double* gcum, const float* beta,
                            const Shape& s, int64_t max_chunks, void* w, void* u, float* kd,
                            void* aqk, float* erq, hipStream_t st) {
  _Float16* W = (_Float16*)w;
  _Float16* U = (_Float16*)u;
#define GDN_PREP_CASE(DKv, DVv)                                                               \
  if (s.dk == DKv && s.dv == DVv)                                                             \
    return launch_prep_t<DKv, DVv>(q, k, v, cu_seqlens, chunk_off, chunk_seq, gcum, beta, s,  \
                                   max_chunks, W, U, kd, (_Float16*)aqk, erq, st);
  GDN_PREP_CASE(64, 64)
  GDN_PREP_CASE(64, 128)
  GDN_PREP_CASE(64, 256)
  GDN_PREP_CASE(128, 64)
  GDN_PREP_CASE(128, 128)
  GDN_PREP_CASE(128, 256)
  GDN_PREP_CASE(256, 64)
  GDN_PREP_CASE(256, 128)
  GDN_PREP_CASE(256, 256)
#undef GDN_PREP_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
