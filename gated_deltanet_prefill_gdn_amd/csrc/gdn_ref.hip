// Chunkwise GDN forward in fp32 arithmetic: products on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32: fp32 products, fp32 sums), everything else in fp32 vector code.
//
// This family serves fp32 inputs, where every operand must stay in fp32. Per chunk of
// n <= C rows (row convention: S is dv x dk, K and Q are n x dk, V is n x dv; G is the
// chunk-local inclusive log cumulative gate, r_k = 1/|k| and r_q = 1/|q|):
//   A    = tril(diag(beta r_k) K K^T diag(r_k), -1)
//   T    = (I + A)^-1                              the one inverse, M^-1
//   W<-  = diag(e^G) T diag(beta r_k) K            W up to the decay (veitner page,
//                                                  Reminder, equation for W)
//   U~   = (Gamma o T) diag(beta) V,  Gamma_ri = exp(G_r - G_i) for i <= r
//          This is N^-1 B V with N^-1 = G M^-1 G^-1 (veitner page, Save one invert),
//          applied entry by entry so no 1/gamma is formed.
//   A_qk = Gamma o tril0(diag(r_q) Q K^T diag(r_k)),  K~ = diag(e^{G_n - G} r_k) K,
//   Qf   = diag(e^G r_q) Q
// (the prep kernel, one workgroup per chunk and value head), and then, sequentially over
// the chunks of a request (pymllm gdn_chunkwise page, Algorithm, steps 2 and 3, in row
// convention; the state kernel, one workgroup per request, value head and 16 or 32 state
// rows):
//   U     = U~ - W<- S^T
//   O     = Qf S^T + A_qk U
//   S_new = e^{G_n} S + U^T K~
//
// Contraction order. In v_mfma_f32_16x16x4f32 lane (m, g) supplies A[m][k] and B[k][m] for
// the step's k = g. Over a block of 16 contraction indices these kernels let step s take
// k = 4g + s (s = 0..3), so each lane's four values of A (and of B) for four consecutive
// steps are four consecutive floats: one 16-byte load instead of four. The operands are
// stored (or staged) so that those runs are contiguous: U~ and K~ are written transposed,
// and U is kept transposed in LDS.
//
// The prep kernel writes its outputs with non-temporal stores: the state kernel reads each
// block once per workgroup from the L2 it is written through, and dirty lines left in the
// caches slow those reads (measured: 2.6% off the dense batch's call, 1.2% off the wide-head
// one).
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;
constexpr double kLog2e = 1.4426950408889634;

__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }

// Four consecutive input elements from index i: one 16-byte load where the inputs are
// 16-byte aligned (then every row is: dk and dv are multiples of 4), four otherwise (this
// path accepts inputs aligned to their element only).
__device__ __forceinline__ f32x4 ld4(const float* p, int64_t i, bool aligned) {
  if (aligned) return *reinterpret_cast<const f32x4*>(p + i);
  return f32x4{p[i], p[i + 1], p[i + 2], p[i + 3]};
}

// Four fp32 MFMA steps over 16 contraction indices: step s takes k = 4g + s.
__device__ __forceinline__ f32x4 mma4(f32x4 a, f32x4 b, f32x4 acc) {
  acc = mma_f32(a[0], b[0], acc);
  acc = mma_f32(a[1], b[1], acc);
  acc = mma_f32(a[2], b[2], acc);
  acc = mma_f32(a[3], b[3], acc);
  return acc;
}

template <int DM>
struct RefPrepSmem {
  alignas(16) float tile[C][DM + 4];  // K rows (zero past n), later V rows
  alignas(16) float A[C][C + 4];      // A, then T1 = diag(e^G) T diag(beta r_k), then T2
  alignas(16) float T[C][C + 4];      // T = (I + A)^-1
  alignas(16) float X[4][16][20];     // per wave: one 16 x 16 tile of the blocked inverse
  double G2[C];  // G log2(e)
  float bt[C], rk[C], rq[C], kd[C], eq[C], eg[C];
};

// One workgroup per (global chunk, value head); wave w owns chunk rows 16w .. 16w + 15.
// Head dims are compile-time constants, so every staging loop has a fixed trip count and
// issues its loads together.
template <int DK, int DV>
__global__ __launch_bounds__(256) void ref_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ chunk_seq, const double* __restrict__ gcum,
    const float* __restrict__ beta, int H, int HV, int aligned, float* __restrict__ W,
    float* __restrict__ Ut, float* __restrict__ Aqk, float* __restrict__ Kft,
    float* __restrict__ Qf) {
  constexpr int dk = DK, dv = DV;
  __shared__ RefPrepSmem<(DK > DV ? DK : DV)> sm;
  const int64_t c = blockIdx.x;
  const int hv = blockIdx.y;
  const int32_t seq = chunk_seq[c];
  if (seq < 0) return;
  const int h = hv / (HV / H);
  const int64_t t0 = cu[seq] + (int64_t)(c - chunk_off[seq]) * C;
  const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
  const int64_t pair = c * HV + hv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int I = w;  // this wave's row tile

  const bool al = aligned != 0;
  if (tid < C) {
    sm.G2[tid] = gcum[pair * C + tid] * kLog2e;
    sm.bt[tid] = beta[pair * C + tid];
  }
  // K rows in 4-element pieces: piece u of thread tid is e = tid + 256u, row e / (dk / 4)
#pragma unroll
  for (int e = tid; e < C * dk / 4; e += 256) {
    const int r = e / (dk / 4), j = 4 * (e % (dk / 4));
    *reinterpret_cast<f32x4*>(&sm.tile[r][j]) =
        r < n ? ld4(k, ((t0 + r) * H + h) * (int64_t)dk + j, al) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // This lane's fragments of Q: row qr = 16 I + m, columns 16 kb + 4g .. 16 kb + 4g + 3
  // (zero past n), the A operand of A_qk and the source of Qf. Q is read once.
  const int qr = 16 * I + m;
  f32x4 qa[dk / 16];
#pragma unroll
  for (int kb = 0; kb < dk / 16; ++kb)
    qa[kb] = qr < n ? ld4(q, ((t0 + qr) * H + h) * (int64_t)dk + 16 * kb + 4 * g, al)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
  // V rows, loaded now (in the same pieces) and staged in LDS once the K tile is no longer
  // read
  constexpr int kVPer = C * dv / 4 / 256;
  f32x4 vr[kVPer];
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int e = tid + 256 * i, r = e / (dv / 4), j = 4 * (e % (dv / 4));
    vr[i] = r < n ? ld4(v, ((t0 + r) * HV + hv) * (int64_t)dv + j, al) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  // inverse row norms: lane (m, g) sums its columns of row qr, the four lanes of a row add up
  {
    float ak = 0.f, aq = 0.f;
#pragma unroll
    for (int kb = 0; kb < dk / 16; ++kb) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.tile[qr][16 * kb + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ak += x[e] * x[e];
        aq += qa[kb][e] * qa[kb][e];
      }
    }
    ak += __shfl_xor(ak, 16, 64);
    ak += __shfl_xor(ak, 32, 64);
    aq += __shfl_xor(aq, 16, 64);
    aq += __shfl_xor(aq, 32, 64);
    if (g == 0) {
      sm.rk[qr] = qr < n ? (float)(1.0 / sqrt((double)ak + (double)kNormEps)) : 0.f;
      sm.rq[qr] = qr < n ? (float)(1.0 / sqrt((double)aq + (double)kNormEps)) : 0.f;
    }
  }
  __syncthreads();

  // ---- A = tril(diag(beta r_k) K K^T diag(r_k), -1): tiles (I, J <= I) of this wave
  {
    f32x4 acc[4] = {};
#pragma unroll
    for (int k0 = 0; k0 < dk; k0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.tile[16 * I + m][k0 + 4 * g]);
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= I) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.tile[16 * J + m][k0 + 4 * g]);
          acc[J] = mma4(a, b, acc[J]);
        }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * g + i, col = 16 * J + m;
        sm.A[r][col] = (J <= I && col < r && r < n)
                           ? sm.bt[r] * sm.rk[r] * sm.rk[col] * acc[J][i]
                           : 0.f;
      }
  }
  __syncthreads();
  // ---- T = (I + A)^-1, blocked in 16 x 16 tiles. Diagonal tile (I, I) by forward
  // substitution in wave I: lane l < 16 holds column l of the tile in registers, and every
  // lane reads row rr of A_II (the same address, a broadcast). Then by block distance
  // d = I - J on the matrix cores: T_IJ = -T_II X with X = sum_{J <= K < I} A_IK T_KJ.
  {
    float t[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float acc = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < rr; i4 += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.A[16 * I + rr][16 * I + i4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i4 + e < rr) acc += a[e] * t[i4 + e];
      }
      t[rr] = (rr == m ? 1.f : 0.f) - acc;  // columns l < rr only pick up t[i >= l]
    }
    if (l < 16) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.T[16 * I + rr][16 * I + l] = rr >= l ? t[rr] : 0.f;
    }
    // the tiles above the diagonal
#pragma unroll
    for (int J = 0; J < 4; ++J)
      if (J > I)
        for (int idx = l; idx < 256; idx += 64) sm.T[16 * I + idx / 16][16 * J + idx % 16] = 0.f;
  }
  for (int d = 1; d < 4; ++d) {
    __syncthreads();  // every tile at distance < d is in sm.T
    const int J = I - d;
    if (J >= 0) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.A[16 * I + m][16 * K + 4 * g]);
        f32x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = sm.T[16 * K + 4 * g + e][16 * J + m];
        x = mma4(a, b, x);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.X[I][4 * g + i][m] = x[i];
    }
    __syncthreads();  // X of every wave at this distance is in LDS
    if (J >= 0) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.T[16 * I + m][16 * I + 4 * g]);
      f32x4 b;
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = sm.X[I][4 * g + e][m];
      const f32x4 y = mma4(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.T[16 * I + 4 * g + i][16 * J + m] = -y[i];
    }
  }
  __syncthreads();
  // ---- row scales and T1 = diag(e^G) T diag(beta r_k). Decays are powers of two of
  // non-positive exponent differences (G is non-increasing), formed with v_exp_f32.
  const double G2n = sm.G2[n - 1];
  if (tid < C) {
    const float egt = __builtin_amdgcn_exp2f((float)sm.G2[tid]);
    sm.eg[tid] = tid < n ? egt : 0.f;
    sm.kd[tid] = tid < n ? __builtin_amdgcn_exp2f((float)(G2n - sm.G2[tid])) * sm.rk[tid] : 0.f;
    sm.eq[tid] = tid < n ? egt * sm.rq[tid] : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    sm.A[r][i] = (i <= r) ? sm.eg[r] * sm.T[r][i] * sm.bt[i] * sm.rk[i] : 0.f;
  }
  __syncthreads();
  // ---- W<- = T1 K (rows of tile I), A_qk (tiles J <= I), K~^T, Qf
  float* Wp = W + pair * (int64_t)C * dk;
  for (int jd = 0; jd < dk / 16; ++jd) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.A[16 * I + m][k0 + 4 * g]);
      f32x4 b;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = sm.tile[k0 + 4 * g + s][16 * jd + m];
      acc = mma4(a, b, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_nontemporal_store(acc[i], &Wp[(int64_t)(16 * I + 4 * g + i) * dk + 16 * jd + m]);
  }
  {
    f32x4 acc[4] = {};
#pragma unroll
    for (int kb = 0; kb < dk / 16; ++kb) {
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= I) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.tile[16 * J + m][16 * kb + 4 * g]);
          acc[J] = mma4(qa[kb], b, acc[J]);
        }
    }
    float* Ap = Aqk + pair * (int64_t)C * C;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * g + i, col = 16 * J + m;
        const float x = (J <= I && col <= rr && rr < n)
                            ? __builtin_amdgcn_exp2f((float)(sm.G2[rr] - sm.G2[col])) *
                                  sm.rq[rr] * sm.rk[col] * acc[J][i]
                            : 0.f;
        __builtin_nontemporal_store(x, &Ap[rr * C + col]);
      }
  }
  float* Kp = Kft + pair * (int64_t)C * dk;  // K~ transposed: [dk][C]
#pragma unroll
  for (int idx = tid; idx < C * dk; idx += 256) {
    const int j = idx / C, r = idx - j * C;
    __builtin_nontemporal_store(sm.kd[r] * sm.tile[r][j], &Kp[idx]);
  }
  float* Qp = Qf + pair * (int64_t)C * dk + (int64_t)qr * dk + 4 * g;
  const float eqr = sm.eq[qr];  // zero past n
#pragma unroll
  for (int kb = 0; kb < dk / 16; ++kb)
    __builtin_nontemporal_store(eqr * qa[kb], reinterpret_cast<f32x4*>(Qp + 16 * kb));
  __syncthreads();  // the K tile and T1 are no longer read
  // ---- U~ = T2 V with T2 = (Gamma o T) diag(beta), written transposed: [dv][C]
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx / C, i = idx % C;
    sm.A[r][i] = (i <= r && r < n)
                     ? __builtin_amdgcn_exp2f((float)(sm.G2[r] - sm.G2[i])) * sm.T[r][i] * sm.bt[i]
                     : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int e = tid + 256 * i, r = e / (dv / 4), j = 4 * (e % (dv / 4));
    *reinterpret_cast<f32x4*>(&sm.tile[r][j]) = vr[i];
  }
  __syncthreads();
  float* Up = Ut + pair * (int64_t)C * dv;
  for (int jd = 0; jd < dv / 16; ++jd) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.A[16 * I + m][k0 + 4 * g]);
      f32x4 b;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = sm.tile[k0 + 4 * g + s][16 * jd + m];
      acc = mma4(a, b, acc);
    }
    __builtin_nontemporal_store(
        acc, reinterpret_cast<f32x4*>(&Up[(int64_t)(16 * jd + m) * C + 16 * I + 4 * g]));
  }
}

template <int DK, int NC>
struct RefStateSmem {
  alignas(16) float S[16 * NC][DK + 4];  // this workgroup's rows of S, all dk columns
  alignas(16) float Ut[16 * NC][C + 4];  // U of the current chunk, transposed: [column][token]
};

// One workgroup per (request, value head, 16 NC state rows); walks the request's chunks in
// order with its rows of S resident in LDS. Wave w owns chunk rows 16w .. 16w + 15 for U
// and O, and dk rows 16 jd .. for jd = w (mod 4) of the state update; its fragments of
// W<-, Qf, A_qk and K~ serve all NC column tiles. Each wave holds its fragments of the
// chunk's operands in registers and loads the next chunk's into each register as soon as
// the current product has taken it, so every load has about a chunk to land. The
// workgroup's barriers wait for LDS traffic only.
// Workgroup id -> (pair, slice): the slices of one (request, value head) pair get
// consecutive ids of one XCD (ids are dealt to the 8 XCDs in turn), so they are dispatched
// together and read the pair's per-chunk operands through that XCD's L2.
template <int DK, int NC>
__global__ __launch_bounds__(256) void ref_state_kernel(
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const double* __restrict__ gcum,
    const float* __restrict__ W, const float* __restrict__ Ut, const float* __restrict__ Aqk,
    const float* __restrict__ Kft, const float* __restrict__ Qf, int64_t B, int HV, int dv,
    int64_t short_len, float* __restrict__ state_pool, float* __restrict__ out,
    int32_t* __restrict__ nonfinite) {
  constexpr int NK = DK / 16;  // 16-wide contraction blocks over dk
  constexpr int NT = DK / 64;  // dk tiles of the state update per wave
  constexpr int BV = 16 * NC;  // state rows of the workgroup
  __shared__ RefStateSmem<DK, NC> sm;
  const int nsl = dv / BV;
  const int64_t id = blockIdx.x, slot8 = id / 8;
  const int64_t pidx = slot8 / nsl * 8 + id % 8;
  if (pidx >= B * HV) return;  // the pair count rounded up to 8
  const int64_t seq = pidx / HV;
  const int hv = (int)(pidx - seq * HV), v0 = (int)(slot8 % nsl) * BV;
  const int64_t tb = cu[seq], te = cu[seq + 1];
  const int64_t nchunks = path_chunks(te - tb, C, short_len);
  if (nchunks == 0) return;  // empty (slot untouched) or evaluated by the token recurrence
  const int64_t slot = cache_indices[seq];
  const int64_t c0 = chunk_off[seq];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  float* Sg = state_pool + ((slot * HV + hv) * (int64_t)dv + v0) * DK;
  for (int idx = tid; idx < BV * DK; idx += 256) sm.S[idx / DK][idx % DK] = Sg[idx];

  // this wave's fragments of a chunk (lane (m, g): 16-byte runs at contraction 4g)
  f32x4 wa[NK], qa[NK], ut[NC], aa[4], ka[NT][4];
  double gn;
  auto pair_of = [&](int64_t cl) { return (c0 + cl) * HV + hv; };
  auto wq_ptr = [&](const float* base, int64_t cl) {  // rows 16w + m of W<- or Qf
    return base + pair_of(cl) * (int64_t)C * DK + (16 * w + m) * DK + 4 * g;
  };
  auto load_u = [&](int64_t cl) {  // U~ columns v0 + 16c + m, tokens 16w + 4g ..
    const float* up = Ut + pair_of(cl) * (int64_t)C * dv + (int64_t)(v0 + m) * C + 16 * w + 4 * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) ut[c] = *reinterpret_cast<const f32x4*>(up + 16 * c * C);
  };
  auto load_ak = [&](int64_t cl) {  // A_qk rows 16w + m; K~^T rows 16 (w + 4t) + m; G_n
    const int64_t p = pair_of(cl);
    const float* Ap = Aqk + p * (int64_t)C * C + (16 * w + m) * C + 4 * g;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) aa[kb] = *reinterpret_cast<const f32x4*>(Ap + 16 * kb);
    const float* Kp = Kft + p * (int64_t)C * DK + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ka[t][kb] = *reinterpret_cast<const f32x4*>(Kp + (16 * (w + 4 * t) + m) * C + 16 * kb);
    const int64_t n = min((int64_t)C, te - tb - cl * C);
    gn = gcum[p * C + n - 1];
  };
  {
    const float* Wp = wq_ptr(W, 0);
    const float* Qp = wq_ptr(Qf, 0);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      wa[kb] = *reinterpret_cast<const f32x4*>(Wp + 16 * kb);
      qa[kb] = *reinterpret_cast<const f32x4*>(Qp + 16 * kb);
    }
  }
  load_u(0);
  load_ak(0);
  // Two barriers per chunk: every read of S comes before the first, every write of S after
  // the second, and U passes through LDS between them.
  for (int64_t cl = 0; cl < nchunks; ++cl) {
    const int64_t t0 = tb + cl * C;
    const int n = (int)min((int64_t)C, te - t0);
    const int64_t nx = min(cl + 1, nchunks - 1);  // the last chunk reloads itself
    lds_barrier();  // the previous chunk's S update and U reads are complete
    // ---- U = U~ - W<- S^T and the state part Qf S^T of O, tokens 16w .., each column
    // tile (independent accumulator chains)
    f32x4 pu[NC], po[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      pu[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      po[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float* Wn = wq_ptr(W, nx);
    const float* Qn = wq_ptr(Qf, nx);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.S[16 * c + m][16 * kb + 4 * g]);
        pu[c] = mma4(wa[kb], b, pu[c]);
        po[c] = mma4(qa[kb], b, po[c]);
      }
      wa[kb] = *reinterpret_cast<const f32x4*>(Wn + 16 * kb);
      qa[kb] = *reinterpret_cast<const f32x4*>(Qn + 16 * kb);
    }
    // lane (m, g) holds tokens 16w + 4g + i of column v0 + 16c + m
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *reinterpret_cast<f32x4*>(&sm.Ut[16 * c + m][16 * w + 4 * g]) = ut[c] - pu[c];
    load_u(nx);
    lds_barrier();  // U complete; S is not read again in this chunk
    // ---- O += A_qk U (A_qk is causal: tokens up to 16w + 15)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      if (kb <= w) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.Ut[16 * c + m][16 * kb + 4 * g]);
          po[c] = mma4(aa[kb], b, po[c]);
        }
      }
    // ---- S^T <- e^{G_n} S^T + K~^T U, dk tiles jd = w + 4t
    const float egn = expf((float)gn);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.Ut[16 * c + m][16 * kb + 4 * g]);
          acc = mma4(ka[t][kb], b, acc);
        }
        // lane (m, g) holds S^T rows 16 jd + 4g + i, column 16c + m
        f32x4* sp = reinterpret_cast<f32x4*>(&sm.S[16 * c + m][16 * (w + 4 * t) + 4 * g]);
        *sp = egn * *sp + acc;
      }
    }
    load_ak(nx);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i;
        if (r < n) st(out, ((t0 + r) * HV + hv) * (int64_t)dv + v0 + 16 * c + m, po[c][i]);
      }
  }
  lds_barrier();
  bool finite = true;
  for (int idx = tid; idx < BV * DK; idx += 256) {
    const float x = sm.S[idx / DK][idx % DK];
    Sg[idx] = x;
    finite = finite && __builtin_isfinite(x);
  }
  if (!finite) *nonfinite = 1;
}

template <int DK, int DV>
void launch_prep_t(const void* q, const void* k, const void* v, const int64_t* cu,
                   const int32_t* chunk_off, const int32_t* chunk_seq, const double* gcum,
                   const float* beta, const Shape& s, int64_t max_chunks, float* w, float* ut,
                   float* aqk, float* kft, float* qf, hipStream_t st) {
  const dim3 grid((unsigned)max_chunks, (unsigned)s.HV);
  const int aligned = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) == 0;
  hipLaunchKernelGGL((ref_prep_kernel<DK, DV>), grid, dim3(256), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, cu, chunk_off, chunk_seq, gcum, beta, s.H,
                     s.HV, aligned, w, ut, aqk, kft, qf);
}

// Two column tiles (32 state rows) per workgroup where those workgroups fill the device:
// the per-chunk operands a workgroup must take in then serve twice the columns (the pass is
// bound by that intake); one (16 rows) where they would not, which doubles the workgroups
// walking the chains.
template <int DK>
void launch_state_t(const int64_t* cu, const int64_t* idx, const int32_t* chunk_off,
                    const double* gcum, const float* w, const float* ut, const float* aqk,
                    const float* kft, const float* qf, const Shape& s, float* pool, void* out,
                    int32_t* nonfinite, hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8 * 8;
  if (s.B * s.HV * (s.dv / 32) >= 256)
    hipLaunchKernelGGL((ref_state_kernel<DK, 2>), dim3((unsigned)(pairs8 * (s.dv / 32))),
                       dim3(256), 0, st, cu, idx, chunk_off, gcum, w, ut, aqk, kft, qf, s.B,
                       s.HV, s.dv, s.short_len, pool, (float*)out, nonfinite);
  else
    hipLaunchKernelGGL((ref_state_kernel<DK, 1>), dim3((unsigned)(pairs8 * (s.dv / 16))),
                       dim3(256), 0, st, cu, idx, chunk_off, gcum, w, ut, aqk, kft, qf, s.B,
                       s.HV, s.dv, s.short_len, pool, (float*)out, nonfinite);
}

}  // namespace

// fp32 inputs only (bf16 inputs take the matrix-core kernels).
hipError_t launch_ref_prep(const void* q, const void* k, const void* v,
                           const int64_t* cu_seqlens, const int32_t* chunk_off,
                           const int32_t* chunk_seq, const double* gcum, const float* beta,
                           const Shape& s, int64_t max_chunks, float* w, float* ut, float* aqk,
                           float* kft, float* qf, hipStream_t st) {
  if (s.bf16) return hipErrorInvalidValue;
#define GDN_REF_PREP(DKv, DVv)                                                              \
  if (s.dk == DKv && s.dv == DVv) {                                                         \
    launch_prep_t<DKv, DVv>(q, k, v, cu_seqlens, chunk_off, chunk_seq, gcum, beta, s,       \
                            max_chunks, w, ut, aqk, kft, qf, st);                           \
    return hipGetLastError();                                                               \
  }
  GDN_REF_PREP(64, 64)
  GDN_REF_PREP(64, 128)
  GDN_REF_PREP(64, 256)
  GDN_REF_PREP(128, 64)
  GDN_REF_PREP(128, 128)
  GDN_REF_PREP(128, 256)
  GDN_REF_PREP(256, 64)
  GDN_REF_PREP(256, 128)
  GDN_REF_PREP(256, 256)
#undef GDN_REF_PREP
  return hipErrorInvalidValue;
}

hipError_t launch_ref_state(const int64_t* cu_seqlens, const int64_t* cache_indices,
                            const int32_t* chunk_off, const double* gcum, const float* w,
                            const float* ut, const float* aqk, const float* kft, const float* qf,
                            const Shape& s, float* state_pool, void* out, int32_t* nonfinite,
                            hipStream_t st) {
  if (s.bf16) return hipErrorInvalidValue;
#define GDN_REF_STATE(DKv)                                                                  \
  if (s.dk == DKv) {                                                                        \
    launch_state_t<DKv>(cu_seqlens, cache_indices, chunk_off, gcum, w, ut, aqk, kft, qf, s, \
                        state_pool, out, nonfinite, st);                                    \
    return hipGetLastError();                                                               \
  }
  GDN_REF_STATE(64)
  GDN_REF_STATE(128)
  GDN_REF_STATE(256)
#undef GDN_REF_STATE
  return hipErrorInvalidValue;
}

}  // namespace gdn
