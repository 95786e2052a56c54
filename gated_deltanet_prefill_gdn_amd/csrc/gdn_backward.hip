// Backward of the prefill: gradients of every input given the gradients of the outputs
// and of each request's final state.
//
// The forward is the token recurrence ("Simple math to speed up GDN prefill", section
// Reminder; gates and normalisation from the pymllm gdn_chunkwise page, Module Contents)
//   S_t = alpha S_{t-1} - alpha beta (S_{t-1} kh) kh^T + beta v kh^T,   out_t = S_t qh,
// whose chunked evaluation reaches the same map, so these are the chunked forward's
// gradients too. Reverse mode carries D = dL/dS_t from the last token to the first; with
// Sp = S_{t-1} and row i of D, Sp:
//   D     += dout_t qh^T
//   dqh   += S_t^T dout_t                       dv_i   = beta (D kh)_i
//   dbeta += sum_i (D kh)_i (v_i - alpha (Sp kh)_i)
//   dalpha+= sum_i D_i . Sp_i - beta (D kh)_i (Sp kh)_i
//   dkh   += sum_i -alpha beta ((Sp kh)_i D_i + (D kh)_i Sp_i) + beta v_i D_i
//   D     <- alpha (D - beta (D kh) kh^T)
// The rows of S and D are independent; only dqh, dkh, dalpha and dbeta sum over rows.
//
// Kernels (fp32 arithmetic throughout):
//   token   one wave per (token, q/k head): the normalised q and k rows and, for the value
//           heads sharing them, alpha and beta, written once so that the sweeps below only
//           load them.
//   rows    one workgroup per (request, value head, 32 rows), sixteen waves (one
//           workgroup per CU). A forward sweep keeps the rows' state every 8 tokens; the
//           reverse sweep recomputes 8 tokens at a time (4 at dk = 256) from the checkpoint
//           before them, holds the states before each of them in registers (the state
//           after token i is the one before token i + 1, or the sub-chunk's end state), and
//           walks them backwards. Wave w holds rows 2w and 2w + 1, lane l the dk elements
//           l + 64 e: few registers per wave, so four waves share each SIMD and hide the
//           latency of the token-to-token chain. Each group's token inputs (q, k rows,
//           gates, the block's rows of v and dout) are staged once per workgroup in LDS,
//           loaded by all threads one group ahead. A token's row dot products (two per
//           row) are reduced together: a permlane reduce-scatter, then one 16-lane DPP
//           reduction. The per-token sums over the 32 rows go through LDS into a partial
//           buffer per row block (no atomics: the result does not depend on scheduling).
//   finish  one wave per (token, q/k head): sums the partials over row blocks and over
//           the value heads that share the q/k head, then the chain rule through the L2
//           norm (dq = dqh / n - q (q . dqh) / n^3) and the gates (da = dalpha dalpha/dx,
//           db = dbeta beta (1 - beta)).
//   gates   one workgroup per value head: dA_log and dt_bias gradients as sums over tokens.
#include <algorithm>

#include "gdn_internal.h"
#include "gdn_backward.h"

namespace gdn {
namespace {

constexpr int kCk = 8;             // tokens between checkpoints
constexpr int kBwdRows = 32;       // state rows per workgroup
constexpr int kRowsPerWave = 2;
constexpr int kRowWaves = kBwdRows / kRowsPerWave;  // waves of a row workgroup
constexpr int kRowThreads = 64 * kRowWaves;
template <int DK>
constexpr int kSub = DK <= 128 ? 8 : 4;  // tokens recomputed and walked back at a time

__device__ __forceinline__ float ldx(const void* p, int64_t i, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16)
              : reinterpret_cast<const float*>(p)[i];
}

// kRowsPerWave (2) consecutive elements starting at a multiple of 2 (4- or 8-byte aligned).
__device__ __forceinline__ void ld_rows(const void* p, int64_t i, bool bf16,
                                        float (&x)[kRowsPerWave]) {
  static_assert(kRowsPerWave == 2, "one 2-element load");
  if (bf16) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(p) + i);
    x[0] = __uint_as_float(u << 16);
    x[1] = __uint_as_float(u & 0xFFFF0000u);
  } else {
    const float2 f = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(p) + i);
    x[0] = f.x;
    x[1] = f.y;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the wave, in every lane, without LDS: four DPP steps reduce each row of 16 lanes
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror), then gfx950's
// permlane16/permlane32 swaps add row pairs and the wave's halves. Each swap exchanges two
// disjoint lane sets, so the sum of its two results is the same whichever result is which.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// Sum over each 16-lane row, in every lane of the row (the first four steps above).
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}

// One permlane swap step of a reduce-scatter: returns, in lanes whose (32- or 16-lane)
// group comes first, a's sum over that group and its partner group, and b's in the
// others. The permlane32 form pairs the wave's halves, the permlane16 form the two
// 16-lane rows of each half (rows 0, 1 and rows 2, 3).
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Wave sums of two values at once (a reduce-scatter: each step halves the lanes a value
// occupies instead of reducing each value over all 64 lanes), as wave-uniform results.
__device__ __forceinline__ void wave_sum2(float a, float b, float& sa, float& sb) {
  float x = swap_add32(a, b);  // a in lanes 0-31, b in 32-63
  x = row_sum(swap_add16(x, x));
  sa = lane_value(x, 0);
  sb = lane_value(x, 32);
}

// Wave sums of six values at once, as wave-uniform results.
__device__ __forceinline__ void wave_sum6(const float (&v)[6], float (&r)[6]) {
  const float p0 = swap_add32(v[0], v[1]);  // v0 | v1 by wave half
  const float p1 = swap_add32(v[2], v[3]);  // v2 | v3
  const float p2 = swap_add32(v[4], v[5]);  // v4 | v5
  const float y0 = row_sum(swap_add16(p0, p1));  // rows: v0, v2, v1, v3
  const float y1 = row_sum(swap_add16(p2, p2));  // rows: v4, v4, v5, v5
  r[0] = lane_value(y0, 0);
  r[1] = lane_value(y0, 32);
  r[2] = lane_value(y0, 16);
  r[3] = lane_value(y0, 48);
  r[4] = lane_value(y1, 0);
  r[5] = lane_value(y1, 32);
}

__device__ __forceinline__ float softplusf(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoidf(float x) {
  const float e = expf(-fabsf(x));
  return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *a, *b, *A_log, *dt_bias, *state_pool, *dstate;
  const int64_t *cu, *cache_indices;
  const int32_t* chunk_off;
  float *dq, *dk, *dv, *da, *db, *dA_log, *ddt_bias, *dstate0;
  float* ck;      // [chunk][HV][dv][dk]: state before the chunk's first token
  float* part;    // [dv / 16][N][HV][2 dk + 2]: dqh, dkh, dalpha, dbeta per row block
  float* dal;     // [N][HV]: dalpha * dalpha/dA_log per token
  float* qn;      // [N][H][dk]: q / |q|
  float* kn;      // [N][H][dk]: k / |k|
  float* ab;      // [N][HV][2]: alpha, beta
  int64_t N;
  int B, H, HV, DV;
  float eps;
  int bf16;
};

// One wave per (token, q/k head).
template <int DK>
__global__ __launch_bounds__(256) void bwd_token_kernel(BwdArgs A) {
  constexpr int E = DK / 64;
  const int l = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= A.N * A.H) return;
  const int64_t t = wid / A.H;
  const int h = (int)(wid % A.H);
  float qe[E], ke[E], sq = 0.f, sk = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qe[e] = ldx(A.q, (t * A.H + h) * DK + 64 * e + l, A.bf16);
    ke[e] = ldx(A.k, (t * A.H + h) * DK + 64 * e + l, A.bf16);
    sq += qe[e] * qe[e];
    sk += ke[e] * ke[e];
  }
  const float rq = 1.f / sqrtf(wave_sum(sq) + A.eps), rk = 1.f / sqrtf(wave_sum(sk) + A.eps);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    A.qn[(t * A.H + h) * DK + 64 * e + l] = qe[e] * rq;
    A.kn[(t * A.H + h) * DK + 64 * e + l] = ke[e] * rk;
  }
  const int grp = A.HV / A.H;
  for (int j = l; j < grp; j += 64) {
    const int hv = h * grp + j;
    const float xg = A.a[t * A.HV + hv] + A.dt_bias[hv];
    float2 ab;
    ab.x = expf(-expf(A.A_log[hv]) * softplusf(xg));
    ab.y = sigmoidf(A.b[t * A.HV + hv]);
    *reinterpret_cast<float2*>(A.ab + (t * A.HV + hv) * 2) = ab;
  }
}

template <int DK>
struct Token {
  float qh[DK / 64], kh[DK / 64];
  float alpha, beta;
  float v[kRowsPerWave];
};

// Token t's inputs for this lane's elements and this wave's rows (all precomputed).
template <int DK>
__device__ __forceinline__ void fetch(const BwdArgs& A, int64_t t, int h, int hv, int row0, int l,
                                      Token<DK>& x) {
  constexpr int E = DK / 64;
  const float* qp = A.qn + (t * A.H + h) * DK + l;
  const float* kp = A.kn + (t * A.H + h) * DK + l;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x.qh[e] = qp[64 * e];
    x.kh[e] = kp[64 * e];
  }
  const float2 ab = *reinterpret_cast<const float2*>(A.ab + (t * A.HV + hv) * 2);
  x.alpha = ab.x;
  x.beta = ab.y;
  ld_rows(A.v, (t * A.HV + hv) * (int64_t)A.DV + row0, A.bf16, x.v);
}

// The inputs of a group of SUB consecutive tokens, staged in LDS once per row workgroup
// (every wave of the workgroup needs the same q and k rows and gates).
template <int DK, int SUB>
struct TokBuf {
  alignas(16) float qh[SUB][DK];
  float kh[SUB][DK];
  float ab[SUB][2];             // alpha, beta
  float v[SUB][kBwdRows];       // the workgroup's rows of v
  float dout[SUB][kBwdRows];    // ... and of dout
};

// Token i of the staged group, for this lane's elements and the rows rl, rl + 1 of the
// workgroup's block.
template <int DK, int SUB>
__device__ __forceinline__ void from_lds(const TokBuf<DK, SUB>& b, int i, int rl, int l,
                                         Token<DK>& x) {
  constexpr int E = DK / 64;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x.qh[e] = b.qh[i][64 * e + l];
    x.kh[e] = b.kh[i][64 * e + l];
  }
  const float2 ab = *reinterpret_cast<const float2*>(&b.ab[i][0]);
  x.alpha = ab.x;
  x.beta = ab.y;
  const float2 vv = *reinterpret_cast<const float2*>(&b.v[i][rl]);
  x.v[0] = vv.x;
  x.v[1] = vv.y;
}

// One token's step on this wave's rows: s <- alpha s - alpha beta (s kh) kh + beta v kh.
template <int DK>
__device__ __forceinline__ void step(const Token<DK>& x, float (&s)[kRowsPerWave][DK / 64]) {
  constexpr int E = DK / 64;
  static_assert(kRowsPerWave == 2, "the two rows' sums are reduced together");
  float p[kRowsPerWave] = {}, sk[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) p[j] += s[j][e] * x.kh[e];
  wave_sum2(p[0], p[1], sk[0], sk[1]);
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const float c = x.beta * (x.v[j] - x.alpha * sk[j]);
#pragma unroll
    for (int e = 0; e < E; ++e) s[j][e] = x.alpha * s[j][e] + c * x.kh[e];
  }
}

template <int DK>
__global__ __launch_bounds__(kRowThreads) void bwd_rows_kernel(BwdArgs A) {
  constexpr int E = DK / 64;
  constexpr int SUB = kSub<DK>;
  constexpr int NF = 2 * DK + 2;  // fields per token of a partial: dqh, dkh, dalpha, dbeta
  __shared__ float part[kRowWaves][SUB][NF];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup id -> (request, value head, row block): the row blocks of one (request, head)
  // get consecutive ids of one XCD (ids are dealt to the 8 XCDs in turn), so they run
  // together and read the same token rows through that XCD's L2.
  const int nrb = A.DV / kBwdRows;
  const int64_t x = blockIdx.x, k8 = x >> 3;
  const int rb = (int)(k8 % nrb);
  const int64_t p = k8 / nrb * 8 + (x & 7);
  if (p >= (int64_t)A.B * A.HV) return;  // the pair count rounded up to 8
  const int bq = (int)(p / A.HV), hv = (int)(p % A.HV);
  const int h = hv / (A.HV / A.H);
  const int row0 = rb * kBwdRows + kRowsPerWave * w;  // this wave's first row
  const int64_t t0 = A.cu[bq], L = A.cu[bq + 1] - t0;
  const int64_t slot = A.cache_indices[bq];
  const int64_t cbase = A.chunk_off[bq];
  auto state_at = [&](const float* base, int j, int e) {
    return base[((int64_t)(row0 + j)) * DK + 64 * e + l];
  };
  const float* S0 = A.state_pool + (slot * A.HV + hv) * (int64_t)A.DV * DK;
  const float* DS = A.dstate + ((int64_t)bq * A.HV + hv) * A.DV * DK;
  float* DS0 = A.dstate0 + ((int64_t)bq * A.HV + hv) * A.DV * DK;
  auto ck_at = [&](int64_t c) { return A.ck + ((cbase + c) * A.HV + hv) * (int64_t)A.DV * DK; };

  auto tok = [&](int64_t t) { return t0 + min(t, L - 1); };  // clamped into the request

  // Token inputs go through an LDS buffer of SUB tokens, loaded cooperatively: every thread
  // loads one 16-byte piece of the q, k rows and one gate, v or dout value of the next
  // group into registers while the current group is used, and stores them after the
  // barrier that ends the current group's use.
  __shared__ TokBuf<DK, SUB> tb;
  constexpr int P4 = SUB * DK / 4;  // 16-byte pieces of the group's q rows (and of its k rows)
  struct Pf {
    float4 qk;
    float sm;
  };
  const int rl = kRowsPerWave * w;  // this wave's first row within the block
  auto tok_load = [&](int64_t g0, bool with_q, Pf& r) {
    if (tid < 2 * P4) {
      const int which = tid / P4, rem = tid % P4, i = rem / (DK / 4), c4 = rem % (DK / 4);
      if (which == 1 || with_q)
        r.qk = *reinterpret_cast<const float4*>((which ? A.kn : A.qn) +
                                                 (tok(g0 + i) * A.H + h) * DK + 4 * c4);
    }
    if (tid < 2 * SUB) {
      const int i = tid >> 1;
      r.sm = A.ab[(tok(g0 + i) * A.HV + hv) * 2 + (tid & 1)];
    } else if (tid < 2 * SUB + SUB * kBwdRows) {
      const int x = tid - 2 * SUB, i = x / kBwdRows, row = x % kBwdRows;
      r.sm = ldx(A.v, (tok(g0 + i) * A.HV + hv) * (int64_t)A.DV + rb * kBwdRows + row, A.bf16);
    } else if (with_q && tid < 2 * SUB + 2 * SUB * kBwdRows) {
      const int x = tid - 2 * SUB - SUB * kBwdRows, i = x / kBwdRows, row = x % kBwdRows;
      r.sm = ldx(A.dout, (tok(g0 + i) * A.HV + hv) * (int64_t)A.DV + rb * kBwdRows + row,
                 A.bf16);
    }
  };
  auto tok_store = [&](const Pf& r, bool with_q) {
    if (tid < 2 * P4) {
      const int which = tid / P4, rem = tid % P4, i = rem / (DK / 4), c4 = rem % (DK / 4);
      if (which == 1)
        *reinterpret_cast<float4*>(&tb.kh[i][4 * c4]) = r.qk;
      else if (with_q)
        *reinterpret_cast<float4*>(&tb.qh[i][4 * c4]) = r.qk;
    }
    if (tid < 2 * SUB) {
      tb.ab[tid >> 1][tid & 1] = r.sm;
    } else if (tid < 2 * SUB + SUB * kBwdRows) {
      const int x = tid - 2 * SUB;
      tb.v[x / kBwdRows][x % kBwdRows] = r.sm;
    } else if (with_q && tid < 2 * SUB + 2 * SUB * kBwdRows) {
      const int x = tid - 2 * SUB - SUB * kBwdRows;
      tb.dout[x / kBwdRows][x % kBwdRows] = r.sm;
    }
  };
  Pf pf;
  pf.qk = float4{0.f, 0.f, 0.f, 0.f};
  pf.sm = 0.f;

  // ---- forward sweep: checkpoint every kCk tokens, groups of SUB tokens
  float s[kRowsPerWave][E];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) s[j][e] = state_at(S0, j, e);
  if (L > 0) {
    tok_load(0, false, pf);
    tok_store(pf, false);
  }
  __syncthreads();
  for (int64_t g0 = 0; g0 < L; g0 += SUB) {
    const bool more = g0 + SUB < L;
    if (more) tok_load(g0 + SUB, false, pf);
    if (g0 % kCk == 0) {
      float* c = ck_at(g0 / kCk);
#pragma unroll
      for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) c[((int64_t)(row0 + j)) * DK + 64 * e + l] = s[j][e];
    }
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      if (g0 + i < L) {
        Token<DK> x;
        from_lds(tb, i, rl, l, x);
        step<DK>(x, s);
      }
    }
    __syncthreads();  // every wave is done with this group
    if (more) tok_store(pf, false);
    __syncthreads();  // the next group is staged
  }
  // the checkpoints are read back by the same lanes that wrote them: no barrier needed

  // ---- reverse sweep
  float D[kRowsPerWave][E];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) D[j][e] = state_at(DS, j, e);
  const int64_t nsub = (L + SUB - 1) / SUB;
  float cpr[kRowsPerWave][E];  // the checkpoint the next sub-chunk starts from
  auto load_ck = [&](int64_t u) {
    const float* cp = ck_at(u * SUB / kCk);
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) cpr[j][e] = cp[((int64_t)(row0 + j)) * DK + 64 * e + l];
  };
  if (nsub > 0) {
    load_ck(nsub - 1);
    tok_load((nsub - 1) * SUB, true, pf);
    tok_store(pf, true);  // the forward sweep ended with a barrier
  }
  __syncthreads();
  for (int64_t u = nsub - 1; u >= 0; --u) {
    const int64_t u_lo = u * SUB, u_hi = min(u_lo + SUB, L);
    const int64_t c = u_lo / kCk;
    if (u > 0) tok_load(u_lo - SUB, true, pf);  // the next sub-chunk's inputs
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) s[j][e] = cpr[j][e];
    // recompute from the checkpoint to the sub-chunk (sub-chunks shorter than kCk only),
    // with the inputs from global memory one token ahead
    if (c * kCk < u_lo) {
      Token<DK> pk, pn;
      fetch<DK>(A, t0 + c * kCk, h, hv, row0, l, pk);
      for (int64_t t = c * kCk; t < u_lo; ++t) {
        fetch<DK>(A, t0 + t + 1, h, hv, row0, l, pn);  // t + 1 <= u_lo < L
        step<DK>(pk, s);
        pk = pn;
      }
    }
    float sb[SUB][kRowsPerWave][E];  // S_{t-1} for the sub-chunk's tokens
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      if (u_lo + i < u_hi) {
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
          for (int e = 0; e < E; ++e) sb[i][j][e] = s[j][e];
        Token<DK> x;
        from_lds(tb, i, rl, l, x);
        step<DK>(x, s);
      }
    }
    if (u > 0) load_ck(u - 1);
    // s is now the state after the sub-chunk's last token. Walk back from that token.
#pragma unroll
    for (int i = SUB - 1; i >= 0; --i) {
      if (u_lo + i < u_hi) {  // (uniform)
        Token<DK> tk;
        from_lds(tb, i, rl, l, tk);
        const float2 dO2 = *reinterpret_cast<const float2*>(&tb.dout[i][rl]);
        const float dO[kRowsPerWave] = {dO2.x, dO2.y};
        const int64_t t = t0 + u_lo + i;
        // S_t: the state before the next token, or the sub-chunk's end state
        const bool last = (i == SUB - 1) || (u_lo + i + 1 >= u_hi);
        float dqh[E] = {}, dkh[E] = {};
        float dal = 0.f, dbe = 0.f;
        float dvr[kRowsPerWave];
        // the three row dot products of both rows, reduced together:
        // (S_{t-1} kh, D kh, D . S_{t-1})
        float dots[6] = {}, sums[6];
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float st = last ? s[j][e] : sb[i < SUB - 1 ? i + 1 : i][j][e];
            D[j][e] += dO[j] * tk.qh[e];
            dqh[e] += dO[j] * st;
            dots[3 * j] += sb[i][j][e] * tk.kh[e];
            dots[3 * j + 1] += D[j][e] * tk.kh[e];
            dots[3 * j + 2] += D[j][e] * sb[i][j][e];
          }
        }
        wave_sum6(dots, sums);
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j) {
          const float Spk = sums[3 * j], Dk = sums[3 * j + 1], Ds = sums[3 * j + 2];
          dvr[j] = tk.beta * Dk;
          dbe += Dk * (tk.v[j] - tk.alpha * Spk);
          dal += Ds - tk.beta * Dk * Spk;
          const float cS = -tk.alpha * tk.beta * Spk, cD = -tk.alpha * tk.beta * Dk;
          const float cV = tk.beta * tk.v[j], cK = tk.alpha * tk.beta * Dk;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            dkh[e] += cS * D[j][e] + cD * sb[i][j][e] + cV * D[j][e];
            D[j][e] = tk.alpha * D[j][e] - cK * tk.kh[e];
          }
        }
        if (l == 0)
          *reinterpret_cast<float2*>(A.dv + (t * A.HV + hv) * (int64_t)A.DV + row0) =
              make_float2(dvr[0], dvr[1]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          part[w][i][64 * e + l] = dqh[e];
          part[w][i][DK + 64 * e + l] = dkh[e];
        }
        if (l == 0) {
          part[w][i][2 * DK] = dal;
          part[w][i][2 * DK + 1] = dbe;
        }
      }
    }
    __syncthreads();  // every wave is done with the staged inputs and has written its sums
    if (u > 0) tok_store(pf, true);
    // this row block's partial sums for the sub-chunk's tokens
    const int nt = (int)(u_hi - u_lo);
    for (int idx = tid; idx < nt * NF; idx += kRowThreads) {
      const int i = idx / NF, f = idx % NF;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < kRowWaves; ++ww) v += part[ww][i][f];
      A.part[(((int64_t)rb * A.N + t0 + u_lo + i) * A.HV + hv) * NF + f] = v;
    }
    __syncthreads();
  }
  // gradient of the request's initial state
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) DS0[((int64_t)(row0 + j)) * DK + 64 * e + l] = D[j][e];
}

// One wave per (token, q/k head).
template <int DK>
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs A) {
  constexpr int E = DK / 64;
  constexpr int NF = 2 * DK + 2;
  const int l = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= A.N * A.H) return;
  const int64_t t = wid / A.H;
  const int h = (int)(wid % A.H);
  const int grp = A.HV / A.H, nrb = A.DV / kBwdRows;
  float dqh[E] = {}, dkh[E] = {};
  for (int j = 0; j < grp; ++j) {
    const int hv = h * grp + j;
    float dal = 0.f, dbe = 0.f;
    for (int rb = 0; rb < nrb; ++rb) {
      const float* P = A.part + (((int64_t)rb * A.N + t) * A.HV + hv) * NF;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dqh[e] += P[64 * e + l];
        dkh[e] += P[DK + 64 * e + l];
      }
      dal += P[2 * DK];
      dbe += P[2 * DK + 1];
    }
    if (l == 0) {
      const float xg = A.a[t * A.HV + hv] + A.dt_bias[hv];
      const float Aexp = expf(A.A_log[hv]);
      const float sp = softplusf(xg);
      const float alpha = expf(-Aexp * sp);
      const float beta = sigmoidf(A.b[t * A.HV + hv]);
      A.da[t * A.HV + hv] = dal * (-alpha * Aexp * sigmoidf(xg));
      A.dal[t * A.HV + hv] = dal * (-alpha * Aexp * sp);
      A.db[t * A.HV + hv] = dbe * beta * (1.f - beta);
    }
  }
  // L2 norm: d(x / n)/dx applied to the summed gradient of the normalised vector
  float qe[E], ke[E], sq = 0.f, sk = 0.f, qd = 0.f, kd = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qe[e] = ldx(A.q, (t * A.H + h) * DK + 64 * e + l, A.bf16);
    ke[e] = ldx(A.k, (t * A.H + h) * DK + 64 * e + l, A.bf16);
    sq += qe[e] * qe[e];
    sk += ke[e] * ke[e];
    qd += qe[e] * dqh[e];
    kd += ke[e] * dkh[e];
  }
  const float nq = sqrtf(wave_sum(sq) + A.eps), nk = sqrtf(wave_sum(sk) + A.eps);
  qd = wave_sum(qd);
  kd = wave_sum(kd);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    A.dq[(t * A.H + h) * DK + 64 * e + l] = dqh[e] / nq - qe[e] * qd / (nq * nq * nq);
    A.dk[(t * A.H + h) * DK + 64 * e + l] = dkh[e] / nk - ke[e] * kd / (nk * nk * nk);
  }
}

// One workgroup per value head: sums over every token, in a fixed order.
__global__ __launch_bounds__(256) void bwd_gates_kernel(BwdArgs A) {
  __shared__ float s1[256], s2[256];
  const int hv = blockIdx.x, tid = threadIdx.x;
  float x1 = 0.f, x2 = 0.f;
  for (int64_t t = tid; t < A.N; t += 256) {
    x1 += A.da[t * A.HV + hv];
    x2 += A.dal[t * A.HV + hv];
  }
  s1[tid] = x1;
  s2[tid] = x2;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      s1[tid] += s1[tid + o];
      s2[tid] += s2[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    A.ddt_bias[hv] = s1[0];
    A.dA_log[hv] = s2[0];
  }
}

}  // namespace

BwdLayout bwd_layout_for(const Shape& s) {
  BwdLayout L;
  L.max_chunks = s.N / kCk + s.B;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  L.chunk_off = take(sizeof(int32_t) * (size_t)(s.B + 1));
  L.chunk_seq = take(sizeof(int32_t) * (size_t)L.max_chunks);
  L.ck = take(sizeof(float) * (size_t)L.max_chunks * s.HV * s.dv * s.dk);
  L.part = take(sizeof(float) * (size_t)(s.dv / kBwdRows) * s.N * s.HV * (2 * s.dk + 2));
  L.dal = take(sizeof(float) * (size_t)s.N * s.HV);
  L.qn = take(sizeof(float) * (size_t)s.N * s.H * s.dk);
  L.kn = take(sizeof(float) * (size_t)s.N * s.H * s.dk);
  L.ab = take(sizeof(float) * 2 * (size_t)s.N * s.HV);
  L.total = off;
  return L;
}

bool bwd_grids_fit(const Shape& s) {
  const int64_t rows = (s.B * s.HV + 7) / 8 * 8 * (s.dv / kBwdRows);
  const int64_t fin = (s.N * s.H + 3) / 4;
  return rows * kRowThreads <= 0xFFFFFFFFLL && fin * 256 <= 0xFFFFFFFFLL && s.HV <= 0x7FFFFFFF;
}

hipError_t launch_backward(const Shape& s, const BwdLayout& L, char* ws, const void* q,
                           const void* k, const void* v, const float* a, const float* b,
                           const float* A_log, const float* dt_bias, const float* state_pool,
                           const int64_t* cache_indices, const int64_t* cu_seqlens,
                           const void* dout, const float* dstate, float* dq, float* dk,
                           float* dv, float* da, float* db, float* dA_log, float* ddt_bias,
                           float* dstate0, hipStream_t st) {
  int32_t* chunk_off = (int32_t*)(ws + L.chunk_off);
  Shape sp = s;
  sp.C = kCk;
  hipError_t e = launch_plan(cu_seqlens, sp, chunk_off, (int32_t*)(ws + L.chunk_seq),
                             L.max_chunks, st);
  if (e != hipSuccess) return e;
  BwdArgs A;
  A.q = q;
  A.k = k;
  A.v = v;
  A.dout = dout;
  A.a = a;
  A.b = b;
  A.A_log = A_log;
  A.dt_bias = dt_bias;
  A.state_pool = state_pool;
  A.dstate = dstate;
  A.cu = cu_seqlens;
  A.cache_indices = cache_indices;
  A.chunk_off = chunk_off;
  A.dq = dq;
  A.dk = dk;
  A.dv = dv;
  A.da = da;
  A.db = db;
  A.dA_log = dA_log;
  A.ddt_bias = ddt_bias;
  A.dstate0 = dstate0;
  A.ck = (float*)(ws + L.ck);
  A.part = (float*)(ws + L.part);
  A.dal = (float*)(ws + L.dal);
  A.qn = (float*)(ws + L.qn);
  A.kn = (float*)(ws + L.kn);
  A.ab = (float*)(ws + L.ab);
  A.N = s.N;
  A.B = (int)s.B;
  A.H = s.H;
  A.HV = s.HV;
  A.DV = s.dv;
  A.eps = kNormEps;
  A.bf16 = s.bf16 ? 1 : 0;
  const dim3 rows((unsigned)((s.B * s.HV + 7) / 8 * 8 * (s.dv / kBwdRows))),
      fin((unsigned)((s.N * s.H + 3) / 4));
#define GDN_BWD_CASE(DKv)                                                              \
  if (s.dk == DKv) {                                                                   \
    if (s.N > 0) hipLaunchKernelGGL((bwd_token_kernel<DKv>), fin, dim3(256), 0, st, A); \
    hipLaunchKernelGGL((bwd_rows_kernel<DKv>), rows, dim3(kRowThreads), 0, st, A);     \
    if ((e = hipGetLastError()) != hipSuccess) return e;                               \
    if (s.N > 0) hipLaunchKernelGGL((bwd_finish_kernel<DKv>), fin, dim3(256), 0, st, A); \
  }
  GDN_BWD_CASE(64)
  GDN_BWD_CASE(128)
  GDN_BWD_CASE(256)
#undef GDN_BWD_CASE
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_gates_kernel, dim3((unsigned)s.HV), dim3(256), 0, st, A);
  return hipGetLastError();
}

}  // namespace gdn
