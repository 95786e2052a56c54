// Sequential state pass on matrix cores (bf16 inputs).
//
// Per chunk, in row convention (pymllm gdn_chunkwise page, Algorithm steps 2-3; "Simple
// math to speed up GDN prefill", Reminder, chunkwise transition with decorated S->, W<-,
// K->):
//   U     = U~ - W<- S^T
//   O     = diag(e^G) Qh S^T + A_qk U,  Qh = diag(r_q) Q              (to out)
//   S^T  <- e^{G_n} S^T + K^T diag(e^{G_n - G} r_k) U
// with r_q, r_k the inverse L2 norms of the rows of q and k and
// A_qk = Gamma o tril0(diag(r_q) Q K^T diag(r_k)), Gamma_ri = e^{G_r - G_i}, which the
// chunk-prep kernel has already formed together with the row scales (they depend on no
// state). Chunks of a request are processed in order (pymllm page: the propagation
// between chunks remains sequential over ceil(T/C) steps).
//
// Work split: one workgroup per (request, value head, 16 state rows); its DS wavefronts
// split dk, wave hs owning dk steps hs * NOWN .. (hs + 1) * NOWN - 1 of the 16 rows of
// S^T, in fp32 registers for the whole request. Every operand comes straight from
// global memory into MFMA operand registers, in the fragment orders the prep kernel
// wrote (one contiguous 1 KiB piece per fragment); each register set is reloaded
// with the next chunk's data right after its last use, so the loads have about one
// chunk of time to land. LDS carries only the partial sums over dk (double-buffered by
// chunk parity): P = W<- S^T for all rows, which every wave completes into U itself,
// and Q S^T for the rows another wave finishes. One barrier per chunk; none when one
// wave holds all of dk.
//
// Matrix-core operands: W<- and S in fp16 for P = W<- S^T; normalised q and S in fp16
// for Qh S^T; raw bf16 k with diag(e^{G_n-G} r_k) U as bf16 hi + lo for the update;
// A_qk and U in fp16 for A_qk U.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;

template <int DS>
struct StateSmem {
  f32x4 partP[2][DS][4][64];  // partial W<- S^T: chunk parity, dk owner, row tile, lane
  f32x4 partO[2][DS][4][64];  // partial Q S^T
};

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 h;
  h[0] = (__bf16)x[0];
  h[1] = (__bf16)x[1];
  h[2] = (__bf16)x[2];
  h[3] = (__bf16)x[3];
  return h;
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 h) {
  f32x4 r;
  r[0] = (float)h[0];
  r[1] = (float)h[1];
  r[2] = (float)h[2];
  r[3] = (float)h[3];
  return r;
}
__device__ __forceinline__ bf16x8 cat_bf(bf16x4 a, bf16x4 b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

template <int DK, int DS>
__global__ __launch_bounds__(64 * DS) void mfma_state_kernel(
    const _Float16* __restrict__ Qf, const uint16_t* __restrict__ Kf,
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const double* __restrict__ gcum,
    const _Float16* __restrict__ W, const _Float16* __restrict__ Ut,
    const float* __restrict__ kdws, const _Float16* __restrict__ Aqk,
    const float* __restrict__ egws, int B, int H, int HV, int DV,
    float* __restrict__ state_pool, uint16_t* __restrict__ out) {
  constexpr int NKS = DK / 32;    // 32-wide dk steps
  constexpr int NOWN = NKS / DS;  // dk steps per wave
  constexpr int NOR = 4 / DS;     // output row tiles per wave: I = hs + DS * r
  __shared__ StateSmem<DS> sm;

  // Blocks of the same (request, head) share blockIdx.x mod 8, so they run on one
  // XCD and re-read q, k and W<- from its L2.
  const int nvb = DV / 16;
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int ct = (int)(rest % nvb);  // column tile: state rows 16 ct .. 16 ct + 15
  const int64_t p = (rest / nvb) * 8 + (x & 7);
  if (p >= (int64_t)B * HV) return;
  const int seq = (int)(p / HV), hv = (int)(p % HV);
  const int64_t L = cu[seq + 1] - cu[seq];
  if (L <= 0) return;
  const int h = hv / (HV / H);
  const int64_t slot = cache_indices[seq];
  const int tid = threadIdx.x, hs = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int nch = (int)((L + C - 1) / C);
  const int64_t cbase = chunk_off[seq];
  const int64_t tseq = cu[seq];
  const int64_t tend = cu[seq + 1];

  // ---- resident state: S^T tiles of the owned dk steps sp' = hs * NOWN + sp
  float* Sg = state_pool + ((slot * HV + hv) * (int64_t)DV + 16 * ct + m) * DK;
  f32x4 S[NOWN][2];
#pragma unroll
  for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      S[sp][tt] = *reinterpret_cast<const f32x4*>(Sg + 32 * (hs * NOWN + sp) + 16 * tt + 4 * g);

  // ---- operand registers of one chunk
  u32x4 wf[4][NOWN], qf[4][NOWN];  // W<- and Qh fragments: row tile, own dk step
  u32x4 kf[NOWN][2][2];            // k^T fragments: own dk step, 16-dk half, token step
  u32x2 uf[4];                     // U~ (fp16 D tiles) of column tile ct, row tile
  u32x4 af[NOR][2];                // A_qk fragments of the own output row tiles
  f32x4 kdv[4];                    // e^{G_n - G} r_k of rows 16I + 4g + i
  f32x4 egv[NOR];                  // e^G of the own output rows
  double gn;                       // G_n (the gate pass pads G with zero log-decay)

  auto pair_of = [&](int cl) { return (cbase + cl) * HV + hv; };
  auto load_wq = [&](int cl) {
    const int64_t pr = pair_of(cl);
    const _Float16* wb = W + pr * C * DK;
    const _Float16* qb = Qf + ((cbase + cl) * H + h) * (int64_t)(C * DK);
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp) {
        const int spg = hs * NOWN + sp;
        wf[I][sp] = *reinterpret_cast<const u32x4*>(wb + ((I * NKS + spg) * 64 + l) * 8);
        qf[I][sp] = *reinterpret_cast<const u32x4*>(qb + ((I * NKS + spg) * 64 + l) * 8);
      }
  };
  auto load_ukd = [&](int cl) {
    const int64_t pr = pair_of(cl);
    const _Float16* ub = Ut + pr * C * DV + (ct * 4 * 64 + l) * 4;
#pragma unroll
    for (int I = 0; I < 4; ++I) uf[I] = *reinterpret_cast<const u32x2*>(ub + I * 64 * 4);
#pragma unroll
    for (int I = 0; I < 4; ++I)
      kdv[I] = *reinterpret_cast<const f32x4*>(kdws + pr * C + 16 * I + 4 * g);
  };
  auto load_k = [&](int cl) {
    const int64_t pr = pair_of(cl);
    const uint16_t* kb = Kf + ((cbase + cl) * H + h) * (int64_t)(C * DK);
#pragma unroll
    for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          kf[sp][tt][s] = *reinterpret_cast<const u32x4*>(
              kb + ((((hs * NOWN + sp) * 2 + tt) * 2 + s) * 64 + l) * 8);
    gn = gcum[pr * C + C - 1];
  };
  auto load_out = [&](int cl) {
    const int64_t pr = pair_of(cl);
#pragma unroll
    for (int r = 0; r < NOR; ++r) {
      const int I = hs + DS * r;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        af[r][s] = *reinterpret_cast<const u32x4*>(Aqk + pr * C * C + ((I * 2 + s) * 64 + l) * 8);
      egv[r] = *reinterpret_cast<const f32x4*>(egws + pr * C + 16 * I + 4 * g);
    }
  };
  load_wq(0);
  load_ukd(0);
  load_k(0);
  load_out(0);

  // Each register set is reloaded with chunk cl + 1 right after its last use in chunk
  // cl (chunk nch - 1 is reloaded on the last step: in bounds, and no branch).
  for (int cl = 0; cl < nch; ++cl) {
    const int buf = cl & 1;
    const int nx = min(cl + 1, nch - 1);
    const int64_t t0 = tseq + (int64_t)cl * C;
    const int n = (int)min((int64_t)C, tend - t0);

    // ---- partial P = W<- S^T and O1 = Qh S^T over the owned dk steps
    half8 s16[NOWN];
#pragma unroll
    for (int sp = 0; sp < NOWN; ++sp) s16[sp] = cat(to_half4(S[sp][0]), to_half4(S[sp][1]));
    f32x4 pp[4], po[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      pp[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      po[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp) {
        pp[I] = mma_f16(half8_from_u32x4(wf[I][sp]), s16[sp], pp[I]);
        po[I] = mma_f16(half8_from_u32x4(qf[I][sp]), s16[sp], po[I]);
      }
    }
    load_wq(nx);
    if (DS > 1) {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        sm.partP[buf][hs][I][l] = pp[I];
        if (I % DS != hs) sm.partO[buf][hs][I][l] = po[I];
      }
      lds_barrier();
    }

    // ---- U = U~ - P for all rows (every wave of the block forms the same U)
    f32x4 U[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 pt = pp[I];
#pragma unroll
      for (int o = 0; o < DS; ++o)
        if (o != hs) pt += sm.partP[buf][o][I][l];
      const half4 ut = __builtin_bit_cast(half4, uf[I]);
#pragma unroll
      for (int i = 0; i < 4; ++i) U[I][i] = (float)ut[i] - pt[i];
    }
    // U'' = diag(e^{G_n - G} r_k) U as the bf16 hi + lo B operand of the update
    bf16x8 bh[2], bl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 ua = U[2 * s] * kdv[2 * s], ub = U[2 * s + 1] * kdv[2 * s + 1];
      const bf16x4 ha = to_bf16x4(ua), hb = to_bf16x4(ub);
      bh[s] = cat_bf(ha, hb);
      bl[s] = cat_bf(to_bf16x4(ua - to_f32x4(ha)), to_bf16x4(ub - to_f32x4(hb)));
    }
    load_ukd(nx);

    // ---- S^T <- e^{G_n} S^T + K^T U'' on the owned dk steps
    const float egn = expf((float)gn);
#pragma unroll
    for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 acc = S[sp][tt] * egn;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 a = bf16x8_from_u32x4(kf[sp][tt][s]);
          acc = mma_bf16(a, bh[s], acc);
          acc = mma_bf16(a, bl[s], acc);
        }
        S[sp][tt] = acc;
      }
    load_k(nx);

    // ---- O for the own row tiles: e^G (Qh S^T) + A_qk U
#pragma unroll
    for (int r = 0; r < NOR; ++r) {
      const int I = hs + DS * r;
      f32x4 o1 = po[0];  // po[I], selected without indexing registers at run time
#pragma unroll
      for (int I2 = 1; I2 < 4; ++I2)
        if (I2 == I) o1 = po[I2];
#pragma unroll
      for (int o = 0; o < DS; ++o)
        if (o != hs) o1 += sm.partO[buf][o][I][l];
      f32x4 AU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s <= (I >> 1))
          AU = mma_f16(half8_from_u32x4(af[r][s]),
                       cat(to_half4(U[2 * s]), to_half4(U[2 * s + 1])), AU);
      const bf16x4 ov = to_bf16x4(egv[r] * o1 + AU);  // round to nearest even
      __bf16* ob = reinterpret_cast<__bf16*>(out) +
                   ((t0 + 16 * I + 4 * g) * HV + hv) * (int64_t)DV + 16 * ct + m;
      if (n == C) {  // full chunk: no per-row test
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i * (int64_t)HV * DV] = ov[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * I + 4 * g + i < n) ob[i * (int64_t)HV * DV] = ov[i];
      }
    }
    load_out(nx);
  }

  // ---- write the state back in place
#pragma unroll
  for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      *reinterpret_cast<f32x4*>(Sg + 32 * (hs * NOWN + sp) + 16 * tt + 4 * g) = S[sp][tt];
}

template <int DK, int DS>
hipError_t launch_state_t(const void* qf, const void* kf, const int64_t* cu, const int64_t* idx,
                          const int32_t* off, const double* gcum, const _Float16* w,
                          const _Float16* u, const float* kd, const _Float16* aqk,
                          const float* eg, const Shape& s, float* pool, void* out,
                          hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8;
  const int64_t blocks = pairs8 * 8 * (s.dv / 16);
  hipLaunchKernelGGL((mfma_state_kernel<DK, DS>), dim3((unsigned)blocks), dim3(64 * DS), 0, st,
                     (const _Float16*)qf, (const uint16_t*)kf, cu, idx, off, gcum, w, u, kd, aqk,
                     eg, (int)s.B, s.H, s.HV, s.dv, pool, (uint16_t*)out);
  return hipGetLastError();
}

// Waves per workgroup (dk split): each wave holds 64 dk (two 32-wide steps) of its 16
// state rows, or 32 when that is needed to give every SIMD of the 256 compute units a
// wave (B * HV * dv / 16 workgroups in all). Splitting further costs more in exchanged
// partial sums than the extra waves win back in hidden latency.
int choose_ds(const Shape& s) {
  const int64_t tiles = s.B * s.HV * (s.dv / 16);
  const int ds = s.dk / 64;
  if (tiles * ds < 1024 && ds < 4) return 2 * ds;
  return ds;
}

}  // namespace

hipError_t launch_mfma_state(const void* qf, const void* kf, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const double* gcum, const void* w, const void* u, const float* kd,
                             const void* aqk, const float* eg, const Shape& s,
                             float* state_pool, void* out, hipStream_t st) {
  const _Float16* W = (const _Float16*)w;
  const _Float16* U = (const _Float16*)u;
  const int ds = choose_ds(s);
#define GDN_STATE_CASE(DKv, DSv)                                                              \
  if (s.dk == DKv && ds == DSv)                                                               \
    return launch_state_t<DKv, DSv>(qf, kf, cu_seqlens, cache_indices, chunk_off, gcum, W, U,  \
                                    kd, (const _Float16*)aqk, eg, s, state_pool, out, st);
  GDN_STATE_CASE(64, 1)
  GDN_STATE_CASE(64, 2)
  GDN_STATE_CASE(128, 2)
  GDN_STATE_CASE(128, 4)
  GDN_STATE_CASE(256, 4)
#undef GDN_STATE_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
