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
// Work split: one workgroup per (request, value head, NC x 16 state rows), with two
// roles.
//   * DS state waves split dk: wave hs holds dk steps hs * NOWN .. of the NC x 16 rows of
//     S^T in fp32 registers for the whole request and runs only the chain that carries
//     the state from chunk to chunk: P = W<- S^T over its dk slice, the exchange of those
//     partial sums (LDS, double-buffered), U, and the update of its slice. Each W<- and
//     k^T fragment it loads serves all NC column tiles, which halves the bytes every
//     compute unit requests per chunk at NC = 2.
//   * NO output waves form O for the previous chunk from the fp16 copies of S^T and U
//     that the state waves leave in LDS (triple- and double-buffered), so the output
//     products and stores stay off that chain; wave ow takes row tiles NRO ow .. of all
//     NC column tiles.
// Every operand comes straight from global memory into MFMA operand registers, in the
// fragment orders the prep kernel wrote (one contiguous 1 KiB piece per fragment); each
// register set is reloaded with the next chunk's data right after its last use. One
// barrier per chunk for the whole workgroup.
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
constexpr int NO = 4;       // output waves per workgroup
constexpr int NRO = 4 / NO;  // row tiles per output wave

template <int DS, int NKS, int NC>
struct StateSmem {
  f32x4 partP[2][DS][NC][4][64];  // partial W<- S^T: parity, dk owner, column tile, row tile
  half8 s16[3][NC][NKS][64];      // fp16 S^T fragments: chunk mod 3, column tile, dk step
  half8 u16[2][NC][2][64];        // fp16 U (B operand of A_qk U): parity, column tile, step
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

template <int DK, int DS, int NC>
__global__ __launch_bounds__(64 * (DS + NO)) void mfma_state_kernel(
    const _Float16* __restrict__ Qf, const uint16_t* __restrict__ Kf,
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const double* __restrict__ gcum,
    const _Float16* __restrict__ W, const _Float16* __restrict__ Ut,
    const float* __restrict__ kdws, const _Float16* __restrict__ Aqk,
    const float* __restrict__ egws, int B, int H, int HV, int DV,
    float* __restrict__ state_pool, uint16_t* __restrict__ out) {
  constexpr int NKS = DK / 32;    // 32-wide dk steps
  constexpr int NOWN = NKS / DS;  // dk steps per state wave
  __shared__ StateSmem<DS, NKS, NC> sm;

  // Blocks of the same (request, head) share blockIdx.x mod 8, so they run on one
  // XCD and re-read the fragment blocks from its L2.
  const int nvb = DV / (16 * NC);
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int ct0 = (int)(rest % nvb) * NC;  // first column tile: state rows 16 ct0 ..
  const int64_t p = (rest / nvb) * 8 + (x & 7);
  if (p >= (int64_t)B * HV) return;
  const int seq = (int)(p / HV), hv = (int)(p % HV);
  const int64_t L = cu[seq + 1] - cu[seq];
  if (L <= 0) return;
  const int h = hv / (HV / H);
  const int64_t slot = cache_indices[seq];
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int nch = (int)((L + C - 1) / C);
  const int64_t cbase = chunk_off[seq];
  const int64_t tseq = cu[seq];
  const int64_t tend = cu[seq + 1];
  auto pair_of = [&](int cl) { return (cbase + cl) * HV + hv; };

  if (wv < DS) {
    // ======================= state wave =======================
    const int hs = wv;
    float* Sg = state_pool + ((slot * HV + hv) * (int64_t)DV + 16 * ct0 + m) * DK;
    f32x4 S[NC][NOWN][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          S[c][sp][tt] = *reinterpret_cast<const f32x4*>(Sg + c * 16 * DK + 32 * (hs * NOWN + sp) +
                                                         16 * tt + 4 * g);

    u32x4 wf[4][NOWN];     // W<- fragments: row tile, own dk step
    u32x4 kf[NOWN][2][2];  // k^T fragments: own dk step, 16-dk half, token step
    u32x2 uf[NC][4];       // U~ (fp16 D tiles): column tile, row tile
    f32x4 kdv[4];          // e^{G_n - G} r_k of rows 16I + 4g + i
    double gn;             // G_n (the gate pass pads G with zero log-decay)
    auto load_w = [&](int cl) {
      const _Float16* wb = W + pair_of(cl) * C * DK;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp)
          wf[I][sp] = *reinterpret_cast<const u32x4*>(
              wb + ((I * NKS + hs * NOWN + sp) * 64 + l) * 8);
    };
    auto load_ukd = [&](int cl) {
      const int64_t pr = pair_of(cl);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const _Float16* ub = Ut + pr * C * DV + ((ct0 + c) * 4 * 64 + l) * 4;
#pragma unroll
        for (int I = 0; I < 4; ++I) uf[c][I] = *reinterpret_cast<const u32x2*>(ub + I * 64 * 4);
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
        kdv[I] = *reinterpret_cast<const f32x4*>(kdws + pr * C + 16 * I + 4 * g);
    };
    auto load_k = [&](int cl) {
      const uint16_t* kb = Kf + ((cbase + cl) * H + h) * (int64_t)(C * DK);
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            kf[sp][tt][s] = *reinterpret_cast<const u32x4*>(
                kb + ((((hs * NOWN + sp) * 2 + tt) * 2 + s) * 64 + l) * 8);
      gn = gcum[pair_of(cl) * C + C - 1];
    };
    load_w(0);
    load_ukd(0);
    load_k(0);

    // Each register set is reloaded with chunk cl + 1 right after its last use in chunk
    // cl (chunk nch - 1 is reloaded on the last step: in bounds, and no branch).
    for (int cl = 0; cl < nch; ++cl) {
      const int buf = cl & 1;
      const int nx = min(cl + 1, nch - 1);

      // ---- S^T in fp16: operand of P here, and of Qh S^T for the output waves
      half8 s16[NC][NOWN];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp) {
          s16[c][sp] = cat(to_half4(S[c][sp][0]), to_half4(S[c][sp][1]));
          sm.s16[cl % 3][c][hs * NOWN + sp][l] = s16[c][sp];
        }
      // ---- partial P = W<- S^T over the owned dk steps (each W<- fragment serves every
      // column tile of the wave)
      f32x4 pp[NC][4];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          pp[c][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sp = 0; sp < NOWN; ++sp)
            pp[c][I] = mma_f16(half8_from_u32x4(wf[I][sp]), s16[c][sp], pp[c][I]);
        }
      load_w(nx);
      if (DS > 1) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int I = 0; I < 4; ++I) sm.partP[buf][hs][c][I][l] = pp[c][I];
      }
      lds_barrier();  // chunk cl: partial sums and S^T copies visible

      // ---- U = U~ - P for all rows (every state wave forms the same U); U'' =
      // diag(e^{G_n - G} r_k) U as the bf16 hi + lo B operand of the update
      bf16x8 bh[NC][2], bl[NC][2];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x4 U[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          f32x4 pt = pp[c][I];
#pragma unroll
          for (int o = 0; o < DS; ++o)
            if (o != hs) pt += sm.partP[buf][o][c][I][l];
          const half4 ut = __builtin_bit_cast(half4, uf[c][I]);
#pragma unroll
          for (int i = 0; i < 4; ++i) U[I][i] = (float)ut[i] - pt[i];
        }
        if (hs == 0) {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            sm.u16[buf][c][s][l] = cat(to_half4(U[2 * s]), to_half4(U[2 * s + 1]));
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x4 ua = U[2 * s] * kdv[2 * s], ub = U[2 * s + 1] * kdv[2 * s + 1];
          const bf16x4 ha = to_bf16x4(ua), hb = to_bf16x4(ub);
          bh[c][s] = cat_bf(ha, hb);
          bl[c][s] = cat_bf(to_bf16x4(ua - to_f32x4(ha)), to_bf16x4(ub - to_f32x4(hb)));
        }
      }
      load_ukd(nx);

      // ---- S^T <- e^{G_n} S^T + K^T U'' on the owned dk steps (each k^T fragment serves
      // every column tile of the wave)
      const float egn = expf((float)gn);
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            f32x4 acc = S[c][sp][tt] * egn;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const bf16x8 a = bf16x8_from_u32x4(kf[sp][tt][s]);
              acc = mma_bf16(a, bh[c][s], acc);
              acc = mma_bf16(a, bl[c][s], acc);
            }
            S[c][sp][tt] = acc;
          }
      load_k(nx);
    }
    lds_barrier();  // the output waves' last chunk: U of chunk nch - 1 visible

    // ---- write the state back in place
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<f32x4*>(Sg + c * 16 * DK + 32 * (hs * NOWN + sp) + 16 * tt + 4 * g) =
              S[c][sp][tt];
  } else {
    // ======================= output wave =======================
    // Output wave ow finishes row tiles I = NRO ow .. NRO ow + NRO - 1 of chunk cl, for every
    // column tile of the workgroup, after the barrier that ends the state waves' chunk
    // cl + 1 prologue, when U of chunk cl is in LDS: one barrier before the loop and one
    // per chunk, matching the state waves' count.
    const int ow = wv - DS;
    u32x4 qf[NRO][NKS];  // Qh fragments: own row tile, dk step
    u32x4 af[NRO][2];    // A_qk fragments: own row tile, token step
    f32x4 egv[NRO];      // e^G of rows 16I + 4g + i
    auto load_q = [&](int cl) {
      const int64_t pr = pair_of(cl);
      const _Float16* qb = Qf + ((cbase + cl) * H + h) * (int64_t)(C * DK);
#pragma unroll
      for (int r = 0; r < NRO; ++r) {
        const int I = NRO * ow + r;
#pragma unroll
        for (int sp = 0; sp < NKS; ++sp)
          qf[r][sp] = *reinterpret_cast<const u32x4*>(qb + ((I * NKS + sp) * 64 + l) * 8);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          af[r][s] = *reinterpret_cast<const u32x4*>(Aqk + pr * C * C + ((I * 2 + s) * 64 + l) * 8);
        egv[r] = *reinterpret_cast<const f32x4*>(egws + pr * C + 16 * I + 4 * g);
      }
    };
    load_q(0);
    lds_barrier();  // chunk 0 partial sums (state waves)
    for (int cl = 0; cl < nch; ++cl) {
      const int buf = cl & 1;
      const int nx = min(cl + 1, nch - 1);
      const int64_t t0 = tseq + (int64_t)cl * C;
      const int n = (int)min((int64_t)C, tend - t0);
      lds_barrier();  // U of chunk cl visible (S^T copy of chunk cl since the last one)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        half8 sf[NKS];
#pragma unroll
        for (int sp = 0; sp < NKS; ++sp) sf[sp] = sm.s16[cl % 3][c][sp][l];
        const half8 uh0 = sm.u16[buf][c][0][l], uh1 = sm.u16[buf][c][1][l];
#pragma unroll
        for (int r = 0; r < NRO; ++r) {
          const int I = NRO * ow + r;
          f32x4 o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sp = 0; sp < NKS; ++sp) o1 = mma_f16(half8_from_u32x4(qf[r][sp]), sf[sp], o1);
          f32x4 AU = mma_f16(half8_from_u32x4(af[r][0]), uh0, f32x4{0.f, 0.f, 0.f, 0.f});
          if (I >= 2) AU = mma_f16(half8_from_u32x4(af[r][1]), uh1, AU);
          const bf16x4 ov = to_bf16x4(egv[r] * o1 + AU);  // round to nearest even
          __bf16* ob = reinterpret_cast<__bf16*>(out) +
                       ((t0 + 16 * I + 4 * g) * HV + hv) * (int64_t)DV + 16 * (ct0 + c) + m;
          if (n == C) {  // full chunk: no per-row test
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i * (int64_t)HV * DV] = ov[i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * I + 4 * g + i < n) ob[i * (int64_t)HV * DV] = ov[i];
          }
        }
      }
      load_q(nx);
    }
  }
}

template <int DK, int DS, int NC>
hipError_t launch_state_t(const void* qf, const void* kf, const int64_t* cu, const int64_t* idx,
                          const int32_t* off, const double* gcum, const _Float16* w,
                          const _Float16* u, const float* kd, const _Float16* aqk,
                          const float* eg, const Shape& s, float* pool, void* out,
                          hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8;
  const int64_t blocks = pairs8 * 8 * (s.dv / (16 * NC));
  hipLaunchKernelGGL((mfma_state_kernel<DK, DS, NC>), dim3((unsigned)blocks),
                     dim3(64 * (DS + NO)), 0, st, (const _Float16*)qf, (const uint16_t*)kf, cu,
                     idx, off, gcum, w, u, kd, aqk, eg, (int)s.B, s.H, s.HV, s.dv, pool,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_state(const void* qf, const void* kf, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const double* gcum, const void* w, const void* u, const float* kd,
                             const void* aqk, const float* eg, const Shape& s,
                             float* state_pool, void* out, hipStream_t st) {
  const _Float16* W = (const _Float16*)w;
  const _Float16* U = (const _Float16*)u;
  // Each state wave holds 64 dk (two 32-wide steps) of its 16 state rows.
#define GDN_STATE_CASE(DKv)                                                                   \
  if (s.dk == DKv)                                                                            \
    return launch_state_t<DKv, DKv / 64, 2>(qf, kf, cu_seqlens, cache_indices, chunk_off,     \
                                            gcum, W, U, kd, (const _Float16*)aqk, eg, s,      \
                                            state_pool, out, st);
  GDN_STATE_CASE(64)
  GDN_STATE_CASE(128)
  GDN_STATE_CASE(256)
#undef GDN_STATE_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
