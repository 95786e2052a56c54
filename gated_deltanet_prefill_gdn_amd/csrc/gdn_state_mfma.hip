// Sequential state pass on matrix cores (bf16 inputs).
//
// Per chunk, in row convention (pymllm gdn_chunkwise page, Algorithm steps 2-3; "Simple
// math to speed up GDN prefill", Reminder, chunkwise transition with decorated S->, W<-,
// K->):
//   U     = U~ - W<- S^T
//   O     = diag(e^G) Qh S^T + A_qk U,  Qh = diag(r_q) Q              (to out)
//   S^T  <- e^{G_n} S^T + K~^T U,       K~ = diag(e^{G_n - G} r_k) K
// with r_q, r_k the inverse L2 norms of the rows of q and k and
// A_qk = Gamma o tril0(diag(r_q) Q K^T diag(r_k)), Gamma_ri = e^{G_r - G_i}, which the
// chunk-prep kernel has already formed together with K~ and the row scales (they depend
// on no state). Chunks of a request are processed in order (pymllm page: the propagation
// between chunks remains sequential over ceil(T/C) steps).
//
// Work split: one workgroup per (request, value head, NC x 16 state rows), with three
// roles; the chunk size C is 64 or 128.
//   * C / 32 state waves (two at C = 64). Wave hs holds dk rows hs * DK / (C / 32) .. of
//     the NC x 16 columns of S^T in fp32 registers for the whole request, and forms
//     P = W<- S^T and U for tokens 32 hs .. 32 hs + 31 over all of dk. The fp16 copies of
//     the S^T slices and of the U token steps, which the output waves need anyway, are
//     the only data the state waves exchange (LDS, double-buffered). Each wave then
//     updates its own rows with every token step of U. Two barriers per chunk: one after
//     the S^T copies, one after the U copies.
//   * C / 32 output waves form O from those LDS copies off the state chain: Qh S^T between
//     the two barriers, A_qk U after the second, two row tiles each. They compute O^T
//     (operands swapped), so each lane holds four consecutive columns of one token row,
//     and write O in bf16 to a double-buffered output tile in LDS.
//   * One store wave copies each finished tile to out with row-contiguous 16-byte
//     stores, so that no wave that waits for its prefetched operands has stores queued
//     among its loads (a wave's loads and stores retire in order). This is up to
//     dk = 128 at C = 64; otherwise the output waves store O themselves (see
//     kStoreWaves).
// With C / 32 state waves each wave's share of a chunk's operands, and so its registers,
// is the same at both chunk sizes.
// Every operand comes straight from global memory into MFMA operand registers, in the
// fragment orders the prep kernel wrote (one contiguous 1 KiB piece per fragment). Two
// register sets (one at dk = 256 and with four column tiles) alternate between chunks,
// each reloaded right after its last use (the output waves' q fragments right after
// Qh S^T, before barrier B), so every load has about two chunks of the chain to land.
//
// Matrix-core operands, all fp16 with fp32 accumulation: W<- and S for P; normalised q
// and S for Qh S^T; K~ and U for the update; A_qk and U for A_qk U. The state itself
// stays fp32; P starts from -U~ in the accumulator so U needs no separate subtraction.
#include <type_traits>

#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
// Waves per workgroup by chunk size CC (64 or 128): CC / 32 state waves, each owning one
// 32-token step of the chunk and DK / (CC / 32) rows of S^T, and CC / 32 output waves of
// two row tiles each.
template <int CC>
constexpr int kStateWaves = CC / 32;
template <int CC>
constexpr int kOutWaves = CC / 32;
constexpr int NRO = 2;  // row tiles per output wave

template <int NKS, int NC, int CC>
struct StateSmem {
  // Row stride (bf16) of the output tile: 16 bytes of padding spread the rows that the
  // 8-byte writes of one wave touch evenly over the banks.
  static constexpr int SO = 16 * NC + 8;
  half8 s16[2][NC][NKS][64];  // fp16 S^T fragments: chunk parity, column tile, dk step
  half8 u16[2][NC][CC / 32][64];  // fp16 U fragments: chunk parity, column tile, token step
  uint16_t o16[2][CC][SO];        // bf16 rows of O (16 NC columns): chunk parity, token
};

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 h;
  h[0] = (__bf16)x[0];
  h[1] = (__bf16)x[1];
  h[2] = (__bf16)x[2];
  h[3] = (__bf16)x[3];
  return h;
}

// Store waves: one up to dk = 128 at C = 64. At dk = 256 the state and output waves need
// more than half of a SIMD's registers, so they keep a SIMD each and store O themselves;
// at C = 128 the eight state and output waves take two per SIMD already.
template <int DK, int CC>
constexpr int kStoreWaves = (DK <= 128 && CC == 64) ? 1 : 0;
template <int DK, int CC>
constexpr int kStateThreads = 64 * (kStateWaves<CC> + kOutWaves<CC> + kStoreWaves<DK, CC>);

template <int DK, int NC, int PD, int CC>
__global__ __launch_bounds__((kStateThreads<DK, CC>)) void mfma_state_kernel(
    const _Float16* __restrict__ Qf, const _Float16* __restrict__ Kf,
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const _Float16* __restrict__ W, const _Float16* __restrict__ Ut,
    const _Float16* __restrict__ Aqk, const float* __restrict__ egws, int B, int H, int HV,
    int DV, int64_t short_len, float* __restrict__ state_pool, uint16_t* __restrict__ out,
    int32_t* __restrict__ nonfinite) {
  constexpr int C = CC;
  constexpr int NSW = kStateWaves<CC>;  // state waves = token steps of 32
  constexpr int NO = kOutWaves<CC>;
  constexpr int NRT = C / 16;           // row tiles of a chunk
  constexpr int NKS = DK / 32;          // 32-wide dk steps
  constexpr int NOWN = NKS / NSW;       // dk steps of S^T held by each state wave
  constexpr int NOTH = NSW - 1;         // the other state waves
  static_assert(NOWN >= 1 && NOWN * NSW == NKS, "dk steps split evenly over the state waves");
  __shared__ StateSmem<NKS, NC, CC> sm;

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
  const int nch = (int)path_chunks(L, C, short_len);
  if (nch == 0) return;  // empty (slot untouched) or evaluated by the token recurrence
  const int h = hv / (HV / H);
  const int64_t slot = cache_indices[seq];
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int64_t cbase = chunk_off[seq];
  const int64_t tseq = cu[seq];
  const int64_t tend = cu[seq + 1];
  auto pair_of = [&](int cl) { return (cbase + cl) * HV + hv; };

  if (wv < NSW) {
    // ======================= state wave =======================
    const int hs = wv;
    // the other state waves, in turn (NSW is a power of two)
    auto other = [hs](int o) { return NSW == 2 ? 1 - hs : (hs + 1 + o) & (NSW - 1); };
    float* Sg = state_pool + ((slot * HV + hv) * (int64_t)DV + 16 * ct0 + m) * DK;
    f32x4 S[NC][NOWN][2];  // S^T rows 32 (hs NOWN + sp) + 16 tt + 4g + i, column 16 c + m
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          S[c][sp][tt] = *reinterpret_cast<const f32x4*>(Sg + c * 16 * DK + 32 * (hs * NOWN + sp) +
                                                         16 * tt + 4 * g);

    // Register sets, split into the own and the other dk half (or token half) so that
    // every index into them is static. PD sets take the chunks in turn: each is reloaded
    // right after its last use with the chunk PD ahead.
    struct Regs {
      u32x4 wfo[2][NOWN];         // W<- fragments, row tiles 2hs + r: own dk steps
      u32x4 wfx[2][NOTH][NOWN];   // ... the other waves' dk steps
      u32x2 uf[NC][2];            // U~ D tiles: column tile, own row tile
      u32x4 kf[NOWN][2][NSW];  // K~^T fragments: own dk step, 16-row half, own/other tokens
      float egn;             // e^{G_n}: e^G of the chunk's last row (padding rows do not decay)
    };
    auto load_wu = [&](Regs& R, int cl) {
      const int64_t pr = pair_of(cl);
      const _Float16* wb = W + pr * C * DK;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp) {
          R.wfo[r][sp] = *reinterpret_cast<const u32x4*>(
              wb + (((2 * hs + r) * NKS + hs * NOWN + sp) * 64 + l) * 8);
#pragma unroll
          for (int o = 0; o < NOTH; ++o)
            R.wfx[r][o][sp] = *reinterpret_cast<const u32x4*>(
                wb + (((2 * hs + r) * NKS + other(o) * NOWN + sp) * 64 + l) * 8);
        }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const _Float16* ub = Ut + pr * C * DV + ((ct0 + c) * NRT * 64 + l) * 4;
#pragma unroll
        for (int r = 0; r < 2; ++r)
          R.uf[c][r] = *reinterpret_cast<const u32x2*>(ub + (2 * hs + r) * 64 * 4);
      }
    };
    auto load_k = [&](Regs& R, int cl) {
      const int64_t pr = pair_of(cl);
      const _Float16* kb = Kf + pr * (int64_t)(C * DK);
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int f = ((hs * NOWN + sp) * 2 + tt) * NSW;
          R.kf[sp][tt][0] = *reinterpret_cast<const u32x4*>(kb + ((f + hs) * 64 + l) * 8);
#pragma unroll
          for (int o = 0; o < NOTH; ++o)
            R.kf[sp][tt][1 + o] =
                *reinterpret_cast<const u32x4*>(kb + ((f + other(o)) * 64 + l) * 8);
        }
      R.egn = egws[pr * C + C - 1];
    };

    // A step with cl >= nch (the loop runs in groups of PD) leaves S unchanged: U = 0
    // and no decay.
    auto step = [&](Regs& R, int cl) {
      const int b = cl & 1;
      const int nx = min(cl + PD, nch - 1);  // chunks past the end reload the last one
      const bool live = cl < nch;

      // ---- own half of S^T in fp16: operand of P (both state waves) and of Qh S^T
      half8 so[NC][NOWN];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp) {
          so[c][sp] = cat(to_half4(S[c][sp][0]), to_half4(S[c][sp][1]));
          sm.s16[b][c][hs * NOWN + sp][l] = so[c][sp];
        }
      const float egn = live ? R.egn : 1.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) S[c][sp][tt] *= egn;
      lds_barrier();  // (A) both halves of S^T visible

      // ---- -U = W<- S^T - U~ for the own tokens, over all of dk
      half8 uo[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        half8 sx[NOTH][NOWN];
#pragma unroll
        for (int o = 0; o < NOTH; ++o)
#pragma unroll
          for (int sp = 0; sp < NOWN; ++sp) sx[o][sp] = sm.s16[b][c][other(o) * NOWN + sp][l];
        f32x4 nu[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const half4 ut = __builtin_bit_cast(half4, R.uf[c][r]);
          nu[r] = f32x4{-(float)ut[0], -(float)ut[1], -(float)ut[2], -(float)ut[3]};
#pragma unroll
          for (int sp = 0; sp < NOWN; ++sp) {
            nu[r] = mma_f16(half8_from_u32x4(R.wfo[r][sp]), so[c][sp], nu[r]);
#pragma unroll
            for (int o = 0; o < NOTH; ++o)
              nu[r] = mma_f16(half8_from_u32x4(R.wfx[r][o][sp]), sx[o][sp], nu[r]);
          }
        }
        // U in fp16, tokens 32 hs + kperm: B operand of the update and of A_qk U
        uo[c] = live ? cat(to_half4(-nu[0]), to_half4(-nu[1])) : half8{};
        sm.u16[b][c][hs][l] = uo[c];
      }
      load_wu(R, nx);
      lds_barrier();  // (B) every token step of U visible

      // ---- S^T <- e^{G_n} S^T + K~^T U on the own dk rows
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        half8 ux[NOTH];
#pragma unroll
        for (int o = 0; o < NOTH; ++o) ux[o] = sm.u16[b][c][other(o)][l];
#pragma unroll
        for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = mma_f16(half8_from_u32x4(R.kf[sp][tt][0]), uo[c], S[c][sp][tt]);
#pragma unroll
            for (int o = 0; o < NOTH; ++o)
              acc = mma_f16(half8_from_u32x4(R.kf[sp][tt][1 + o]), ux[o], acc);
            S[c][sp][tt] = acc;
          }
      }
      load_k(R, nx);
    };

    Regs rs[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      load_wu(rs[j], min(j, nch - 1));
      load_k(rs[j], min(j, nch - 1));
    }
    // Groups of PD chunks, with no branch and no tail: the load counter waits stay
    // static and no register set is copied at the back edge.
    for (int cl = 0; cl < nch; cl += PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) step(rs[j], cl + j);
    }

    lds_barrier();  // (F) the store wave reads the last chunk's O

    // ---- write the state back in place; raise the flag if it is not finite (an fp16
    // intermediate out of range)
    bool finite = true;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int sp = 0; sp < NOWN; ++sp)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          *reinterpret_cast<f32x4*>(Sg + c * 16 * DK + 32 * (hs * NOWN + sp) + 16 * tt + 4 * g) =
              S[c][sp][tt];
#pragma unroll
          for (int i = 0; i < 4; ++i) finite = finite && __builtin_isfinite(S[c][sp][tt][i]);
        }
    if (__ballot(!finite) != 0 && l == 0) *nonfinite = 1;
  } else if (wv < NSW + NO) {
    // ======================= output wave =======================
    // Output wave ow finishes row tiles I = NRO ow .. NRO ow + NRO - 1 of every column
    // tile: Qh S^T after barrier (A) of chunk cl, A_qk U after barrier (B). Computed as
    // O^T = S Qh^T + U^T A_qk^T: lane (g, m) holds row 16 I + m, columns 4g .. 4g + 3,
    // which it writes as bf16 to the chunk's output tile in LDS. The row tiles are
    // compile-time constants of each wave's code, so the causal skip of A_qk's upper
    // token step is static.
    auto run = [&](auto OWc) {
      constexpr int ow = decltype(OWc)::value;
      struct Regs {
        u32x4 qf[NRO][NKS];  // Qh fragments: own row tile, dk step
        u32x4 af[NRO][C / 32];  // A_qk fragments: own row tile, token step
        float egr[NRO];      // e^G of row 16 I + m
      };
      // The Qh fragments are reloaded as soon as Qh S^T has used them, while the wave
      // waits for barrier (B) anyway; the A_qk fragments and row scales after A_qk U.
      auto load_qf = [&](Regs& R, int cl) {
        const _Float16* qb = Qf + ((cbase + cl) * H + h) * (int64_t)(C * DK);
#pragma unroll
        for (int r = 0; r < NRO; ++r) {
          const int I = NRO * ow + r;
#pragma unroll
          for (int sp = 0; sp < NKS; ++sp)
            R.qf[r][sp] = *reinterpret_cast<const u32x4*>(qb + ((I * NKS + sp) * 64 + l) * 8);
        }
      };
      auto load_af = [&](Regs& R, int cl) {
        const int64_t pr = pair_of(cl);
#pragma unroll
        for (int r = 0; r < NRO; ++r) {
          const int I = NRO * ow + r;
#pragma unroll
          for (int s = 0; s < C / 32; ++s)
            if (I >= 2 * s)  // token steps past the row tile are above the diagonal
              R.af[r][s] = *reinterpret_cast<const u32x4*>(Aqk + pr * C * C +
                                                           ((I * (C / 32) + s) * 64 + l) * 8);
          R.egr[r] = egws[pr * C + 16 * I + m];
        }
      };
      auto step = [&](Regs& R, int cl) {
        const int b = cl & 1;
        const int nx = min(cl + PD, nch - 1);
        lds_barrier();  // (A) S^T copies of chunk cl visible
        f32x4 o1[NRO][NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          half8 sf[NKS];
#pragma unroll
          for (int sp = 0; sp < NKS; ++sp) sf[sp] = sm.s16[b][c][sp][l];
#pragma unroll
          for (int r = 0; r < NRO; ++r) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < NKS; ++sp)
              acc = mma_f16(sf[sp], half8_from_u32x4(R.qf[r][sp]), acc);
            o1[r][c] = acc;
          }
        }
        load_qf(R, nx);
        lds_barrier();  // (B) U of chunk cl visible
        f32x4 au[NRO][NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          half8 uh[C / 32];
#pragma unroll
          for (int s = 0; s < C / 32; ++s) uh[s] = sm.u16[b][c][s][l];
#pragma unroll
          for (int r = 0; r < NRO; ++r) {
            const int I = NRO * ow + r;
            au[r][c] = mma_f16(uh[0], half8_from_u32x4(R.af[r][0]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int s = 1; s < C / 32; ++s)
              if (I >= 2 * s) au[r][c] = mma_f16(uh[s], half8_from_u32x4(R.af[r][s]), au[r][c]);
          }
        }
        const int64_t t0 = tseq + (int64_t)cl * C;
        const int n = (int)min((int64_t)C, tend - t0);  // cl >= nch: n <= 0
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int r = 0; r < NRO; ++r) {
            const int I = NRO * ow + r;
            const bf16x4 ov = to_bf16x4(R.egr[r] * o1[r][c] + au[r][c]);  // nearest even
            if constexpr (kStoreWaves<DK, CC> > 0) {
              *reinterpret_cast<bf16x4*>(&sm.o16[b][16 * I + m][16 * c + 4 * g]) = ov;
            } else if (16 * I + m < n) {
              *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) +
                                         ((t0 + 16 * I + m) * HV + hv) * (int64_t)DV +
                                         16 * (ct0 + c) + 4 * g) = ov;
            }
          }
        load_af(R, nx);
      };
      Regs rs[PD];
#pragma unroll
      for (int j = 0; j < PD; ++j) {
        load_qf(rs[j], min(j, nch - 1));
        load_af(rs[j], min(j, nch - 1));
      }
      for (int cl = 0; cl < nch; cl += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) step(rs[j], cl + j);
      }
      lds_barrier();  // (F)
    };
    // one code copy per output wave
    if (wv == NSW)
      run(std::integral_constant<int, 0>{});
    else if (NO == 2 || wv == NSW + 1)
      run(std::integral_constant<int, 1>{});
    else if constexpr (NO == 4) {
      if (wv == NSW + 2)
        run(std::integral_constant<int, 2>{});
      else
        run(std::integral_constant<int, 3>{});
    }
  } else if constexpr (kStoreWaves<DK, CC> > 0) {
    // ======================= store wave =======================
    // Copies each chunk's output tile from LDS to out once it is complete (after barrier
    // (A) of the next chunk, or the final barrier), 16 bytes per lane, so that one store
    // instruction writes whole 32 NC-byte row pieces. Only this wave writes global memory
    // inside the chunk loop: the loads and stores of a wave retire in order, and stores
    // among the other waves' prefetches would make their load waits wait for the stores.
    const int ns = (nch + PD - 1) / PD * PD;  // chunk steps of the other waves
    constexpr int PR = NC * 16 / 8;           // 16-byte pieces per row
    auto store_o = [&](int cl) {              // cl >= nch: n <= 0, nothing is stored
      const int64_t t0 = tseq + (int64_t)cl * C;
      const int n = (int)min((int64_t)C, tend - t0);
      const int b = cl & 1;
      __bf16* ob = reinterpret_cast<__bf16*>(out) + (t0 * HV + hv) * (int64_t)DV + 16 * ct0;
#pragma unroll
      for (int i = 0; i < C * PR / 64; ++i) {
        const int r = (64 * i + l) / PR, pc = l % PR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.o16[b][r][8 * pc]);
        if (r < n) *reinterpret_cast<u32x4*>(ob + (int64_t)r * HV * DV + 8 * pc) = v;
      }
    };
    for (int cl = 0; cl < ns; ++cl) {
      lds_barrier();  // (A) of chunk cl: the tile of chunk cl - 1 is complete
      if (cl > 0) store_o(cl - 1);
      lds_barrier();  // (B)
    }
    lds_barrier();  // (F)
    store_o(ns - 1);
  }
}

template <int DK, int NC, int PD, int CC>
hipError_t launch_state_t(const void* qf, const void* kf, const int64_t* cu, const int64_t* idx,
                          const int32_t* off, const _Float16* w,
                          const _Float16* u, const _Float16* aqk, const float* eg, const Shape& s,
                          float* pool, void* out, int32_t* nonfinite, hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8;
  const int64_t blocks = pairs8 * 8 * (s.dv / (16 * NC));
  hipLaunchKernelGGL((mfma_state_kernel<DK, NC, PD, CC>), dim3((unsigned)blocks),
                     dim3(kStateThreads<DK, CC>), 0, st, (const _Float16*)qf,
                     (const _Float16*)kf, cu, idx, off, w, u, aqk, eg, (int)s.B, s.H, s.HV, s.dv,
                     s.short_len, pool, (uint16_t*)out, nonfinite);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_state(const void* qf, const void* kf, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const void* w, const void* u, const void* aqk,
                             const float* eg, const Shape& s, float* state_pool, void* out,
                             int32_t* nonfinite, hipStream_t st) {
  const _Float16* W = (const _Float16*)w;
  const _Float16* U = (const _Float16*)u;
  // The widest column block whose workgroups still fill the device: four column tiles (64
  // state rows, dk <= 128; every workgroup takes in the chunk's W<-, K~, Qh and A_qk in
  // full, so wider blocks serve more columns per byte taken in: 410 -> 350 us on the
  // varlen GQA workload), else two (32 rows), else one (16 rows), which doubles the
  // workgroups walking the chains (at dk = dv = 256 on one request of 8 heads,
  // 533 -> 442 us). dv is a multiple of 64. At C = 64 loads run two chunks ahead with up
  // to two column tiles at dk <= 128, one chunk ahead otherwise, where two register sets
  // would not fit. At C = 128 the same rule at dk = 128; at dk = 256 one column tile and
  // one chunk ahead (two column tiles would spill).
  const int64_t pairs = s.B * s.HV;
  const bool narrow = pairs * (s.dv / 32) < 256;
  const bool wide = s.dk <= 128 && pairs * (s.dv / 64) >= 256;
#define GDN_STATE_ARGS                                                                   \
  qf, kf, cu_seqlens, cache_indices, chunk_off, W, U, (const _Float16*)aqk, eg, s, state_pool, \
      out, nonfinite, st
#define GDN_STATE_CASE(DKv, PDv, CCv)                                                    \
  if (s.dk == DKv && s.C == CCv) {                                                       \
    if (narrow) return launch_state_t<DKv, 1, PDv, CCv>(GDN_STATE_ARGS);                 \
    if constexpr (DKv <= 128) {                                                          \
      if (wide) return launch_state_t<DKv, 4, 1, CCv>(GDN_STATE_ARGS);                   \
    }                                                                                    \
    return launch_state_t<DKv, 2, PDv, CCv>(GDN_STATE_ARGS);                             \
  }
  GDN_STATE_CASE(64, 2, 64)
  GDN_STATE_CASE(128, 2, 64)
  GDN_STATE_CASE(256, 1, 64)
  GDN_STATE_CASE(128, 2, 128)
  // dk = 256 at C = 128: one column tile (two would spill)
  if (s.dk == 256 && s.C == 128) return launch_state_t<256, 1, 1, 128>(GDN_STATE_ARGS);
#undef GDN_STATE_CASE
#undef GDN_STATE_ARGS
  return hipErrorInvalidValue;
}

}  // namespace gdn
