// The Promote update scan on matrix cores (bf16 keys and values).
//
// One level of the nested model of the awehrs.io page "NRM training kernels" (section
// General implementation, the Promote algorithm; section Kernel: a scan over firings,
// split over batch, heads and blocks of the value dimension, never over the key
// dimension, which the erase contracts). Each scan holds a dk x dv memory M in fp32. At
// firing f it receives n pairs at once: unit keys K (n x dk), values V (n x dv), erase
// and write gates beta, w (n) and one log-decay vector gamma (dk). In the page's order,
//   M' = diag(e^gamma) M;   M <- M' - K^T (beta o K) M' + K^T (w o V),
// which is computed as
//   P = K M' (n x dv),   U = w o V - beta o P,   M <- M' + K^T U.
// All pairs act on M as it stood before the firing (no order among them), so unlike the
// chunked delta rule there is no triangular solve: two products per firing.
//
// Work split: one workgroup per (scan, 64 value columns) with four compute waves and one
// store wave. Compute wave c holds columns 16 c .. 16 c + 15 of M, all dk rows, as fp32
// MFMA D tiles for the whole scan, and after each firing writes them to an LDS tile; the
// store wave copies that tile to `states` with row-contiguous 16-byte stores during the
// next firing (two barriers per firing), so the compute waves issue no global store.
// Per firing every workgroup stages K (converted to fp16), its V columns, the gates and
// e^gamma in LDS (double-buffered: the next firing's global loads are in flight while
// this one computes). The fp16 copy of a wave's M', two stacked D
// tiles per 32 key rows, is exactly the B operand of P = K M'; P's D tiles, two stacked
// per 32 pairs, become the B operand of the update once turned into U. K is the A
// operand of both products: read by rows (kperm order) for P and by columns (LDS
// transpose read) for K^T U, so it is loaded from HBM once per workgroup and firing. The
// workgroups of one scan share blockIdx.x mod 8 (one XCD) and so re-read K from its L2.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int kPromoteCols = 64;                       // value columns per workgroup
constexpr int kComputeWaves = kPromoteCols / 16;        // one wave per 16 columns
constexpr int kPromoteThreads = 64 * (kComputeWaves + 1);  // and one store wave

template <int DK, int NP>
struct PromoteSmem {
  static constexpr int SK = DK + 16;  // row stride (fp16) of the key tile: spreads banks
  static constexpr int SS = kPromoteCols + 4;  // row stride (fp32) of the state tile
  struct Buf {
    uint16_t kh[NP * SK];             // fp16 keys, rows n .. NP - 1 zero
    uint16_t vb[NP * kPromoteCols];   // bf16 values of the workgroup's columns
    float bt[NP], wt[NP];             // erase and write gates (0 past n)
    float eg[DK];                     // e^gamma
  };
  Buf b[2];
  float st[DK * SS];                  // the memory after a firing, for the store wave
};

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int DK, int NP>
__global__ __launch_bounds__(kPromoteThreads) void promote_scan_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ beta, const float* __restrict__ wg, const float* __restrict__ gamma,
    int64_t BH, int F, int n, int DV, float* __restrict__ M, float* __restrict__ states) {
  constexpr int SK = PromoteSmem<DK, NP>::SK;
  constexpr int NKS = DK / 32;   // 32-row key steps of M (B operand of P)
  constexpr int NRT = DK / 16;   // key row tiles of M
  constexpr int NPT = NP / 16;   // pair tiles
  constexpr int NPS = NP / 32;   // 32-pair steps (B operand of the update)
  constexpr int KPC = DK / 8;    // 16-byte pieces per key row
  constexpr int NT = 64 * kComputeWaves;  // threads that stage the operands
  constexpr int KPT = (NP * KPC + NT - 1) / NT;           // ... per thread
  constexpr int VPT = (NP * (kPromoteCols / 8) + NT - 1) / NT;
  static_assert(NP <= NT && DK <= NT, "one thread per pair and per key row");
  constexpr int SS = PromoteSmem<DK, NP>::SS;
  __shared__ PromoteSmem<DK, NP> sm;

  const int nvb = DV / kPromoteCols;
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int vb = (int)(rest % nvb);
  const int64_t bh = (rest / nvb) * 8 + (x & 7);
  if (bh >= BH) return;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int col = vb * kPromoteCols + 16 * wv + m;  // this lane's memory column

  // ---- global -> register prefetch of one firing's operands (zeros past n)
  u32x4 kr[KPT], vr[VPT];
  float br = 0.f, wr = 0.f, gr = 0.f;
  auto fetch = [&](int f) {  // compute waves only
    const int64_t bf = bh * F + f;
    const uint16_t* kb = K + bf * (int64_t)n * DK;
    const uint16_t* vbp = V + bf * (int64_t)n * DV + vb * kPromoteCols;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int e = tid + NT * u, row = e / KPC, c8 = (e % KPC) * 8;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (row < n) z = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)row * DK + c8));
      kr[u] = z;
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int e = tid + NT * u, row = e / (kPromoteCols / 8), c8 = (e % (kPromoteCols / 8)) * 8;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (row < n) z = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbp + (int64_t)row * DV + c8));
      vr[u] = z;
    }
    br = tid < n ? beta[bf * n + tid] : 0.f;
    wr = tid < n ? wg[bf * n + tid] : 0.f;
    gr = tid < DK ? gamma[bf * DK + tid] : 0.f;
  };
  // ---- registers -> LDS buffer (keys converted to fp16)
  auto stage = [&](typename PromoteSmem<DK, NP>::Buf& B) {  // compute waves only
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int e = tid + NT * u, row = e / KPC, c8 = (e % KPC) * 8;
      if (row < NP) {
        u32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = bf16_bits_to_f32((uint16_t)(kr[u][i] & 0xFFFFu));
          const float hi = bf16_bits_to_f32((uint16_t)(kr[u][i] >> 16));
          h[i] = (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
        }
        *reinterpret_cast<u32x4*>(&B.kh[row * SK + c8]) = h;
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int e = tid + NT * u, row = e / (kPromoteCols / 8), c8 = (e % (kPromoteCols / 8)) * 8;
      if (row < NP) *reinterpret_cast<u32x4*>(&B.vb[row * kPromoteCols + c8]) = vr[u];
    }
    if (tid < NP) {
      B.bt[tid] = br;
      B.wt[tid] = wr;
    }
    if (tid < DK) B.eg[tid] = expf(gr);
  };

  if (wv == kComputeWaves) {
    // ======================= store wave =======================
    // Writes the memory after firing f - 1 from the LDS tile to states while the compute
    // waves work on firing f: 16 bytes per lane, whole rows of the workgroup's columns per
    // instruction. Only this wave writes global memory inside the loop, so the compute
    // waves' waits for their prefetched operands never wait for these stores.
    constexpr int LPR = kPromoteCols / 4;  // lanes per tile row (4 fp32 each)
    constexpr int RPI = 64 / LPR;          // tile rows per store instruction
    static_assert(kPromoteCols % 4 == 0 && 64 % LPR == 0 && DK % RPI == 0, "store tiling");
    auto store_state = [&](int f) {
      const int c = 4 * (l % LPR);
      float* sg = states + ((bh * F + f) * DK) * (int64_t)DV + vb * kPromoteCols + c;
#pragma unroll 8
      for (int r = l / LPR; r < DK; r += RPI)
        *reinterpret_cast<f32x4*>(sg + (int64_t)r * DV) =
            *reinterpret_cast<const f32x4*>(&sm.st[r * SS + c]);
    };
    for (int f = 0; f < F; ++f) {
      lds_barrier();  // (A) firing f staged; the tile holds the memory after firing f - 1
      if (states && f > 0) store_state(f - 1);
      lds_barrier();  // (B) the tile is read; the compute waves may overwrite it
    }
    lds_barrier();    // (F) the tile holds the memory after the last firing
    if (states && F > 0) store_state(F - 1);
    return;
  }

  // ======================= compute waves =======================
  // This wave's 16 columns of M: rows 16 R + 4 g + i, column col.
  f32x4 Mt[NRT];
  float* Mg = M + (bh * DK) * (int64_t)DV + col;
#pragma unroll
  for (int R = 0; R < NRT; ++R)
#pragma unroll
    for (int i = 0; i < 4; ++i) Mt[R][i] = Mg[(int64_t)(16 * R + 4 * g + i) * DV];

  if (F > 0) fetch(0);
  for (int f = 0; f < F; ++f) {
    auto& B = sm.b[f & 1];
    stage(B);
    // (A) Buffer f & 1 complete; its previous reader (firing f - 2) finished before the
    // barrier (A) of firing f - 1. LDS-only barriers: no thread reads global memory that
    // another thread writes.
    lds_barrier();
    if (f + 1 < F) fetch(f + 1);

    // decay: M' = diag(e^gamma) M, and its fp16 copy as the B operand of P
    half8 so[NKS];
#pragma unroll
    for (int R = 0; R < NRT; ++R) {
      const f32x4 e = *reinterpret_cast<const f32x4*>(&B.eg[16 * R + 4 * g]);
      Mt[R] *= e;
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) so[s] = cat(to_half4(Mt[2 * s]), to_half4(Mt[2 * s + 1]));

    // P = K M' and U = w o V - beta o P, pair rows 16 I + 4 g + i
    f32x4 U[NPT];
#pragma unroll
    for (int I = 0; I < NPT; ++I) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        acc = mma_f16(half8_from_u32x4(row_frag_kperm(B.kh, SK, 16 * I + m, 32 * s, g)), so[s],
                      acc);
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&B.bt[16 * I + 4 * g]);
      const f32x4 wt = *reinterpret_cast<const f32x4*>(&B.wt[16 * I + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float vv = bf16_bits_to_f32(B.vb[(16 * I + 4 * g + i) * kPromoteCols + 16 * wv + m]);
        U[I][i] = wt[i] * vv - bt[i] * acc[i];
      }
    }
    // M <- M' + K^T U: A operand = columns of the key tile (transpose read)
    half8 us[NPS];
#pragma unroll
    for (int t = 0; t < NPS; ++t) us[t] = cat(to_half4(U[2 * t]), to_half4(U[2 * t + 1]));
#pragma unroll
    for (int R = 0; R < NRT; ++R)
#pragma unroll
      for (int t = 0; t < NPS; ++t)
        Mt[R] = mma_f16(half8_from_u32x4(col_frag_tr(B.kh, SK, 16 * R, t, g, m)), us[t], Mt[R]);

    lds_barrier();  // (B) the store wave has read the previous firing's tile
    if (states) {
#pragma unroll
      for (int R = 0; R < NRT; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.st[(16 * R + 4 * g + i) * SS + 16 * wv + m] = Mt[R][i];
    }
  }
  lds_barrier();  // (F)

#pragma unroll
  for (int R = 0; R < NRT; ++R)
#pragma unroll
    for (int i = 0; i < 4; ++i) Mg[(int64_t)(16 * R + 4 * g + i) * DV] = Mt[R][i];
}

template <int DK, int NP>
hipError_t launch_promote_t(const PromoteShape& s, const void* K, const void* V,
                            const float* beta, const float* w, const float* gamma, float* M,
                            float* states, hipStream_t st) {
  const int nvb = s.dv / kPromoteCols;
  const int64_t blocks = (s.BH + 7) / 8 * 8 * nvb;
  hipLaunchKernelGGL((promote_scan_kernel<DK, NP>), dim3((unsigned)blocks), dim3(kPromoteThreads), 0, st,
                     (const uint16_t*)K, (const uint16_t*)V, beta, w, gamma, s.BH, s.F, s.n,
                     s.dv, M, states);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_promote(const PromoteShape& s, const void* K, const void* V, const float* beta,
                          const float* w, const float* gamma, float* M, float* states,
                          hipStream_t st) {
  const int np = s.n <= 32 ? 32 : s.n <= 64 ? 64 : 128;
#define GDN_PROMOTE_CASE(DKv, NPv)                                                  \
  if (s.dk == DKv && np == NPv)                                                     \
    return launch_promote_t<DKv, NPv>(s, K, V, beta, w, gamma, M, states, st);
  GDN_PROMOTE_CASE(64, 32)
  GDN_PROMOTE_CASE(64, 64)
  GDN_PROMOTE_CASE(128, 32)
  GDN_PROMOTE_CASE(128, 64)
  GDN_PROMOTE_CASE(128, 128)
#undef GDN_PROMOTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
