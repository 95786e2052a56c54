// Sequential state pass on matrix cores (bf16 inputs).
//
// One workgroup per (request, value head, block of NB x 16 state rows). Per chunk,
// in row convention (pymllm gdn_chunkwise page, Algorithm steps 2-3; "Simple math
// to speed up GDN prefill", Reminder, chunkwise transition with decorated S->, W<-,
// K->):
//   U     = U~ - W<- S^T
//   O     = diag(e^G r_q) Q S^T + A_qk U                           (to out)
//   S^T  <- e^{G_n} S^T + K^T diag(e^{G_n - G} r_k) U
// with r_q, r_k the inverse L2 norms of the rows of q and k and
// A_qk = Gamma o tril0(diag(r_q) Q K^T diag(r_k)), Gamma_ri = e^{G_r - G_i}, which the
// chunk-prep kernel has already formed (it depends on no state). Chunks of a request
// are processed in order (pymllm page: the propagation between chunks remains
// sequential over ceil(T/C) steps).
//
// Work split: 4 NB wavefronts; wave (wr, cb) serves column tile cb (16 state rows).
// It keeps the dk steps wr, wr + 4, ... of that tile of S^T in its registers for the
// whole request and contracts only over them: partial W<- S^T and Q S^T for all 64
// chunk rows go through LDS once per chunk and are summed by every wave, which then
// forms U for all rows itself. Wave (wr, cb) writes rows 16wr..16wr+15 of O. The
// next chunk's tiles are staged into a second LDS buffer while the current chunk's
// update runs: two barriers per chunk.
//
// Matrix-core operands: W<- and S in fp16 for P = W<- S^T; raw bf16 q with S as
// bf16 hi + lo for Q S^T; raw bf16 k with diag(e^{G_n-G} r_k) U as bf16 hi + lo
// for the update; A_qk and U in fp16 for A_qk U.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;

template <int DK, int NB>
struct StateSmem {
  static constexpr int SK = DK + 8;      // q/k row stride (bf16)
  static constexpr int NKS = DK / 32;
  uint16_t kt[2][C * SK];                // raw bf16 k rows, double-buffered by chunk parity
  uint16_t qt[C * SK];                   // raw bf16 q rows of the current chunk
  f32x4 partP[NB][4][4][64];             // partial W<- S^T (column tile, dk owner, row tile)
  f32x4 partO[NB][4][4][64];             // partial Q S^T
  float kd[2][C], erq[2][C];             // e^{G_n - G} r_k; e^G r_q
  float egn[2];                          // e^{G_n}
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

// Column `col` of a row-major 16-bit tile, rows row0 + kperm(g, 0..7).
__device__ __forceinline__ u32x4 col_frag(const uint16_t* base, int stride, int col, int row0,
                                          int g) {
  uint32_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = base[(row0 + kperm(g, j)) * stride + col];
  u32x4 r;
  r[0] = e[0] | (e[1] << 16);
  r[1] = e[2] | (e[3] << 16);
  r[2] = e[4] | (e[5] << 16);
  r[3] = e[6] | (e[7] << 16);
  return r;
}

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

template <int DK, int NB>
__global__ __launch_bounds__(256 * NB) void mfma_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const int64_t* __restrict__ cu, const int64_t* __restrict__ cache_indices,
    const int32_t* __restrict__ chunk_off, const double* __restrict__ gcum,
    const _Float16* __restrict__ W, const _Float16* __restrict__ Ut,
    const float* __restrict__ kdws, const _Float16* __restrict__ Aqk,
    const float* __restrict__ erqws, int B, int H, int HV, int DV,
    float* __restrict__ state_pool, uint16_t* __restrict__ out) {
  using Sm = StateSmem<DK, NB>;
  constexpr int SK = Sm::SK;
  constexpr int NT = 256 * NB;              // threads
  constexpr int NKS = DK / 32;              // 32-wide dk steps
  constexpr int NOWN = (NKS + 3) / 4;       // dk steps owned per wave (upper bound)
  constexpr int TILE_P = C * DK / 8;        // 16-byte pieces in one q or k tile
  constexpr int NP = (2 * TILE_P + NT - 1) / NT;  // pieces staged per thread
  __shared__ Sm sm;

  // Blocks of the same (request, head) share blockIdx.x mod 8, so they run on one
  // XCD and re-read q, k and W<- from its L2.
  const int nvb = DV / (16 * NB);
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int vb = (int)(rest % nvb);
  const int64_t p = (rest / nvb) * 8 + (x & 7);
  if (p >= (int64_t)B * HV) return;
  const int seq = (int)(p / HV), hv = (int)(p % HV);
  const int64_t L = cu[seq + 1] - cu[seq];
  if (L <= 0) return;
  const int h = hv / (HV / H);
  const int64_t slot = cache_indices[seq];
  const int tid = threadIdx.x, w8 = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int wr = w8 & 3, cb = w8 >> 2;
  const int ctile = NB * vb + cb;           // this wave's column tile (16 state rows)
  const int64_t nch = (L + C - 1) / C;
  const int64_t cbase = chunk_off[seq];
  const int64_t tseq = cu[seq];
  const int64_t tend = cu[seq + 1];

  // ---- resident state: S^T tiles of the owned dk steps of column tile ctile
  float* Sg = state_pool + ((slot * HV + hv) * (int64_t)DV + 16 * ctile + m) * DK;
  f32x4 Sacc[NOWN][2];
#pragma unroll
  for (int i = 0; i < NOWN; ++i) {
    const int sp = wr + 4 * i;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (sp < NKS) z = *reinterpret_cast<const f32x4*>(Sg + 32 * sp + 16 * tt + 4 * g);
      Sacc[i][tt] = z;
    }
  }

  // ---- prefetch registers for one chunk: staged pieces of k and q; this wave's W<-
  // fragments (its dk steps, all four row tiles); U~ of all four row tiles of its
  // column tile; A_qk fragments of its row tile; e^{G_n - G} r_k and e^G r_q (wave 0)
  // and G_n (thread 0; the gate pass extends G over padding rows with zero log-decay)
  u32x4 preg[NP];
  u32x4 wreg[NOWN][4];
  u32x2 ureg[4];
  u32x4 areg[2];
  double greg = 0.0;
  float kdreg = 0.f, erqreg = 0.f;
  auto load_chunk = [&](int64_t cl) {
    const int64_t pr = (cbase + cl) * HV + hv;
    const int64_t t0 = tseq + cl * C;
    const int n = (int)min((int64_t)C, tend - t0);
    const uint16_t* kb = k + (t0 * H + h) * (int64_t)DK;
    const uint16_t* qb = q + (t0 * H + h) * (int64_t)DK;
    const _Float16* wb = W + pr * C * DK;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = tid + NT * u;
      u32x4 z = {0u, 0u, 0u, 0u};
      if (e < 2 * TILE_P) {
        const int f = e < TILE_P ? e : e - TILE_P;
        const int row = f / (DK / 8), c8 = (f % (DK / 8)) * 8;
        if (row < n)
          z = *reinterpret_cast<const u32x4*>((e < TILE_P ? kb : qb) + (int64_t)row * H * DK + c8);
      }
      preg[u] = z;
    }
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
      const int sp = wr + 4 * i;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        u32x4 z = {0u, 0u, 0u, 0u};
        if (sp < NKS) z = *reinterpret_cast<const u32x4*>(wb + ((I * NKS + sp) * 64 + l) * 8);
        wreg[i][I] = z;
      }
    }
    const _Float16* ub = Ut + pr * C * DV + (ctile * 4 * 64 + l) * 4;
#pragma unroll
    for (int I = 0; I < 4; ++I) ureg[I] = *reinterpret_cast<const u32x2*>(ub + I * 64 * 4);
    const _Float16* ab = Aqk + pr * C * C + (wr * 2 * 64 + l) * 8;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) areg[s2] = *reinterpret_cast<const u32x4*>(ab + s2 * 64 * 8);
    if (tid < C) {
      kdreg = kdws[pr * C + tid];
      erqreg = erqws[pr * C + tid];
    }
    if (tid == 0) greg = gcum[pr * C + C - 1];
  };
  // Write one chunk's prefetched registers into LDS (k into buffer kb).
  auto stage_chunk = [&](int kbuf) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int e = tid + NT * u;
      if (e < 2 * TILE_P) {
        const int f = e < TILE_P ? e : e - TILE_P;
        const int row = f / (DK / 8), c8 = (f % (DK / 8)) * 8;
        *reinterpret_cast<u32x4*>(&(e < TILE_P ? sm.kt[kbuf] : sm.qt)[row * SK + c8]) = preg[u];
      }
    }
    if (tid < C) {  // wave 0, every lane
      sm.kd[kbuf][tid] = kdreg;
      sm.erq[kbuf][tid] = erqreg;
      if (tid == 0) sm.egn[kbuf] = expf((float)greg);
    }
  };
  // The next chunk's loads are issued at the top of an iteration and consumed at its
  // bottom, so no register with a load in flight is live across the loop back edge
  // (a copy there would wait for the load and expose its latency every chunk).
  load_chunk(0);
  stage_chunk(0);
  u32x2 ucur[4];
  u32x4 wcur[NOWN][4];
  u32x4 acur[2] = {areg[0], areg[1]};
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    ucur[I] = ureg[I];
#pragma unroll
    for (int i = 0; i < NOWN; ++i) wcur[i][I] = wreg[i][I];
  }
  lds_barrier();

  for (int64_t cl = 0; cl < nch; ++cl) {
    const int kb = (int)(cl & 1);
    const int64_t t0 = tseq + cl * C;
    const int n = (int)min((int64_t)C, tend - t0);
    if (cl + 1 < nch) load_chunk(cl + 1);

    // ================= phase 1: partial contractions ==================
    {
      // S^T fragments of the owned dk steps, from the resident accumulators
      half8 s16[NOWN];
      bf16x8 sbh[NOWN], sbl[NOWN];
#pragma unroll
      for (int i = 0; i < NOWN; ++i) {
        s16[i] = cat(to_half4(Sacc[i][0]), to_half4(Sacc[i][1]));
        const bf16x4 ah = to_bf16x4(Sacc[i][0]), bh = to_bf16x4(Sacc[i][1]);
        sbh[i] = cat_bf(ah, bh);
        sbl[i] = cat_bf(to_bf16x4(Sacc[i][0] - to_f32x4(ah)), to_bf16x4(Sacc[i][1] - to_f32x4(bh)));
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 pp = {0.f, 0.f, 0.f, 0.f}, po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NOWN; ++i) {
          const int sp = wr + 4 * i;
          if (sp < NKS) {
            pp = mma_f16(half8_from_u32x4(wcur[i][I]), s16[i], pp);
            const bf16x8 qa = bf16x8_from_u32x4(row_frag(sm.qt, SK, 16 * I + m, 32 * sp, g));
            po = mma_bf16(qa, sbh[i], po);
            po = mma_bf16(qa, sbl[i], po);
          }
        }
        sm.partP[cb][wr][I][l] = pp;
        sm.partO[cb][wr][I][l] = po;
      }
    }
    lds_barrier();  // (X)

    // ================= phase 2: U, state update, outputs, next chunk's staging =================
    f32x4 U[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 pt = sm.partP[cb][0][I][l];
#pragma unroll
      for (int o = 1; o < 4; ++o) pt += sm.partP[cb][o][I][l];
      const half4 ut = __builtin_bit_cast(half4, ucur[I]);
#pragma unroll
      for (int i = 0; i < 4; ++i) U[I][i] = (float)ut[i] - pt[i];
    }
    {  // S^T <- e^{G_n} S^T + K^T diag(e^{G_n - G} r_k) U on the owned dk steps
      bf16x8 bh[2], bl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        f32x4 ua = U[2 * s], ub2 = U[2 * s + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ua[i] *= sm.kd[kb][32 * s + 4 * g + i];
          ub2[i] *= sm.kd[kb][32 * s + 16 + 4 * g + i];
        }
        const bf16x4 ha = to_bf16x4(ua), hb = to_bf16x4(ub2);
        bh[s] = cat_bf(ha, hb);
        bl[s] = cat_bf(to_bf16x4(ua - to_f32x4(ha)), to_bf16x4(ub2 - to_f32x4(hb)));
      }
      const float egn = sm.egn[kb];
#pragma unroll
      for (int i = 0; i < NOWN; ++i) {
        const int sp = wr + 4 * i;
        if (sp < NKS) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = Sacc[i][tt] * egn;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const bf16x8 a = bf16x8_from_u32x4(col_frag(sm.kt[kb], SK, 32 * sp + 16 * tt + m, 32 * s, g));
              acc = mma_bf16(a, bh[s], acc);
              acc = mma_bf16(a, bl[s], acc);
            }
            Sacc[i][tt] = acc;
          }
        }
      }
    }
    {  // O rows 16wr..16wr+15 of column tile ctile
      f32x4 o1 = sm.partO[cb][0][wr][l];
#pragma unroll
      for (int o = 1; o < 4; ++o) o1 += sm.partO[cb][o][wr][l];
      f32x4 AU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s <= (wr >> 1))
          AU = mma_f16(half8_from_u32x4(acur[s]), cat(to_half4(U[2 * s]), to_half4(U[2 * s + 1])),
                       AU);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wr + 4 * g + i;
        if (r < n) {
          const float o = sm.erq[kb][r] * o1[i] + AU[i];
          out[((t0 + r) * HV + hv) * (int64_t)DV + 16 * ctile + m] = f32_to_bf16_bits(o);
        }
      }
    }
    // next chunk: stage its tiles (k into the other buffer)
    if (cl + 1 < nch) {
      stage_chunk(kb ^ 1);
      acur[0] = areg[0];
      acur[1] = areg[1];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        ucur[I] = ureg[I];
#pragma unroll
        for (int i = 0; i < NOWN; ++i) wcur[i][I] = wreg[i][I];
      }
    }
    lds_barrier();  // (Y)
  }

  // ---- write the state back in place
#pragma unroll
  for (int i = 0; i < NOWN; ++i) {
    const int sp = wr + 4 * i;
    if (sp < NKS) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        *reinterpret_cast<f32x4*>(Sg + 32 * sp + 16 * tt + 4 * g) = Sacc[i][tt];
    }
  }
}

template <int DK, int NB>
hipError_t launch_state_t(const void* q, const void* k, const int64_t* cu, const int64_t* idx,
                          const int32_t* off, const double* gcum, const _Float16* w,
                          const _Float16* u, const float* kd, const _Float16* aqk,
                          const float* erq, const Shape& s, float* pool, void* out,
                          hipStream_t st) {
  const int64_t pairs8 = (s.B * s.HV + 7) / 8;
  const int64_t blocks = pairs8 * 8 * (s.dv / (16 * NB));
  hipLaunchKernelGGL((mfma_state_kernel<DK, NB>), dim3((unsigned)blocks), dim3(256 * NB), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, cu, idx, off, gcum, w, u, kd, aqk,
                     erq, (int)s.B, s.H, s.HV, s.dv, pool, (uint16_t*)out);
  return hipGetLastError();
}

// Column tiles per workgroup: two when that still gives every compute unit (256)
// one workgroup (fewer blocks per head repeat less per-chunk shared work). At
// dk = 256 two tiles exceed the 160 KiB of LDS.
int choose_nb(const Shape& s) {
  const int64_t heads = s.B * s.HV;
  if (s.dk <= 128 && s.dv % 32 == 0 && heads * (s.dv / 32) >= 256) return 2;
  return 1;
}

}  // namespace

hipError_t launch_mfma_state(const void* q, const void* k, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const double* gcum, const void* w, const void* u, const float* kd,
                             const void* aqk, const float* erq, const Shape& s,
                             float* state_pool, void* out, hipStream_t st) {
  const _Float16* W = (const _Float16*)w;
  const _Float16* U = (const _Float16*)u;
  const int nb = choose_nb(s);
#define GDN_STATE_CASE(DKv, NBv)                                                              \
  if (s.dk == DKv && nb == NBv)                                                               \
    return launch_state_t<DKv, NBv>(q, k, cu_seqlens, cache_indices, chunk_off, gcum, W, U, kd, \
                                    (const _Float16*)aqk, erq, s, state_pool, out, st);
  GDN_STATE_CASE(64, 1)
  GDN_STATE_CASE(64, 2)
  GDN_STATE_CASE(128, 1)
  GDN_STATE_CASE(128, 2)
  GDN_STATE_CASE(256, 1)
#undef GDN_STATE_CASE
  return hipErrorInvalidValue;
}

}  // namespace gdn
