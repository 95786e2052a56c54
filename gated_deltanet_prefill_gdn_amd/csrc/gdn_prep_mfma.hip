// Chunk preparation on matrix cores (bf16 inputs), at C = 64 (this kernel) and C = 128 (the
// second kernel of this file).
//
// Row convention (S is dv x dk; K, Q, V are the chunk's n <= C rows; G the chunk-local
// inclusive log cumulative gate; r_k = 1/|k|, r_q = 1/|q|):
//   A    = tril(diag(beta r_k) K K^T diag(r_k), -1)       Gram of raw bf16 keys, exact
//                                                         products, fp32 accumulation
//   T    = (I + A)^-1                                     the single inverse, M^-1
//   W<-  = diag(e^G) T diag(beta r_k) K                   ("Simple math to speed up GDN
//                                                         prefill", Reminder: W up to a
//                                                         decay factor, arrow decoration)
//   U~   = (Gamma o T) diag(beta) V,  Gamma_ri = e^{G_r - G_i}   the decayed inverse
//          N^-1 = G M^-1 G^-1 of the Save-one-invert section, taken entry by entry
//   A_qk = Gamma o tril0(diag(r_q) Q K^T diag(r_k))       the intra-chunk read with the
//          causal mask that includes the diagonal (pymllm gdn_chunkwise page, Algorithm)
//   K~   = diag(e^{G_n - G} r_k) K                      the keys of the state update,
//          decayed to the chunk end (same Reminder, K decorated with the right arrow)
// plus the row scale e^G that the state pass applies to the read of the state.
//
// Work split: the chunk's K and Q rows are staged in LDS with row-contiguous loads (a
// fragment load straight from global memory would touch 16 rows per instruction, which
// costs the address unit four times as much). Wave w owns chunk rows 16w .. 16w + 15
// (row tile w): it reads the operand fragments of its rows, and of the earlier tiles
// J < w, from LDS and forms both Grams of its rows in registers. The inverse is blocked
// in 16 x 16 tiles: the diagonal tile by forward substitution in fp32, then
// T_wJ = -T_ww sum_{J <= K < w} A_wK T_KJ by block distance w - J on fp32 matrix cores;
// only tiles another wave needs pass through LDS. Every wave keeps the transposed tiles
// T_wJ^T of its own rows, which are exactly the operand fragments of its rows of W<- and
// U~. The token contractions read column fragments of K and V with the LDS transpose
// read. Five barriers after staging. For the state pass the kernel also writes K~ (fp16,
// per value head, since the gates are) and normalised q (fp16, once per q/k head) in
// that kernel's operand-fragment order. The gates themselves (g, beta and the chunk-local
// log cumulative decay G) are formed here too, by wave 0 for the next item at the end of
// the current one.
//
// Fragment notation: Dl(X) is the MFMA result layout of a 16 x 16 tile X, lane
// l = 16 g + m holding X[4g + i][m], i = 0..3. A product P Q takes Dl(P^T) as its A
// operand and Dl(Q) as its B operand (for 16x16x4 fp32 with k = 4g + s at step s; for
// 16x16x32, two stacked tiles in kperm order). T1 = diag(e^G) T diag(beta r_k) and
// T2 = (Gamma o T) diag(beta) are split into bf16 hi + lo so the bf16 products with the
// exact raw K and V keep fp32 accuracy. W<-, U~, A_qk and K~ are stored as fp16 in the
// fragment layouts the state kernel loads directly into registers. These stores are
// non-temporal: the blocks are read once, by the state pass, and left as dirty lines in the
// caches they slowed that pass's reads by about 15% (measured).
#include <algorithm>

#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;
constexpr double kLog2e = 1.4426950408889634;
constexpr int SA = 20;      // row stride (fp32) of a wave's 16 x 16 scratch tile

template <int DK, int DV>
struct PrepSmem {
  // Row strides (bf16) of the staged tiles: 16 elements of padding put the four rows a
  // transpose read touches per lane group in different banks.
  static constexpr int SK = DK + 16;
  static constexpr int SQV = (DK > DV ? DK : DV) + 16;
  uint16_t ks[C * SK];    // K rows
  uint16_t qv[C * SQV];   // Q rows, later V rows
  f32x4 tex[9][64];       // Dl(T_IJ) tiles that other waves read: diagonal, distance 1, 2
  float sq[4][16 * SA];   // per-wave scratch: A_ww, then the columns of T_ww
  double G2[2][C];        // G log2(e), by item parity
  float bt[2][C];         // beta, by item parity
  float rk[C];            // r_k
  int32_t coff[kMaxSelfPlanRequests + 1];  // chunk table formed here: first chunk of each request
};

// LDS slot of an exchanged tile T_IJ (I - J <= 2).
__device__ __forceinline__ int tex_slot(int I, int J) {
  return I == J ? I : (I - J == 1 ? 4 + J : 7 + J);
}

// Load rows of a row-major bf16 tile (global row stride rs, D columns) into registers,
// zeros past n rows. Consecutive threads take consecutive 16-byte pieces of a row, so
// one wavefront instruction covers whole rows; piece u of thread tid is element
// e = tid + 256u: row e / (D / 8), columns 8 (e % (D / 8)) ...
template <int D>
__device__ __forceinline__ void load_tile_rows(u32x4 (&r)[C * D / 8 / 256], const uint16_t* src,
                                               int64_t rs, int n, int tid) {
#pragma unroll
  for (int u = 0; u < C * D / 8 / 256; ++u) {
    const int e = tid + 256 * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
    u32x4 z = {0u, 0u, 0u, 0u};
    // non-temporal: the rows are read once (measured slightly faster than cached loads)
    if (row < n) z = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + row * rs + c8));
    r[u] = z;
  }
}

// Store such pieces into an LDS tile of row stride ld.
template <int D>
__device__ __forceinline__ void store_tile_rows(uint16_t* dst, int ld,
                                                const u32x4 (&r)[C * D / 8 / 256], int tid) {
#pragma unroll
  for (int u = 0; u < C * D / 8 / 256; ++u) {
    const int e = tid + 256 * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(&dst[row * ld + c8]) = r[u];
  }
}

// Row fragment of an LDS tile: row `row`, elements 32s + 8g .. 32s + 8g + 7 of every
// 32-wide step s (the contraction order of the Gram products).
template <int D>
__device__ __forceinline__ void row_frags(u32x4 (&f)[D / 32], const uint16_t* base, int ld,
                                          int row, int g) {
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    f[s] = *reinterpret_cast<const u32x4*>(base + row * ld + 32 * s + 8 * g);
}

// A copy of a lane index that the compiler cannot treat as loop-invariant. Per-lane
// predicates built from it are recomputed where they are used (one compare each) instead
// of being hoisted out of the item loop as 64-bit lane masks, which exhaust the scalar
// registers and spill.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Squared norm of the row a lane group shares (the four lane groups hold one row).
template <int D>
__device__ __forceinline__ float sum_sq(const u32x4 (&f)[D / 32]) {
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc += bf_lo(f[s][j]) * bf_lo(f[s][j]) + bf_hi(f[s][j]) * bf_hi(f[s][j]);
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  return acc;
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

// Up to dk + dv = 256 three workgroups share a compute unit (168 VGPRs, no spills; the
// LDS of three fits): the item's phases are short chains separated by barriers, and the
// third workgroup fills the gaps (about 8% faster than two at dk = dv = 128, measured).
template <int DK, int DV, bool SELF_PLAN>
__global__ __launch_bounds__(256, (DK + DV <= 256) ? 3 : 1) void mfma_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ cu, int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ chunk_seq, const float* __restrict__ ga,
    const float* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, int B, int H, int HV, int64_t short_len,
    _Float16* __restrict__ Wout,
    _Float16* __restrict__ Uout, _Float16* __restrict__ Aout, float* __restrict__ eg_out,
    _Float16* __restrict__ Kout, _Float16* __restrict__ Qout, int32_t* __restrict__ nonfinite) {
  constexpr int NKS = DK / 32;
  using Sm = PrepSmem<DK, DV>;
  constexpr int SK = Sm::SK, SQV = Sm::SQV;
  __shared__ Sm sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int t = 16 * w + m;  // this lane's chunk row
  const int64_t rsk = (int64_t)H * DK;
  constexpr int KP = C * DK / 8 / 256;  // 16-byte pieces per thread of a K or Q tile
  constexpr int VP = C * DV / 8 / 256;  // ... of a V tile

  // Persistent: workgroups stride over the (chunk, q/k head) groups of the chunk_off[B]
  // real chunks and take the HV / H value heads of a group as consecutive items, which
  // share the group's K rows: those are loaded and staged once per group (the staged K
  // tile stays in LDS for the group's next item). The next item's rows are loaded into
  // registers while the current one is processed, so no register set is merged or copied
  // at the loop back edge.
  struct Item {
    int hv, h, n;
    int64_t c, t0;
  };
  auto geom = [&](int64_t it, Item& x) {
    x.c = it / HV;
    x.hv = (int)(it % HV);
    x.h = x.hv / (HV / H);
    int32_t sq, first;
    if constexpr (SELF_PLAN) {
      // the owner of chunk c: the number of requests whose chunks all precede c (the
      // chunk ends coff[b + 1] do not decrease, so they are the first sq requests)
      // (the lane index is opaque so the LDS read is not hoisted out of the item loop,
      // where it would hold a register for the whole loop)
      const int lo = opaque(l);
      sq = __popcll(__ballot(lo < B && sm.coff[lo + 1] <= x.c));
      first = sm.coff[sq];
    } else {
      sq = chunk_seq[x.c];
      first = chunk_off[sq];
    }
    x.t0 = cu[sq] + (int64_t)(x.c - first) * C;
    x.n = (int)min((int64_t)C, cu[sq + 1] - x.t0);
  };
  u32x4 kreg[KP], qreg[KP], vreg[VP];
  float areg, breg;  // raw gate inputs a, b of chunk row tid % C
  auto load_kq = [&](const Item& x, bool with_k) {
    if (with_k) {
      load_tile_rows<DK>(kreg, k + (x.t0 * H + x.h) * (int64_t)DK, rsk, x.n, tid);
    } else {
      // unused; defined so the registers are not live through the item
#pragma unroll
      for (int u = 0; u < KP; ++u) kreg[u] = u32x4{0u, 0u, 0u, 0u};
    }
    load_tile_rows<DK>(qreg, q + (x.t0 * H + x.h) * (int64_t)DK, rsk, x.n, tid);
  };
  // the next item shares the current one's K rows (the same chunk and q/k head)
  auto same_k = [](const Item& a, const Item& b) { return a.c == b.c && a.h == b.h && a.n == b.n; };
  auto load_vg = [&](const Item& x) {
    load_tile_rows<DV>(vreg, v + (x.t0 * HV + x.hv) * (int64_t)DV, (int64_t)HV * DV, x.n, tid);
    if (tid < C) {
      // rows past the request's end read its last token (in bounds) and are zeroed later;
      // the empty item after a workgroup's last one reads its first row
      const int64_t tr = x.t0 + min(tid & (C - 1), max(x.n - 1, 0));
      areg = ga[tr * HV + x.hv];
      breg = gb[tr * HV + x.hv];
    }
  };
  // Gates of item x (wave 0, one lane per row, from that item's prefetched a and b):
  // g = log(alpha) = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); zero on padding
  // rows (alpha = 1, beta = 0). G = the chunk-local inclusive sum of g, in fp64. Wave 0
  // forms the next item's gates at the end of the current one, where it waits for the
  // waves with more triangular work anyway; the two LDS copies alternate by item parity.
  auto gates = [&](const Item& x, int buf) {
    float gt = 0.f, bt = 0.f;
    if (tid < x.n) {
      const float xg = areg + dt_bias[x.hv];
      const float sp = fmaxf(xg, 0.f) + log1pf(expf(-fabsf(xg)));
      gt = -expf(A_log[x.hv]) * sp;
      bt = 1.f / (1.f + expf(-breg));
    }
    double G = (double)gt;
  #pragma unroll
    for (int off = 1; off < C; off <<= 1) {
      const double y = __shfl_up(G, off, C);
      if (tid >= off) G += y;
    }
    sm.G2[buf][tid] = G * kLog2e;
    sm.bt[buf][tid] = bt;
  };
  if constexpr (SELF_PLAN) {
    // At most 64 requests: wave 0 forms the chunk table with one scan (coff[b] = sum of
    // ceil(L_b' / C) over b' < b), and workgroup 0 writes it out for the state pass, so no
    // separate table kernel runs.
    if (w == 0) {
      int32_t nb = 0;
      if (l < B) {
        const int64_t L = cu[l + 1] - cu[l];
        nb = (int32_t)path_chunks(L, C, short_len);
      }
      int32_t x = nb;  // inclusive scan over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (l >= off) x += y;
      }
      sm.coff[l + 1] = x;
      if (l == 0) sm.coff[0] = 0;
    }
    __syncthreads();
    if (blockIdx.x == 0 && tid <= B) chunk_off[tid] = sm.coff[tid];
  }
  if (blockIdx.x == 0 && tid == 0) *nonfinite = 0;  // the state pass raises it
  const int64_t n_items = (int64_t)(SELF_PLAN ? sm.coff[B] : chunk_off[B]) * HV;
  const int GQ = HV / H;  // value heads per q/k head
  // the workgroup's j-th item: value head j % GQ of its (j / GQ)-th group
  auto item_of = [&](int64_t j) {
    return ((int64_t)blockIdx.x + (int64_t)gridDim.x * (j / GQ)) * GQ + j % GQ;
  };
  if (item_of(0) >= n_items) return;
  Item cur;
  geom(item_of(0), cur);
  load_kq(cur, true);
  load_vg(cur);
  if (tid < C) gates(cur, 0);
  int ib = 0;           // item parity: this item's gate copy
  bool stage_k = true;  // this item's K rows are in kreg, not yet in LDS
  for (int64_t jw = 0, it = item_of(0); it < n_items; ++jw, it = item_of(jw), ib ^= 1) {
    // The next item; after the workgroup's last item an empty one (n = 0) whose
    // prefetch loads nothing.
    const int64_t itn = item_of(jw + 1);
    Item nx;
    geom(itn < n_items ? itn : it, nx);
    if (itn >= n_items) nx.n = 0;
    const int hv = cur.hv, h = cur.h, n = cur.n;
    const int64_t c = cur.c, t0 = cur.t0;
    const int64_t pair = c * HV + hv;

    // ---- stage K (unless this group's previous item left it in LDS) and Q rows in LDS
    // from the prefetch registers
    if (stage_k) store_tile_rows<DK>(sm.ks, SK, kreg, tid);
    store_tile_rows<DK>(sm.qv, SQV, qreg, tid);
    const double* G2 = sm.G2[ib];
    const float* bts = sm.bt[ib];
    lds_barrier();  // (0) K, Q staged (and this item's gates)

    // ---- operand fragments of the own rows; norms (the earlier tiles' fragments are
    // read from LDS where the Grams use them)
    u32x4 kw[NKS], qf[NKS];
    row_frags<DK>(kw, sm.ks, SK, t, g);
    row_frags<DK>(qf, sm.qv, SQV, t, g);
    const float rkt = 1.0f / sqrtf(sum_sq<DK>(kw) + kNormEps);
    const float rqt = 1.0f / sqrtf(sum_sq<DK>(qf) + kNormEps);
    if (g == 0) sm.rk[t] = rkt;

    // ---- q in the state pass's operand order, once per q/k head: fragment (I, sp) holds
    // rows 16I + m of diag(r_q) Q in fp16, columns 32sp + kperm(g, .)
    if (hv % (HV / H) == 0) {
      const int64_t fo = (c * H + h) * (int64_t)(C * DK);
  #pragma unroll
      for (int sp = 0; sp < NKS; ++sp) {
        const u32x4 x = row_frag_kperm(sm.qv, SQV, t, 32 * sp, g);
        half8 y;
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[2 * j] = (_Float16)(bf_lo(x[j]) * rqt);
          y[2 * j + 1] = (_Float16)(bf_hi(x[j]) * rqt);
        }
        __builtin_nontemporal_store(y, reinterpret_cast<half8*>(Qout + fo + ((w * NKS + sp) * 64 + l) * 8));
      }
    }

    // ---- Grams of the own rows against tiles J <= w, transposed:
    // D[J] = Dl(K_J K_w^T), E[J] = Dl(K_J Q_w^T); lane (g, m): row 16J + 4g + i, column t
    f32x4 D[4], E[4];
  #pragma unroll
    for (int J = 0; J < 4; ++J) {
      D[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      E[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (J < w) {
  #pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 kj = bf16x8_from_u32x4(
              *reinterpret_cast<const u32x4*>(sm.ks + (16 * J + m) * SK + 32 * s + 8 * g));
          D[J] = mma_bf16(kj, bf16x8_from_u32x4(kw[s]), D[J]);
          E[J] = mma_bf16(kj, bf16x8_from_u32x4(qf[s]), E[J]);
        }
      } else if (J == w) {
  #pragma unroll
        for (int s = 0; s < NKS; ++s) {
          D[J] = mma_bf16(bf16x8_from_u32x4(kw[s]), bf16x8_from_u32x4(kw[s]), D[J]);
          E[J] = mma_bf16(bf16x8_from_u32x4(kw[s]), bf16x8_from_u32x4(qf[s]), E[J]);
        }
      }
    }
    lds_barrier();  // (1) r_k visible; Q no longer read

    // ---- V rows into the Q region (every wave is done with Q); visible after (2)
    store_tile_rows<DV>(sm.qv, SQV, vreg, tid);
    load_vg(nx);

    // ---- K~ = diag(e^{G_n - G} r_k) K in fp16, in the state update's operand order:
    // fragment f = (sp * 2 + tt) * 2 + s holds K~^T rows 32sp + 16tt + m, tokens
    // 32s + kperm(g, .). Wave w writes the fragments f = w (mod 4), whose token step is
    // s = w & 1.
    {
      const int s = w & 1;
      float kdj[8];
  #pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tk = 32 * s + kperm(g, j);
        kdj[j] = __builtin_amdgcn_exp2f((float)(G2[C - 1] - G2[tk])) * sm.rk[tk];
      }
      // lane offset taken in the loop: hoisted, one address per fragment stays live
      half8* kb = reinterpret_cast<half8*>(Kout + pair * (int64_t)(C * DK)) + w * 64 + opaque(l);
  #pragma unroll
      for (int f = w; f < NKS * 4; f += 4) {
        const int sp = f >> 2, tt = (f >> 1) & 1;
        const u32x4 x = col_frag_tr(sm.ks, SK, 32 * sp + 16 * tt, s, g, m);
        half8 y;
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[2 * j] = (_Float16)(bf_lo(x[j]) * kdj[2 * j]);
          y[2 * j + 1] = (_Float16)(bf_hi(x[j]) * kdj[2 * j + 1]);
        }
        __builtin_nontemporal_store(y, kb + (f - w) * 64);
      }
    }

    // ---- scale: a[J] = Dl(A_wJ^T) (A[t][i], i = 16J + 4g + ii < t) and the A_qk rows
    const double G2t = G2[t];
    const float btt = bts[t];
    const float egt = __builtin_amdgcn_exp2f((float)G2t);
    if (g == 0) eg_out[pair * C + t] = egt;
    f32x4 a[4];
    half4 aq[4];
    // Tiles J < w lie wholly below the diagonal and J > w wholly above it (uniform
    // branches); only the diagonal tile J = w needs the per-element tests i < t, i <= t.
    const int dm = opaque(m) - 4 * g;  // i < t  <=>  ii < dm on the diagonal tile
  #pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      a[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * J + 4 * g + ii;
          const float rki = sm.rk[i];
          const float av = btt * rkt * rki * D[J][ii];
          const float xv = __builtin_amdgcn_exp2f((float)(G2t - G2[i])) * rqt * rki * E[J][ii];
          a[J][ii] = (J < w || ii < dm) ? av : 0.f;
          x[ii] = (J < w || ii <= dm) ? xv : 0.f;
        }
      }
      aq[J] = to_half4(x);
    }
    // the fragment of row tiles 0 and 1 at token step 1 lies above the diagonal: zero, and
    // never read by the state pass
  #pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s == 0 || w >= 2)
        __builtin_nontemporal_store(cat(aq[2 * s], aq[2 * s + 1]), reinterpret_cast<half8*>(Aout + pair * C * C + ((w * 2 + s) * 64 + l) * 8));

    // ---- diagonal tile: T_ww = (I + A_ww)^-1 by forward substitution, lane = column m
    float* sqw = sm.sq[w];
    f32x4 aw = a[0];
  #pragma unroll
    for (int J = 1; J < 4; ++J)
      if (J == w) aw = a[J];
    *reinterpret_cast<f32x4*>(&sqw[m * SA + 4 * g]) = aw;  // row m of A_ww, columns 4g..
    __builtin_amdgcn_wave_barrier();
    float x[16];
    const int mo = opaque(m);
  #pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
  #pragma unroll
      for (int i = 0; i < r; ++i) acc += sqw[r * SA + i] * x[i];
      x[r] = (r < mo) ? 0.f : ((r == mo) ? 1.f : -acc);
    }
    __builtin_amdgcn_wave_barrier();
    if (g == 0) {
  #pragma unroll
      for (int r = 0; r < 16; ++r) sqw[r * SA + m] = x[r];  // column m of T_ww
    }
    __builtin_amdgcn_wave_barrier();
    const f32x4 tww_t = *reinterpret_cast<const f32x4*>(&sqw[m * SA + 4 * g]);  // Dl(T_ww^T)
    f32x4 tww;                                                                  // Dl(T_ww)
    const int go = opaque(g);
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y = x[i];
  #pragma unroll
      for (int gg = 1; gg < 4; ++gg)
        if (go == gg) y = x[4 * gg + i];
      tww[i] = y;
    }
    sm.tex[tex_slot(w, w)][l] = tww;
    f32x4 ttr[4];  // Dl(T_wJ^T), J <= w
  #pragma unroll
    for (int J = 0; J < 4; ++J) ttr[J] = (J == w) ? tww_t : f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();  // (2)

    // ---- off-diagonal tiles by distance d: X = sum_K A_wK T_KJ, T_wJ = -T_ww X
  #pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (w >= d) {
        const int J = w - d;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int K = 0; K < 3; ++K) {
          if (K >= J && K < w) {
            const f32x4 tkj = sm.tex[tex_slot(K, J)][l];
  #pragma unroll
            for (int s = 0; s < 4; ++s) X = mma_f32(a[K][s], tkj[s], X);
          }
        }
        f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int s = 0; s < 4; ++s) {
          Y = mma_f32(tww_t[s], X[s], Y);  // Dl(T_ww X)
          Z = mma_f32(X[s], tww_t[s], Z);  // Dl(X^T T_ww^T)
        }
        if (w < 3 && d < 3) sm.tex[tex_slot(w, J)][l] = -Y;
  #pragma unroll
        for (int JJ = 0; JJ < 3; ++JJ)
          if (JJ == J) ttr[JJ] = -Z;
      }
      if (d < 3) lds_barrier();  // (3), (4)
    }

    // ---- T1^T, T2^T fragments of the own rows (bf16 hi + lo), tiles J <= w
    bf16x4 t1h[4], t1l[4], t2h[4], t2l[4];
    const int dm2 = opaque(m) - 4 * g;  // i <= t  <=>  ii <= dm2 on the diagonal tile
  #pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
      if (J <= w) {  // T[t][i] = 0 on the tiles above the diagonal
  #pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * J + 4 * g + ii;
          const float tv = ttr[J][ii];  // T[t][i], zero for i > t
          const float bti = bts[i];
          x1[ii] = egt * tv * bti * sm.rk[i];
          // e^{G_t - G_i} overflows for i > t under strong decay: mask, do not multiply by 0
          const float ev = __builtin_amdgcn_exp2f((float)(G2t - G2[i])) * tv * bti;
          x2[ii] = (J < w || ii <= dm2) ? ev : 0.f;
        }
      }
      t1h[J] = to_bf16x4(x1);
      t1l[J] = to_bf16x4(x1 - to_f32x4(t1h[J]));
      t2h[J] = to_bf16x4(x2);
      t2l[J] = to_bf16x4(x2 - to_f32x4(t2h[J]));
    }
    const int ns = (w >> 1) + 1;  // token steps that hold tiles J <= w

    // ---- W<-^T = K^T T1^T for the own token columns: D tiles (dk 32sp + 16tt, rows t)
  #pragma unroll
    for (int sp = 0; sp < NKS; ++sp) {
      f32x4 acc[2];
  #pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s < ns) {
            const bf16x8 ka = bf16x8_from_u32x4(col_frag_tr(sm.ks, SK, 32 * sp + 16 * tt, s, g, m));
            acc[tt] = mma_bf16(ka, cat_bf(t1h[2 * s], t1h[2 * s + 1]), acc[tt]);
            acc[tt] = mma_bf16(ka, cat_bf(t1l[2 * s], t1l[2 * s + 1]), acc[tt]);
          }
        }
      }
      __builtin_nontemporal_store(cat(to_half4(acc[0]), to_half4(acc[1])), reinterpret_cast<half8*>(Wout + pair * C * DK + ((w * NKS + sp) * 64 + l) * 8));
    }

    // ---- U~ = T2 V for the own rows: D tiles (rows 16w.., dv 16cc..), each stored as one
    // contiguous 512-byte block (a wave writing whole cache lines)
  #pragma unroll
    for (int cc = 0; cc < DV / 16; ++cc) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s < ns) {
          const bf16x8 vb = bf16x8_from_u32x4(col_frag_tr(sm.qv, SQV, 16 * cc, s, g, m));
          acc = mma_bf16(cat_bf(t2h[2 * s], t2h[2 * s + 1]), vb, acc);
          acc = mma_bf16(cat_bf(t2l[2 * s], t2l[2 * s + 1]), vb, acc);
        }
      }
      __builtin_nontemporal_store(to_half4(acc), reinterpret_cast<half4*>(Uout + pair * C * DV + ((cc * 4 + w) * 64 + l) * 4));
    }
    if (tid < C) gates(nx, ib ^ 1);  // wave 0: the next item's gates
    // issued late so that these registers stay free through the item
    stage_k = !same_k(nx, cur);
    load_kq(nx, stage_k);
    lds_barrier();  // (5) every LDS region is free for the next item
    cur = nx;
  }
}

template <int DK, int DV>
hipError_t launch_prep_t(const void* q, const void* k, const void* v, const int64_t* cu,
                         int32_t* off, const int32_t* cseq, bool self_plan, const float* ga,
                         const float* gb, const float* A_log, const float* dt_bias,
                         const Shape& s, int64_t max_chunks, _Float16* w,
                         _Float16* u, _Float16* aqk, float* eg, _Float16* kf, _Float16* qf,
                         int32_t* nonfinite, hipStream_t st) {
  // Persistent grid: as many workgroups as fit on the device at once.
  auto kern = self_plan ? mfma_prep_kernel<DK, DV, true> : mfma_prep_kernel<DK, DV, false>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess)
    return hipErrorInvalidValue;
  const int64_t groups = max_chunks * s.H;  // (chunk, q/k head) groups
  const int64_t grid = std::min<int64_t>(groups, (int64_t)std::max(cus, 1) * std::max(per_cu, 1));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, cu, off, cseq, ga, gb, A_log,
                     dt_bias, (int)s.B, s.H, s.HV, s.short_len, w, u, aqk, eg, kf, qf, nonfinite);
  return hipGetLastError();
}


// ======================= C = 128 =======================
// The same quantities over chunks of 128 rows (the chunk size the pymllm page's Torch
// function defaults to, Module Contents), in the state pass's fragment orders at C = 128
// (eight row tiles, four 32-token steps): one workgroup of eight waves per (chunk, value
// head), wave w owning chunk rows 16w .. 16w + 15. The structure follows the C = 64 kernel
// with these differences: the inverse has eight diagonal tiles and distances up to 7, so
// every exchanged tile T_IJ (I <= 6) stays in LDS; Q is not staged (each wave loads the
// fragments of its own rows from global memory); V is staged into the K region once W<-
// and K~ are formed; the Grams accumulate dk step by dk step over all tiles J <= w
// (registers for eight tile pairs instead of the operand fragments of every step); the
// chunk table comes from the plan kernel, one item per workgroup. The Grams, the inverse
// and the products with T grow with C per row, so this kernel does about 1.6x the work per
// token of the C = 64 one (measured: 152 against 99 us on the dense batch).
constexpr int C2 = 128;
constexpr int NRT2 = C2 / 16;  // row tiles
constexpr int NTS2 = C2 / 32;  // token steps

template <int DK, int DV>
struct Prep128Smem {
  static constexpr int SKV = (DK > DV ? DK : DV) + 16;  // row stride (bf16), as at C = 64
  uint16_t kv[C2 * SKV];  // K rows, later V rows
  f32x4 tex[28][64];       // Dl(T_IJ) for I <= 6, at slot I (I + 1) / 2 + J
  float sq[8][16 * SA];    // per-wave scratch: A_ww, then the columns of T_ww
  double G2[C2];  // G log2(e)
  float bt[C2];   // beta
  float rk[C2];   // r_k
};

__device__ __forceinline__ int tex2_slot(int I, int J) { return I * (I + 1) / 2 + J; }

// Rows of a row-major bf16 tile of C2 rows into registers (512 threads), zeros past n.
template <int D>
__device__ __forceinline__ void load_rows128(u32x4 (&r)[C2 * D / 8 / 512], const uint16_t* src,
                                             int64_t rs, int n, int tid) {
#pragma unroll
  for (int u = 0; u < C2 * D / 8 / 512; ++u) {
    const int e = tid + 512 * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (row < n) z = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + row * rs + c8));
    r[u] = z;
  }
}
template <int D>
__device__ __forceinline__ void store_rows128(uint16_t* dst, int ld,
                                              const u32x4 (&r)[C2 * D / 8 / 512], int tid) {
#pragma unroll
  for (int u = 0; u < C2 * D / 8 / 512; ++u) {
    const int e = tid + 512 * u, row = e / (D / 8), c8 = (e % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(&dst[row * ld + c8]) = r[u];
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(512, (DK + DV <= 256) ? 4 : 2) void mfma_prep128_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ chunk_seq, const float* __restrict__ ga,
    const float* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, int H, int HV, _Float16* __restrict__ Wout,
    _Float16* __restrict__ Uout, _Float16* __restrict__ Aout, float* __restrict__ eg_out,
    _Float16* __restrict__ Kout, _Float16* __restrict__ Qout, int32_t* __restrict__ nonfinite) {
  constexpr int C = C2;
  constexpr int NKS = DK / 32;
  using Sm = Prep128Smem<DK, DV>;
  constexpr int SKV = Sm::SKV;
  constexpr int KP = C * DK / 8 / 512;  // 16-byte pieces per thread of the K tile
  constexpr int VP = C * DV / 8 / 512;  // ... of the V tile
  __shared__ Sm sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int t = 16 * w + m;  // this lane's chunk row
  if (blockIdx.x == 0 && tid == 0) *nonfinite = 0;  // the state pass raises it
  const int64_t c = blockIdx.x / HV;
  const int hv = (int)(blockIdx.x % HV);
  const int32_t seq = chunk_seq[c];
  if (seq < 0) return;  // unused chunk slot (uniform over the workgroup)
  const int h = hv / (HV / H);
  const int64_t t0 = cu[seq] + (int64_t)(c - chunk_off[seq]) * C;
  const int n = (int)min((int64_t)C, cu[seq + 1] - t0);
  const int64_t pair = c * HV + hv;
  const int64_t rsk = (int64_t)H * DK;

  // ---- loads: K and V rows (V is staged later), the own row of Q as Gram operand
  // fragments (elements 32 sp + 8g .. 32 sp + 8g + 7), zeros past n
  u32x4 kreg[KP], vreg[VP];
  load_rows128<DK>(kreg, k + (t0 * H + h) * (int64_t)DK, rsk, n, tid);
  const uint16_t* qrow = q + ((t0 + t) * H + h) * (int64_t)DK;
  u32x4 qf[NKS];
#pragma unroll
  for (int sp = 0; sp < NKS; ++sp)
    qf[sp] = t < n ? *reinterpret_cast<const u32x4*>(qrow + 32 * sp + 8 * g)
                   : u32x4{0u, 0u, 0u, 0u};

  // ---- gates (wave 0; lane l takes rows l and 64 + l): g = log(alpha) =
  // -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), zero on padding rows; G = the
  // chunk-local inclusive sum of g in fp64
  if (w == 0) {
    double G[2];
    float bt[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = l + 64 * j;
      float gt = 0.f;
      bt[j] = 0.f;
      if (r < n) {
        const int64_t tr = t0 + r;
        const float xg = ga[tr * HV + hv] + dt_bias[hv];
        const float sp = fmaxf(xg, 0.f) + log1pf(expf(-fabsf(xg)));
        gt = -expf(A_log[hv]) * sp;
        bt[j] = 1.f / (1.f + expf(-gb[tr * HV + hv]));
      }
      G[j] = (double)gt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(G[j], off, 64);
        if (l >= off) G[j] += y;
      }
    }
    G[1] += __shfl(G[0], 63, 64);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sm.G2[l + 64 * j] = G[j] * kLog2e;
      sm.bt[l + 64 * j] = bt[j];
    }
  }
  store_rows128<DK>(sm.kv, SKV, kreg, tid);
  lds_barrier();  // (0) K staged, gates

  // ---- norms of the own rows (the four lane groups hold one row)
  float kss = 0.f, qss = 0.f;
#pragma unroll
  for (int sp = 0; sp < NKS; ++sp) {
    const u32x4 kx = *reinterpret_cast<const u32x4*>(sm.kv + t * SKV + 32 * sp + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kss += bf_lo(kx[j]) * bf_lo(kx[j]) + bf_hi(kx[j]) * bf_hi(kx[j]);
      qss += bf_lo(qf[sp][j]) * bf_lo(qf[sp][j]) + bf_hi(qf[sp][j]) * bf_hi(qf[sp][j]);
    }
  }
  kss += __shfl_xor(kss, 16, 64);
  kss += __shfl_xor(kss, 32, 64);
  qss += __shfl_xor(qss, 16, 64);
  qss += __shfl_xor(qss, 32, 64);
  const float rkt = 1.0f / sqrtf(kss + kNormEps);
  const float rqt = 1.0f / sqrtf(qss + kNormEps);
  if (g == 0) sm.rk[t] = rkt;

  // ---- normalised q in the state pass's operand order (elements 32 sp + kperm(g, .),
  // the row read again in that order: cache hits), once per q/k head
  if (hv % (HV / H) == 0) {
    const int64_t fo = (c * H + h) * (int64_t)(C * DK);
#pragma unroll
    for (int sp = 0; sp < NKS; ++sp) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (t < n) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(qrow + 32 * sp + 4 * g);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(qrow + 32 * sp + 16 + 4 * g);
        x = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      half8 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = (_Float16)(bf_lo(x[j]) * rqt);
        y[2 * j + 1] = (_Float16)(bf_hi(x[j]) * rqt);
      }
      __builtin_nontemporal_store(y, reinterpret_cast<half8*>(Qout + fo + ((w * NKS + sp) * 64 + l) * 8));
    }
  }
  lds_barrier();  // (1) r_k visible

  // ---- Grams of the own rows against tiles J <= w, transposed, dk step by dk step:
  // D[J] = Dl(K_J K_w^T), E[J] = Dl(K_J Q_w^T); lane (g, m): row 16J + 4g + i, column t
  f32x4 D[NRT2], E[NRT2];
#pragma unroll
  for (int J = 0; J < NRT2; ++J) {
    D[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    E[J] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int sp = 0; sp < NKS; ++sp) {
    const bf16x8 kws =
        bf16x8_from_u32x4(*reinterpret_cast<const u32x4*>(sm.kv + t * SKV + 32 * sp + 8 * g));
    const bf16x8 qws = bf16x8_from_u32x4(qf[sp]);
#pragma unroll
    for (int J = 0; J < NRT2; ++J) {
      if (J < w) {
        const bf16x8 kj = bf16x8_from_u32x4(
            *reinterpret_cast<const u32x4*>(sm.kv + (16 * J + m) * SKV + 32 * sp + 8 * g));
        D[J] = mma_bf16(kj, kws, D[J]);
        E[J] = mma_bf16(kj, qws, E[J]);
      } else if (J == w) {
        D[J] = mma_bf16(kws, kws, D[J]);
        E[J] = mma_bf16(kws, qws, E[J]);
      }
    }
  }

  // ---- scale: a[J] = Dl(A_wJ^T) (A[t][i], i = 16J + 4g + ii < t) and the A_qk rows
  const double G2t = sm.G2[t];
  const float btt = sm.bt[t];
  const float egt = __builtin_amdgcn_exp2f((float)G2t);
  if (g == 0) eg_out[pair * C + t] = egt;
  const int dm = opaque(m) - 4 * g;  // i < t  <=>  ii < dm on the diagonal tile
  f32x4 a[NRT2];
#pragma unroll
  for (int s = 0; s < NTS2; ++s) {
    half4 aq[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int J = 2 * s + jj;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      a[J] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * J + 4 * g + ii;
          const float rki = sm.rk[i];
          const float av = btt * rkt * rki * D[J][ii];
          // e^{G_t - G_i} overflows for i > t under strong decay: masked, not multiplied
          const float xv = __builtin_amdgcn_exp2f((float)(G2t - sm.G2[i])) * rqt * rki * E[J][ii];
          a[J][ii] = (J < w || ii < dm) ? av : 0.f;
          x[ii] = (J < w || ii <= dm) ? xv : 0.f;
        }
      }
      aq[jj] = to_half4(x);
    }
    // token steps past the own row tile lie above the diagonal: never read
    if (2 * s <= w)
      __builtin_nontemporal_store(cat(aq[0], aq[1]), reinterpret_cast<half8*>(Aout + pair * C * C + ((w * NTS2 + s) * 64 + l) * 8));
  }

  // ---- K~ = diag(e^{G_n - G} r_k) K in fp16: fragment f = (sp * 2 + tt) * 4 + s holds
  // K~^T rows 32sp + 16tt + m, tokens 32s + kperm(g, .); wave w writes f = w (mod 8)
  {
    const int s = w & 3, tt = w >> 2;
    float kdj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tk = 32 * s + kperm(g, j);
      kdj[j] = __builtin_amdgcn_exp2f((float)(sm.G2[C - 1] - sm.G2[tk])) * sm.rk[tk];
    }
    half8* kb = reinterpret_cast<half8*>(Kout + pair * (int64_t)(C * DK)) + w * 64 + opaque(l);
#pragma unroll
    for (int sp = 0; sp < NKS; ++sp) {
      const u32x4 x = col_frag_tr(sm.kv, SKV, 32 * sp + 16 * tt, s, g, m);
      half8 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = (_Float16)(bf_lo(x[j]) * kdj[2 * j]);
        y[2 * j + 1] = (_Float16)(bf_hi(x[j]) * kdj[2 * j + 1]);
      }
      __builtin_nontemporal_store(y, kb + sp * 8 * 64);
    }
  }

  // ---- diagonal tile: T_ww = (I + A_ww)^-1 by forward substitution, lane = column m
  float* sqw = sm.sq[w];
  {
    f32x4 aw = a[0];
#pragma unroll
    for (int J = 1; J < NRT2; ++J)
      if (J == w) aw = a[J];
    *reinterpret_cast<f32x4*>(&sqw[m * SA + 4 * g]) = aw;  // row m of A_ww, columns 4g..
  }
  __builtin_amdgcn_wave_barrier();
  float x[16];
  const int mo = opaque(m);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < r; ++i) acc += sqw[r * SA + i] * x[i];
    x[r] = (r < mo) ? 0.f : ((r == mo) ? 1.f : -acc);
  }
  __builtin_amdgcn_wave_barrier();
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sqw[r * SA + m] = x[r];  // column m of T_ww
  }
  __builtin_amdgcn_wave_barrier();
  const f32x4 tww_t = *reinterpret_cast<const f32x4*>(&sqw[m * SA + 4 * g]);  // Dl(T_ww^T)
  f32x4 tww;                                                                  // Dl(T_ww)
  const int go = opaque(g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y = x[i];
#pragma unroll
    for (int gg = 1; gg < 4; ++gg)
      if (go == gg) y = x[4 * gg + i];
    tww[i] = y;
  }
  if (w < 7) sm.tex[tex2_slot(w, w)][l] = tww;
  f32x4 ttr[NRT2];  // Dl(T_wJ^T), J <= w
#pragma unroll
  for (int J = 0; J < NRT2; ++J) ttr[J] = (J == w) ? tww_t : f32x4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();  // (2)

  // ---- off-diagonal tiles by distance d: X = sum_{J <= K < w} A_wK T_KJ, T_wJ = -T_ww X
#pragma unroll
  for (int d = 1; d < NRT2; ++d) {
    if (w >= d) {
      const int J = w - d;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NRT2 - 1; ++K) {
        if (K >= J && K < w) {
          const f32x4 tkj = sm.tex[tex2_slot(K, J)][l];
#pragma unroll
          for (int s = 0; s < 4; ++s) X = mma_f32(a[K][s], tkj[s], X);
        }
      }
      f32x4 Y = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Y = mma_f32(tww_t[s], X[s], Y);  // Dl(T_ww X)
        Z = mma_f32(X[s], tww_t[s], Z);  // Dl(X^T T_ww^T)
      }
      if (w < 7) sm.tex[tex2_slot(w, J)][l] = -Y;  // read at larger distances
#pragma unroll
      for (int JJ = 0; JJ < NRT2 - 1; ++JJ)
        if (JJ == J) ttr[JJ] = -Z;
    }
    if (d < NRT2 - 1) lds_barrier();  // (3) .. (8)
  }

  load_rows128<DV>(vreg, v + (t0 * HV + hv) * (int64_t)DV, (int64_t)HV * DV, n, tid);

  // ---- W<-^T = K^T T1^T for the own token columns, T1 = diag(e^G) T diag(beta r_k) in
  // bf16 hi + lo: D tiles (dk 32sp + 16tt, rows t)
  const int ns = (w >> 1) + 1;  // token steps that hold tiles J <= w
  {
    bf16x4 t1h[NRT2], t1l[NRT2];
#pragma unroll
    for (int J = 0; J < NRT2; ++J) {
      f32x4 x1 = {0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * J + 4 * g + ii;
          x1[ii] = egt * ttr[J][ii] * sm.bt[i] * sm.rk[i];  // T[t][i] is zero for i > t
        }
      }
      t1h[J] = to_bf16x4(x1);
      t1l[J] = to_bf16x4(x1 - to_f32x4(t1h[J]));
    }
#pragma unroll
    for (int sp = 0; sp < NKS; ++sp) {
      f32x4 acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NTS2; ++s) {
          if (s < ns) {
            const bf16x8 ka = bf16x8_from_u32x4(col_frag_tr(sm.kv, SKV, 32 * sp + 16 * tt, s, g, m));
            acc[tt] = mma_bf16(ka, cat_bf(t1h[2 * s], t1h[2 * s + 1]), acc[tt]);
            acc[tt] = mma_bf16(ka, cat_bf(t1l[2 * s], t1l[2 * s + 1]), acc[tt]);
          }
        }
      }
      __builtin_nontemporal_store(cat(to_half4(acc[0]), to_half4(acc[1])), reinterpret_cast<half8*>(Wout + pair * C * DK + ((w * NKS + sp) * 64 + l) * 8));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();  // (9) the K tile is no longer read
  store_rows128<DV>(sm.kv, SKV, vreg, tid);

  // ---- T2 = (Gamma o T) diag(beta) in bf16 hi + lo, tiles J <= w
  bf16x4 t2h[NRT2], t2l[NRT2];
  const int dm2 = opaque(m) - 4 * g;  // i <= t  <=>  ii <= dm2 on the diagonal tile
#pragma unroll
  for (int J = 0; J < NRT2; ++J) {
    f32x4 x2 = {0.f, 0.f, 0.f, 0.f};
    if (J <= w) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * J + 4 * g + ii;
        const float ev = __builtin_amdgcn_exp2f((float)(G2t - sm.G2[i])) * ttr[J][ii] * sm.bt[i];
        x2[ii] = (J < w || ii <= dm2) ? ev : 0.f;
      }
    }
    t2h[J] = to_bf16x4(x2);
    t2l[J] = to_bf16x4(x2 - to_f32x4(t2h[J]));
  }
  lds_barrier();  // (10) V staged

  // ---- U~ = T2 V for the own rows: D tiles (rows 16w.., dv 16cc..)
#pragma unroll
  for (int cc = 0; cc < DV / 16; ++cc) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NTS2; ++s) {
      if (s < ns) {
        const bf16x8 vb = bf16x8_from_u32x4(col_frag_tr(sm.kv, SKV, 16 * cc, s, g, m));
        acc = mma_bf16(cat_bf(t2h[2 * s], t2h[2 * s + 1]), vb, acc);
        acc = mma_bf16(cat_bf(t2l[2 * s], t2l[2 * s + 1]), vb, acc);
      }
    }
    __builtin_nontemporal_store(to_half4(acc), reinterpret_cast<half4*>(Uout + pair * C * DV + ((cc * NRT2 + w) * 64 + l) * 4));
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int DK, int DV>
hipError_t launch_prep128_t(const void* q, const void* k, const void* v, const int64_t* cu,
                            const int32_t* off, const int32_t* cseq, const float* ga,
                            const float* gb, const float* A_log, const float* dt_bias,
                            const Shape& s, int64_t max_chunks, _Float16* w, _Float16* u,
                            _Float16* aqk, float* eg, _Float16* kf, _Float16* qf,
                            int32_t* nonfinite, hipStream_t st) {
  const int64_t items = max_chunks * s.HV;  // (chunk, value head); unused chunks return
  hipLaunchKernelGGL((mfma_prep128_kernel<DK, DV>), dim3((unsigned)items), dim3(512), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, cu, off, cseq,
                     ga, gb, A_log, dt_bias, s.H, s.HV, w, u, aqk, eg, kf, qf, nonfinite);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_prep(const void* q, const void* k, const void* v,
                            const int64_t* cu_seqlens, int32_t* chunk_off,
                            const int32_t* chunk_seq, bool self_plan, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            const Shape& s, int64_t max_chunks, void* w, void* u, void* aqk,
                            float* eg, void* kf, void* qf, int32_t* nonfinite, hipStream_t st) {
  if (self_plan && (s.B > kMaxSelfPlanRequests || s.C != 64)) return hipErrorInvalidValue;
  _Float16* W = (_Float16*)w;
  _Float16* U = (_Float16*)u;
  if (s.C == 128) {
#define GDN_PREP128_CASE(DKv, DVv)                                                           \
  if (s.dk == DKv && s.dv == DVv)                                                            \
    return launch_prep128_t<DKv, DVv>(q, k, v, cu_seqlens, chunk_off, chunk_seq, a, b, A_log, \
                                      dt_bias, s, max_chunks, W, U, (_Float16*)aqk, eg,     \
                                      (_Float16*)kf, (_Float16*)qf, nonfinite, st);
    GDN_PREP128_CASE(128, 64)
    GDN_PREP128_CASE(128, 128)
    GDN_PREP128_CASE(128, 256)
    GDN_PREP128_CASE(256, 64)
    GDN_PREP128_CASE(256, 128)
    GDN_PREP128_CASE(256, 256)
#undef GDN_PREP128_CASE
    return hipErrorInvalidValue;
  }
  if (s.C != 64) return hipErrorInvalidValue;
#define GDN_PREP_CASE(DKv, DVv)                                                               \
  if (s.dk == DKv && s.dv == DVv)                                                             \
    return launch_prep_t<DKv, DVv>(q, k, v, cu_seqlens, chunk_off, chunk_seq, self_plan, a, b, \
                                   A_log,                                                      \
                                   dt_bias, s,                                                 \
                                   max_chunks, W, U, (_Float16*)aqk, eg, (_Float16*)kf,      \
                                   (_Float16*)qf, nonfinite, st);
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
