// Sequential state pass over chunks with whole state blocks per workgroup, and the scan over
// segments of a long request (bf16 inputs, dk <= 128).
//
// Per chunk, in row convention (pymllm gdn_chunkwise page, Algorithm steps 2-3; "Simple
// math to speed up GDN prefill", Reminder, the chunkwise transition with decorated S->,
// W<-, K->):
//   U     = U~ - W<- S^T
//   O     = diag(e^G) Qh S^T + A_qk U                                   (to out)
//   S^T  <- e^{G_n} S^T + K~^T U,   K~ = diag(e^{G_n - G} r_k) K
// The chunk-prep kernel has already formed W<-, U~, K~, Qh = diag(r_q) Q, A_qk and e^G
// (they depend on no state) in MFMA fragment order.
//
// One chunk's transition is an affine map of the state: S -> S A_c + U~^T K~ with the
// dk x dk operator A_c = e^{G_n} I - W<-^T K~. A request of many chunks is therefore cut
// into segments of at most `lseg` chunks (pymllm page: the inter-chunk propagation is the
// only sequential part):
//   operator pass  every segment but the last runs its chunks from the zero state (R_g)
//                  and from the identity with U~ = 0 (P_g, the product of its operators);
//   combine        S_{g+1} = S_g P_g + R_g in fp32, in order, from the slot's state;
//   output pass    every segment runs its chunks again from its true start state S_g,
//                  writing O; the last one writes the final state back into the slot.
// Segments of one request run on different compute units, so the chain each workgroup
// walks is at most lseg chunks long.
//
// Workgroup: eight compute waves (two per SIMD: one wave alone cannot keep the matrix
// core or the LDS busy) and one loader wave. In the output pass compute wave w holds 16
// columns of S^T (state rows of the value head) over all of dk in fp32 registers, as MFMA
// accumulator tiles; in the operator pass waves 0-3 hold 32 columns of R^T each and waves
// 4-7 32 columns of P^T. Each wave does every product of its columns itself: nothing is
// exchanged between compute waves. The operands every column needs (W<-, K~, Qh, A_qk,
// e^G; and the workgroup's columns of U~) are staged once per workgroup by the loader
// wave with direct global-to-LDS loads into a ring of two chunk slots, one chunk ahead of
// the compute waves; one barrier per chunk hands a slot over. Compute waves issue no
// global loads inside the chunk loop, only the stores of O.
//
// Matrix-core operands are fp16 with fp32 accumulation: W<- and S for W<- S^T; Qh and S
// for Qh S^T; A_qk and U for A_qk U; K~ and U for the update. The state stays fp32.
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

using namespace mfma;
constexpr int C = 64;
constexpr int kComputeWaves = 4;
constexpr int kLoaderWaves = 1;
constexpr int kColsPerBlock = 128;  // state columns of one workgroup

typedef __attribute__((address_space(3))) void* lds_ptr;

// Roles of a compute wave.
enum : int { kRoleOut = 0, kRoleR = 1, kRoleP = 2 };
// Kernel modes: the output pass (four compute waves, role out) or the operator pass (four
// compute waves of role R, whose state starts at zero, and four of role P, whose state
// starts at the identity and sees U~ = 0; the two share every staged W<- and K~).
enum : int { kModeOut = 0, kModeOperator = 1 };
template <int MODE>
constexpr int kCompute = 2 * kComputeWaves;  // two compute waves per SIMD
// 16-column tiles per compute wave: eight waves of 16 columns (out) or of 32 (R, P)
template <int MODE>
constexpr int kTiles = MODE == kModeOut ? 1 : 2;
template <int MODE>
constexpr int kThreads = 64 * (kCompute<MODE> + kLoaderWaves);

// s_waitcnt vmcnt(N), the other counters not waited for (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1: every index is a compile-time
// constant, so register arrays indexed by it stay in registers.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One ring slot: every operand of one chunk, each fragment 1 KiB (lane l's 16 bytes at
// offset 16 l), exactly as the chunk prep wrote them.
template <int DK, int MODE>
struct Slot {
  static constexpr int NKS = DK / 32;
  static constexpr int FW = 4 * NKS;                        // W<-: 4 token tiles x dk steps
  static constexpr int FK = (DK / 16) * 2;                  // K~^T: dk tiles x 2 token steps
  static constexpr int FQ = MODE == kModeOut ? 4 * NKS : 0; // Qh: 4 token tiles x dk steps
  static constexpr int FA = MODE == kModeOut ? 8 : 0;       // A_qk: 4 token tiles x 2 steps
  static constexpr int FU = kColsPerBlock / 8;              // U~: 2 D tiles per KiB
  half8 w[FW][64];
  half8 k[FK][64];
  half8 q[FQ > 0 ? FQ : 1][64];
  half8 a[FA > 0 ? FA : 1][64];
  half8 u[FU][64];
  float eg[C];
};

template <int DK, int MODE>
struct ChainSmem {
  Slot<DK, MODE> s[2];
};

struct ChainArgs {
  const _Float16* W;    // W<-  [chunk][HV][C*dk]
  const _Float16* U;    // U~   [chunk][HV][C*dv]
  const _Float16* Kf;   // K~   [chunk][HV][C*dk]
  const _Float16* Qf;   // Qh   [chunk][H][C*dk]
  const _Float16* Aqk;  // A_qk [chunk][HV][C*C]
  const float* eg;      // e^G  [chunk][HV][C]
  const int64_t* cu;
  const int64_t* cache_indices;
  const int32_t* chunk_off;
  float* state_pool;
  uint16_t* out;
  float* rp;      // [segment][HV][dv + dk][dk]: R_g rows, then P_g rows
  float* sstart;  // [segment][HV][dv][dk]: start state of every segment of a cut request
  int32_t* nonfinite;  // raised by the output pass if a final state is not finite
  int B, H, HV, DV;
  int64_t short_len;  // requests of at most this many tokens are not chunked
  int lseg;       // chunks per segment
  int segmented;  // requests may be cut (at most 64 requests)
  int nb;         // workgroups per (segment, value head): 128-column blocks
  int64_t groups; // (segment, q/k head) groups covered by the grid
};

// Segment sg of the call -> its request b, its index j in the request and the request's
// segment count. With cut requests (B <= 64) every wave forms the segment table with one
// scan: request b has ceil(ceil(L_b / C) / lseg) segments. Returns false past the last
// segment.
__device__ __forceinline__ bool find_segment(const ChainArgs& a, int64_t sg, int l, int& b,
                                             int& j, int& nseg, int& seg0) {
  if (!a.segmented) {
    if (sg >= a.B) return false;
    b = (int)sg;
    j = 0;
    nseg = 1;
    seg0 = (int)sg;
    return true;
  }
  int ns = 0;
  if (l < a.B) {
    const int64_t L = a.cu[l + 1] - a.cu[l];
    const int64_t nch = path_chunks(L, C, a.short_len);
    ns = (int)((nch + a.lseg - 1) / a.lseg);
  }
  int incl = ns;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (l >= off) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  if (sg >= total) return false;
  // the owner of segment sg: the number of requests whose segments all precede it
  b = __popcll(__ballot(l < a.B && incl <= sg));
  const int incl_b = __shfl(incl, b, 64);
  nseg = __shfl(ns, b, 64);
  seg0 = incl_b - nseg;
  j = (int)sg - seg0;
  return true;
}

template <int DK, int MODE>
__global__ __launch_bounds__(kThreads<MODE>, 1) void chain_kernel(ChainArgs a) {
  constexpr int NKS = DK / 32;  // 32-wide dk steps
  constexpr int NDT = DK / 16;  // 16-row dk tiles
  using Sl = Slot<DK, MODE>;
  __shared__ ChainSmem<DK, MODE> sm;

  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  // The workgroups of one (segment, q/k head) group -- its HV/H value heads times the nb
  // column blocks -- share blockIdx.x mod 8, so they run on one XCD and read the group's
  // normalised q blocks once from its L2.
  const int rv = a.HV / a.H;
  const int members = rv * a.nb;
  const int64_t x = blockIdx.x;
  const int64_t rest = x >> 3;
  const int member = (int)(rest % members);
  const int64_t grp = (rest / members) * 8 + (x & 7);
  if (grp >= a.groups) return;
  const int64_t sg = grp / a.H;
  const int hv = (int)(grp % a.H) * rv + member / a.nb;
  const int blk = member % a.nb;
  int b, j, nseg, seg0;
  if (!find_segment(a, sg, l, b, j, nseg, seg0)) return;
  const int64_t L = a.cu[b + 1] - a.cu[b];
  const int nch = (int)path_chunks(L, C, a.short_len);
  if (nch == 0) return;  // empty (slot untouched) or evaluated by the token recurrence
  const int c_lo = j * a.lseg;
  const int n = min(c_lo + a.lseg, nch) - c_lo;  // chunks of this segment (>= 1)
  if constexpr (MODE == kModeOperator)
    if (nseg < 2 || j == nseg - 1) return;  // the last segment's operator is never used
  const int colbase = blk * kColsPerBlock;
  const int ncols_u = max(0, min(kColsPerBlock, a.DV - colbase));  // staged U~ columns
  const int h = hv / (a.HV / a.H);
  const int64_t slot = a.cache_indices[b];
  const int64_t cbase = (int64_t)a.chunk_off[b] + c_lo;  // global index of chunk 0
  const int64_t tseq = a.cu[b] + (int64_t)c_lo * C;      // first token of chunk 0
  const int64_t tend = a.cu[b + 1];

  if (wv >= kCompute<MODE>) {
    // ======================= loader waves =======================
    // The chunk's fragments are numbered W<-, K~, (Qh, A_qk), (U~), e^G; loader wave lw
    // copies those with number = lw mod kLoaderWaves.
    const int lw = wv - kCompute<MODE>;
    auto copy = [&](int idx, const char* src, void* dst) {
      if (idx % kLoaderWaves == lw)
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)dst, 16, 0, 0);
    };
    auto issue = [&](int cl) {
      Sl& s = sm.s[cl & 1];
      const int64_t pair = (cbase + cl) * a.HV + hv;
      const char* wsrc = reinterpret_cast<const char*>(a.W + pair * C * DK) + 16 * l;
      const char* ksrc = reinterpret_cast<const char*>(a.Kf + pair * C * DK) + 16 * l;
      int idx = 0;
#pragma unroll
      for (int f = 0; f < Sl::FW; ++f) copy(idx++, wsrc + 1024 * f, &s.w[f][0]);
#pragma unroll
      for (int f = 0; f < Sl::FK; ++f) copy(idx++, ksrc + 1024 * f, &s.k[f][0]);
      if constexpr (MODE == kModeOut) {
        const char* qsrc =
            reinterpret_cast<const char*>(a.Qf + ((cbase + cl) * a.H + h) * (int64_t)(C * DK)) +
            16 * l;
        const char* asrc = reinterpret_cast<const char*>(a.Aqk + pair * C * C) + 16 * l;
#pragma unroll
        for (int f = 0; f < Sl::FQ; ++f) copy(idx++, qsrc + 1024 * f, &s.q[f][0]);
        // A_qk fragments (token tile I, token step st) = 2 I + st; the two above the
        // diagonal (I < 2, st = 1) are zero and were never written
#pragma unroll
        for (int f = 0; f < 8; ++f)
          if (f != 1 && f != 3) copy(idx++, asrc + 1024 * f, &s.a[f][0]);
      }
      if (ncols_u > 0) {
        // the workgroup's column tiles of U~: ncols_u / 8 contiguous KiB
        const char* usrc =
            reinterpret_cast<const char*>(a.U + pair * C * a.DV + (int64_t)colbase * C) + 16 * l;
        const int nu = ncols_u / 8;
        for (int f = 0; f < nu; ++f) copy(idx + f, usrc + 1024 * f, &s.u[f][0]);
        idx += nu;
      }
      if (idx % kLoaderWaves == lw)
        __builtin_amdgcn_global_load_lds((const void*)(a.eg + pair * C + l), (lds_ptr)&s.eg[0], 4,
                                         0, 0);
    };
    issue(0);
    for (int cl = 0; cl < n; ++cl) {
      wait_vmcnt<0>();  // chunk cl has landed in its slot
      lds_barrier();    // hand slot cl & 1 over; slot (cl + 1) & 1 is free again
      if (cl + 1 < n) issue(cl + 1);
    }
    return;
  }

  // ======================= compute waves =======================
  constexpr int CT = kTiles<MODE>;
  const int role = MODE == kModeOut ? kRoleOut : (wv < kComputeWaves ? kRoleR : kRoleP);
  const int wct = MODE == kModeOut ? wv : CT * (wv % kComputeWaves);  // first column tile
  const int col0 = colbase + 16 * wct;  // first state (or P) column of this wave
  const bool active = col0 < (role == kRoleP ? DK : a.DV);
  const bool use_u = role != kRoleP;
  // S^T tiles: dk rows 16 dt + 4 g + i, column col0 + 16 ct + m (fp32)
  f32x4 S[NDT][CT];
  float* Sinit = nullptr;
  if (role == kRoleOut)
    Sinit = (nseg >= 2) ? a.sstart + ((sg * a.HV + hv) * (int64_t)a.DV + col0) * DK
                        : a.state_pool + ((slot * a.HV + hv) * (int64_t)a.DV + col0) * DK;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (role == kRoleOut && active) {
        S[dt][ct] = *reinterpret_cast<const f32x4*>(Sinit + (16 * ct + m) * DK + 16 * dt + 4 * g);
      } else if (role == kRoleP) {
        // identity: row 16 dt + 4 g + i equals column col0 + 16 ct + m
        const int d = col0 + 16 * ct + m - (16 * dt + 4 * g);
        S[dt][ct] = f32x4{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f,
                          d == 3 ? 1.f : 0.f};
      } else {
        S[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  // One chunk is a fixed sequence of NF fragment steps; each step reads one operand
  // fragment from the slot and issues the two MFMAs (one per column tile) that use it:
  //   W<- S^T     P  = 4 NKS steps (ks-major: consecutive steps feed different tokens)
  //   Qh S^T      O1 = 4 NKS steps (output pass)
  //   A_qk U      O2 = 6 steps     (output pass; the two tiles above the diagonal skipped)
  //   K~^T U      UP = 2 NDT steps (token-step-major)
  // Fragments are read RING steps ahead into a register ring, and a scheduling barrier
  // after each step keeps that distance, so an LDS read has RING - 1 steps of matrix work
  // to land.
  constexpr int RING = MODE == kModeOut ? 8 : 6;
  constexpr int P = 4 * NKS;
  constexpr int O1 = MODE == kModeOut ? 4 * NKS : 0;
  constexpr int O2 = MODE == kModeOut ? 6 : 0;
  constexpr int UP = 2 * NDT;
  constexpr int NF = P + O1 + O2 + UP;
  // A_qk fragment 2 tt + st of the O2 steps: (tt, st) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
  auto frag = [&](const Sl& s, auto I) -> const half8* {
    constexpr int i = decltype(I)::value;
    if constexpr (i < P) {
      return &s.w[(i % 4) * NKS + i / 4][l];
    } else if constexpr (i < P + O1) {
      return &s.q[((i - P) % 4) * NKS + (i - P) / 4][l];
    } else if constexpr (i < P + O1 + O2) {
      constexpr int j2 = i - P - O1;
      return &s.a[j2 < 2 ? 2 * j2 : j2 + 2][l];
    } else {
      constexpr int j2 = i - P - O1 - O2;
      return &s.k[(j2 % NDT) * 2 + j2 / NDT][l];
    }
  };

  for (int cl = 0; cl < n; ++cl) {
    lds_barrier();  // chunk cl's operands are in slot cl & 1
    if (!active) continue;
    const Sl& s = sm.s[cl & 1];
    half8 ring[RING];
    static_for<RING>([&](auto I) { ring[decltype(I)::value] = *frag(s, I); });
    // ---- fp16 copy of S^T: B operand (k = dk) of W<- S^T and A operand of S Qh^T
    half8 s16[NKS][CT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        s16[ks][ct] = cat(to_half4(S[2 * ks][ct]), to_half4(S[2 * ks + 1][ct]));
    // ---- -U = W<- S^T - U~, accumulated from -U~ (token tile tt, column tile ct)
    f32x4 nu[4][CT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (use_u) {
          const u32x2 ur = *reinterpret_cast<const u32x2*>(
              reinterpret_cast<const _Float16*>(&s.u[0][0]) + (((wct + ct) * 4 + tt) * 64 + l) * 4);
          const half4 uh = __builtin_bit_cast(half4, ur);
          nu[tt][ct] = f32x4{-(float)uh[0], -(float)uh[1], -(float)uh[2], -(float)uh[3]};
        } else {
          nu[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    half8 u16[2][CT];          // U in fp16, tokens 32 ts + kperm (B of the update, A of O2)
    f32x4 o[4][CT];            // O^T tiles (column tile ct, token tile tt)
    const int64_t t0 = tseq + (int64_t)cl * C;
    const int nrow = (int)min((int64_t)C, tend - t0);
    static_for<NF>([&](auto I) {
      constexpr int i = decltype(I)::value;
      // phase boundaries
      if constexpr (i == P + O1) {
        // U in fp16 (P's products finished during the O1 steps)
#pragma unroll
        for (int ts = 0; ts < 2; ++ts)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            u16[ts][ct] = cat(to_half4(-nu[2 * ts][ct]), to_half4(-nu[2 * ts + 1][ct]));
        if constexpr (MODE == kModeOut) {
          // O1 rows scaled by e^G before A_qk U is added
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const float er = s.eg[16 * tt + m];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) o[tt][ct] *= er;
          }
        }
      }
      if constexpr (i == P + O1 + O2) {
        if constexpr (MODE == kModeOut) {
          // O^T lane (m, g) of tile (ct, tt): columns 16 ct + 4 g .. + 3 of token 16 tt + m
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int r = 16 * tt + m;
            if (r < nrow) {
              __bf16* orow = reinterpret_cast<__bf16*>(a.out) +
                             ((t0 + r) * a.HV + hv) * (int64_t)a.DV + col0 + 4 * g;
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) {
                bf16x4 ov;
                ov[0] = (__bf16)o[tt][ct][0];
                ov[1] = (__bf16)o[tt][ct][1];
                ov[2] = (__bf16)o[tt][ct][2];
                ov[3] = (__bf16)o[tt][ct][3];
                *reinterpret_cast<bf16x4*>(orow + 16 * ct) = ov;
              }
            }
          }
        }
        // S^T <- e^{G_n} S^T (+ K~^T U in the UP steps); e^{G_n} is e^G of the chunk's
        // last row (padding rows do not decay)
        const float egn = s.eg[C - 1];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) S[dt][ct] *= egn;
      }
      const half8 f = ring[i % RING];
      if constexpr (i + RING < NF) ring[i % RING] = *frag(s, std::integral_constant<int, i + RING>{});
      if constexpr (i < P) {
        constexpr int ks = i / 4, tt = i % 4;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) nu[tt][ct] = mma_f16(f, s16[ks][ct], nu[tt][ct]);
      } else if constexpr (i < P + O1) {
        constexpr int j2 = i - P, ks = j2 / 4, tt = j2 % 4;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          o[tt][ct] = mma_f16(s16[ks][ct], f, (ks == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : o[tt][ct]);
      } else if constexpr (i < P + O1 + O2) {
        constexpr int j2 = i - P - O1, fa = j2 < 2 ? 2 * j2 : j2 + 2, tt = fa / 2, st = fa % 2;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[tt][ct] = mma_f16(u16[st][ct], f, o[tt][ct]);
      } else {
        constexpr int j2 = i - P - O1 - O2, ts = j2 / NDT, dt = j2 % NDT;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[dt][ct] = mma_f16(f, u16[ts][ct], S[dt][ct]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  if (!active) return;
  // ---- the state at the end of the segment
  float* dst = nullptr;
  if (role == kRoleOut) {
    bool finite = true;  // an fp16 intermediate out of range shows up here
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) finite = finite && __builtin_isfinite(S[dt][ct][i]);
    if (__ballot(!finite) != 0 && l == 0) *a.nonfinite = 1;
    if (j != nseg - 1) return;  // a later segment carries the request on
    dst = a.state_pool + ((slot * a.HV + hv) * (int64_t)a.DV + col0) * DK;
  } else {
    const int64_t base = (sg * a.HV + hv) * (int64_t)(a.DV + DK);
    dst = a.rp + (base + (role == kRoleR ? 0 : a.DV) + col0) * DK;
  }
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      *reinterpret_cast<f32x4*>(dst + (16 * ct + m) * DK + 16 * dt + 4 * g) = S[dt][ct];
}

// Combine: for every cut request and value head, in segment order from the slot's state,
// S_{g+1} = S_g P_g + R_g, each S_g stored as the start state of segment g. One workgroup
// per (request, value head, 16 state rows), four waves; the products run on fp32 matrix
// cores (v_mfma_f32_16x16x4f32, full fp32 products and sums). Wave w forms column tiles
// 2 w and 2 w + 1 of the 16 rows; every wave holds the rows of S_g as A fragments (lane
// (r, g) of k step ks: S_g[r][4 ks + g]) and takes P_g's B fragments (lane (m, g): P_g[4 ks
// + g][16 ct + m]) straight from memory, loading the next segment's while it uses the
// current ones. The new rows go through LDS from the accumulator layout to the A layout.
constexpr int kCombineRows = 16;
template <int DK>
__global__ __launch_bounds__(256) void combine_kernel(ChainArgs a) {
  constexpr int NKS = DK / 4;         // fp32 k steps
  constexpr int NCT = DK / 16 / 4;    // column tiles per wave (2 at dk = 128, 1 at 64)
  __shared__ float Ss[kCombineRows][DK + 4];
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, m = l & 15, g = l >> 4;
  const int rb = a.DV / kCombineRows;
  const int64_t x = blockIdx.x;
  const int r0 = (int)(x % rb) * kCombineRows;
  const int64_t p = x / rb;
  const int b = (int)(p / a.HV), hv = (int)(p % a.HV);
  if (b >= a.B) return;
  // the request's segment count and first segment (every wave forms the table)
  int ns = 0;
  if (l < a.B) {
    const int64_t L = a.cu[l + 1] - a.cu[l];
    const int64_t nch = path_chunks(L, C, a.short_len);
    ns = (int)((nch + a.lseg - 1) / a.lseg);
  }
  int incl = ns;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (l >= off) incl += y;
  }
  const int nseg = __shfl(ns, b, 64);
  const int seg0 = __shfl(incl, b, 64) - nseg;
  if (nseg < 2) return;
  const int64_t slot = a.cache_indices[b];
  auto opbase = [&](int jj) { return ((seg0 + jj) * (int64_t)a.HV + hv) * (int64_t)(a.DV + DK); };
  float pf[NCT][NKS];  // B fragments of this step's P
  auto load_p = [&](int jj) {
    const float* P = a.rp + (opbase(jj) + a.DV) * DK;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) pf[c][ks] = P[(4 * ks + g) * DK + 16 * (NCT * wv + c) + m];
  };
  const float* S0 = a.state_pool + ((slot * a.HV + hv) * (int64_t)a.DV + r0) * DK;
  for (int e = tid; e < kCombineRows * DK; e += 256) Ss[e / DK][e % DK] = S0[e];
  load_p(0);
  __syncthreads();
  for (int jj = 0;; ++jj) {
    float* St = a.sstart + (((seg0 + jj) * (int64_t)a.HV + hv) * a.DV + r0) * DK;
    for (int e = tid; e < kCombineRows * DK; e += 256) St[e] = Ss[e / DK][e % DK];
    if (jj == nseg - 1) break;
    float sa[NKS];  // A fragments: S_g[m][4 ks + g]
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sa[ks] = Ss[m][4 * ks + g];
    const float* R = a.rp + (opbase(jj) + r0) * DK;
    f32x4 acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int col = 16 * (NCT * wv + c) + m;
      acc[c] = f32x4{R[(4 * g) * DK + col], R[(4 * g + 1) * DK + col], R[(4 * g + 2) * DK + col],
                     R[(4 * g + 3) * DK + col]};
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int c = 0; c < NCT; ++c) acc[c] = mma_f32(sa[ks], pf[c][ks], acc[c]);
    if (jj + 2 < nseg) load_p(jj + 1);  // the last segment has no operator
    __syncthreads();  // every wave has read S_g from LDS
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ss[4 * g + i][16 * (NCT * wv + c) + m] = acc[c][i];
    __syncthreads();
  }
}

}  // namespace

ChainPlan chain_plan(const Shape& s) {
  ChainPlan p;
  // The column-slice state kernel gives each (request, value head) dv / 32 workgroups of
  // 32 state rows; where those alone fill the device it serves the call. Otherwise
  // requests are cut into segments whose whole-block workgroups fill it.
  const int64_t slices = s.B * s.HV * (s.dv / 32);
  p.use = s.bf16 && s.dk <= 128 && s.C == C && s.B <= kMaxSelfPlanRequests && slices < 256;
  if (!p.use) return p;
  p.nb = (s.dv + kColsPerBlock - 1) / kColsPerBlock;
  p.nb_op = std::max(p.nb, (s.dk + kColsPerBlock - 1) / kColsPerBlock);
  const int64_t mc = s.N / s.C + s.B;  // upper bound on the call's chunks
  p.segmented = true;
  // segments of about the length that gives every compute unit one output workgroup
  const int64_t target = 256;
  int64_t lseg = (mc * s.HV * p.nb + target - 1) / target;
  lseg = std::max<int64_t>(lseg, 16);
  p.lseg = (int)std::min<int64_t>(lseg, 1 << 30);
  p.max_segs = mc / p.lseg + s.B;
  return p;
}

size_t chain_rp_bytes(const Shape& s, const ChainPlan& p) {
  if (!p.use || !p.segmented) return 0;
  return sizeof(float) * (size_t)p.max_segs * s.HV * (size_t)(s.dv + s.dk) * s.dk;
}
size_t chain_sstart_bytes(const Shape& s, const ChainPlan& p) {
  if (!p.use || !p.segmented) return 0;
  return sizeof(float) * (size_t)p.max_segs * s.HV * (size_t)s.dv * s.dk;
}

int64_t chain_grid(const Shape& s, const ChainPlan& p, int stage) {
  if (stage == 1) return (int64_t)s.B * s.HV * (s.dv / kCombineRows);
  const int64_t groups = p.max_segs * s.H;
  const int members = (s.HV / s.H) * (stage == 0 ? p.nb_op : p.nb);
  return (groups + 7) / 8 * 8 * members;
}

int chain_threads(int stage) {
  return stage == 0 ? kThreads<kModeOperator> : stage == 1 ? 256 : kThreads<kModeOut>;
}

hipError_t launch_chain(const ChainPlan& p, const Shape& s, const void* qf, const void* kf,
                        const int64_t* cu, const int64_t* cache_indices, const int32_t* chunk_off,
                        const void* w, const void* u, const void* aqk, const float* eg,
                        float* rp, float* sstart, float* state_pool, void* out,
                        int32_t* nonfinite, int stage, hipStream_t st) {
  ChainArgs a;
  a.W = (const _Float16*)w;
  a.U = (const _Float16*)u;
  a.Kf = (const _Float16*)kf;
  a.Qf = (const _Float16*)qf;
  a.Aqk = (const _Float16*)aqk;
  a.eg = eg;
  a.cu = cu;
  a.cache_indices = cache_indices;
  a.chunk_off = chunk_off;
  a.state_pool = state_pool;
  a.out = (uint16_t*)out;
  a.rp = rp;
  a.sstart = sstart;
  a.nonfinite = nonfinite;
  a.B = (int)s.B;
  a.H = s.H;
  a.HV = s.HV;
  a.DV = s.dv;
  a.short_len = s.short_len;
  a.lseg = p.lseg;
  a.segmented = p.segmented ? 1 : 0;
  a.nb = stage == 0 ? p.nb_op : p.nb;
  a.groups = p.max_segs * s.H;
  const int64_t grid = chain_grid(s, p, stage);
  if (grid <= 0) return hipSuccess;
  const dim3 gd((unsigned)grid), bd((unsigned)chain_threads(stage));
  if (stage == 0) {  // operator pass
    if (s.dk == 64)
      hipLaunchKernelGGL((chain_kernel<64, kModeOperator>), gd, bd, 0, st, a);
    else
      hipLaunchKernelGGL((chain_kernel<128, kModeOperator>), gd, bd, 0, st, a);
  } else if (stage == 1) {  // combine
    if (s.dk == 64)
      hipLaunchKernelGGL((combine_kernel<64>), gd, bd, 0, st, a);
    else
      hipLaunchKernelGGL((combine_kernel<128>), gd, bd, 0, st, a);
  } else {  // output pass
    if (s.dk == 64)
      hipLaunchKernelGGL((chain_kernel<64, kModeOut>), gd, bd, 0, st, a);
    else
      hipLaunchKernelGGL((chain_kernel<128, kModeOut>), gd, bd, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
