// Internal declarations of libgdn: workspace layout and kernel launchers.
// Not part of the public C ABI (include/gdn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr float kNormEps = 1e-6f;  // added to |x|^2 inside the L2 norm of q and k

// Kernel family that serves a call.
enum class Path : int {
  kRef = 0,   // fp32 arithmetic everywhere (fp32 inputs, and any shape the MFMA path lacks)
  kMfma = 1,  // bf16 inputs: MFMA chunk and state kernels
};

// Byte offsets of each region inside the caller's workspace (all 256-byte aligned).
struct WsLayout {
  int64_t max_chunks = 0;  // upper bound on sum_b ceil(L_b / C) = N / C + B
  size_t flags = 0;        // int32 [1]: set when a call's final states are not all finite
  size_t chunk_off = 0;    // int32 [B + 1]: first global chunk of each request
  size_t chunk_seq = 0;    // int32 [max_chunks]: request of each global chunk, -1 if unused
  size_t gcum = 0;         // double [max_chunks][HV][C]: chunk-local inclusive sum of log(alpha)
                           //        (kRef only: the MFMA chunk prep forms its own gates)
  size_t beta = 0;         // float  [max_chunks][HV][C]: beta (0 on padding rows) (kRef only)
  size_t w = 0;            // W<- [max_chunks][HV][C][dk] (fp32 rows on kRef, fp16 fragments
                           //     on kMfma)
  size_t u = 0;            // U~  [max_chunks][HV]: fp32 [dv][C] (transposed) on kRef; fp16 MFMA
                           //     D tiles on kMfma
  size_t aqk = 0;          // A_qk [max_chunks][HV][C][C]: fp32 rows on kRef, fp16 fragments on
                           //      kMfma
  size_t eg = 0;           // float  [max_chunks][HV][C]: e^G per chunk row (kMfma only)
  size_t kf = 0;           // K~ = diag(e^{G_n - G} r_k) K [max_chunks][HV]: fp32 [dk][C]
                           //      (transposed) on kRef; fp16 [C][dk] fragments on kMfma
  size_t qf = 0;           // kRef: fp32 [max_chunks][HV][C][dk], diag(e^G r_q) Q;
                           // kMfma: fp16 [max_chunks][H][C][dk], normalised q in fragments
  size_t rp = 0;           // float  [segments][HV][dv + dk][dk]: each cut segment's state from
                           //        zero (R) and its operator product (P) (segment scan only)
  size_t sstart = 0;       // float  [segments][HV][dv][dk]: start state of every segment of a
                           //        cut request (segment scan only)
  size_t total = 0;
};

struct Shape {
  int64_t N, B;
  int H, HV, dk, dv, C;
  int64_t pool;
  bool bf16;
  int64_t short_len = 0;  // requests of at most this many tokens skip the chunked kernels
};

// Requests of at most this many tokens are evaluated by the token recurrence inside the
// prefill call, longer ones in chunks (a one-token request still costs the chunked path a
// whole 64-row chunk of intermediates per value head and state slice). Measured on bf16
// inputs, dk = dv = 128, 32 value heads, 512 requests of L tokens, per call: chunking
// every request takes 1.59 ms at L = 1, 1.61 ms at 12 and 16; with the recurrence for the
// short ones (whose call still launches the chunked kernels, which find nothing to do)
// 0.53 ms at 1, 1.36 ms at 12 and 1.68 ms at 16.
constexpr int64_t kShortRequest = 10;  // GDN_SHORT_REQUEST of the public header
// The recurrence's launch costs a few microseconds even when it finds no short request
// (5 us at 8 requests and 32 value heads), so a call splits only when the mean request
// length N / B is at most this; longer batches are chunked whole.
constexpr int64_t kSplitMeanLength = 64;  // GDN_SPLIT_MEAN_LENGTH of the public header

// Chunks of a request of L tokens on the chunked path: none if L <= short_len.
__host__ __device__ __forceinline__ int64_t path_chunks(int64_t L, int C, int64_t short_len) {
  return (L > short_len && L > 0) ? (L + C - 1) / C : 0;
}

Path choose_path(const Shape& s);
WsLayout layout_for(const Shape& s, Path p);

// Launchers (host). Each returns hipSuccess or the launch error.
hipError_t launch_plan(const int64_t* cu_seqlens, const Shape& s, int32_t* chunk_off,
                       int32_t* chunk_seq, int64_t max_chunks, hipStream_t st);
hipError_t launch_gate(const float* a, const float* b, const float* A_log, const float* dt_bias,
                       const int64_t* cu_seqlens, const int32_t* chunk_off,
                       const int32_t* chunk_seq, const Shape& s, int64_t max_chunks,
                       double* gcum, float* beta, int32_t* nonfinite, hipStream_t st);
hipError_t launch_ref_prep(const void* q, const void* k, const void* v,
                           const int64_t* cu_seqlens, const int32_t* chunk_off,
                           const int32_t* chunk_seq, const double* gcum, const float* beta,
                           const Shape& s, int64_t max_chunks, float* w, float* ut, float* aqk,
                           float* kft, float* qf, hipStream_t st);
hipError_t launch_ref_state(const int64_t* cu_seqlens, const int64_t* cache_indices,
                            const int32_t* chunk_off, const double* gcum, const float* w,
                            const float* ut, const float* aqk, const float* kft, const float* qf,
                            const Shape& s, float* state_pool, void* out, int32_t* nonfinite,
                            hipStream_t st);

// The chunk prep and the state pass at s.C = 64 or 128 (128: dk of 128 or 256).
// self_plan (C = 64, at most kMaxSelfPlanRequests requests): the prep kernel forms the
// chunk table itself and writes chunk_off (B + 1 entries) for the state pass; chunk_seq is
// then not read and the plan kernel need not run.
constexpr int kMaxSelfPlanRequests = 64;
hipError_t launch_mfma_prep(const void* q, const void* k, const void* v,
                            const int64_t* cu_seqlens, int32_t* chunk_off,
                            const int32_t* chunk_seq, bool self_plan, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            const Shape& s, int64_t max_chunks, void* w, void* u, void* aqk,
                            float* eg, void* kf, void* qf, int32_t* nonfinite, hipStream_t st);
hipError_t launch_mfma_state(const void* qf, const void* kf, const int64_t* cu_seqlens,
                             const int64_t* cache_indices, const int32_t* chunk_off,
                             const void* w, const void* u, const void* aqk,
                             const float* eg, const Shape& s, float* state_pool, void* out,
                             int32_t* nonfinite, hipStream_t st);

// The state pass with whole 128-column state blocks per workgroup and the segment scan of
// long requests (bf16 inputs, dk <= 128).
struct ChainPlan {
  bool use = false;        // this pass serves the call (else the column-slice state kernel)
  bool segmented = false;  // requests may be cut into segments (at most 64 requests)
  int lseg = 1 << 30;      // chunks per segment
  int nb = 1;              // output-pass workgroups per (segment, value head)
  int nb_op = 1;           // operator-pass workgroups per (segment, value head)
  int64_t max_segs = 0;    // upper bound on the call's segments
};
ChainPlan chain_plan(const Shape& s);
size_t chain_rp_bytes(const Shape& s, const ChainPlan& p);
size_t chain_sstart_bytes(const Shape& s, const ChainPlan& p);
// Workgroups and threads per workgroup of a stage's launch: 0 operator pass, 1 combine,
// 2 output pass.
int64_t chain_grid(const Shape& s, const ChainPlan& p, int stage);
int chain_threads(int stage);
hipError_t launch_chain(const ChainPlan& p, const Shape& s, const void* qf, const void* kf,
                        const int64_t* cu, const int64_t* cache_indices, const int32_t* chunk_off,
                        const void* w, const void* u, const void* aqk, const float* eg,
                        float* rp, float* sstart, float* state_pool, void* out,
                        int32_t* nonfinite, int stage, hipStream_t st);

// Decode step (one token per request): workgroups a launch needs, and the launcher.
int64_t decode_blocks(const Shape& s);
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* A_log, const float* dt_bias,
                         const int64_t* cache_indices, const Shape& s, float* state_pool,
                         void* out, hipStream_t st);

// The token recurrence without chunks, for short requests (same grid as the decode step).
hipError_t launch_recurrent(const void* q, const void* k, const void* v, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            const int64_t* cache_indices, const int64_t* cu_seqlens,
                            const Shape& s, int64_t max_len, float* state_pool, void* out,
                            hipStream_t st);  // requests longer than max_len are skipped

// Promote update scan: shape and launcher (bf16 keys and values).
struct PromoteShape {
  int64_t BH;  // independent scans
  int F, n, dk, dv;
};
hipError_t launch_promote(const PromoteShape& s, const void* K, const void* V, const float* beta,
                          const float* w, const float* gamma, float* M, float* states,
                          hipStream_t st);

}  // namespace gdn
