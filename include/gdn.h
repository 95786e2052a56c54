/*
 * libgdn -- Gated DeltaNet chunkwise prefill forward (with the decode step that follows
 * it, and the Promote update scan of the nested variant) on MI355X (gfx950).
 *
 * The operation (pymllm gdn_chunkwise page, "gdn_extend_chunkwise", Module
 * Contents; the recurrence is the state-transition equation of "Simple math to
 * speed up GDN prefill" (veitner), section Reminder):
 *
 *   for every request b (tokens cu_seqlens[b] .. cu_seqlens[b+1]-1) and value head hv,
 *   with q/k head h = hv / (HV / H) and slot s = cache_indices[b]:
 *     S <- state_pool[s, hv]                                   (dv x dk, fp32)
 *     for each token t:
 *       qh = q[t,h] / sqrt(|q[t,h]|^2 + 1e-6),  kh likewise     (q, k NOT pre-normalised)
 *       alpha = exp(-exp(A_log[hv]) * softplus(a[t,hv] + dt_bias[hv])),  beta = sigmoid(b[t,hv])
 *       S <- S * alpha * (I - beta kh kh^T) + beta v[t,hv] kh^T
 *       out[t,hv] = S qh                                       (the token sees its own write)
 *     state_pool[s, hv] <- S                                   (in place)
 *
 * It is evaluated chunkwise (chunks of C tokens restart at every request): one
 * triangular inverse M^-1 = (I + tril(B K K^T, -1))^-1 per chunk, reused for the
 * decayed inverse N^-1 = G M^-1 G^-1 (same page, section Save one invert), then a
 * sequential pass over chunks for the state and the outputs (pymllm page,
 * Algorithm). In batches of short requests on average, requests of at most
 * GDN_SHORT_REQUEST tokens are evaluated token by token instead, in the same call, unless
 * the descriptor's flags say GDN_FLAG_CHUNK_ALL.
 *
 * Layouts: every tensor is dense, contiguous, row-major.
 *   q, k        [N, H, dk]     fp32 or bf16 (qkv_dtype)
 *   v, out      [N, HV, dv]    same dtype as q (out has v's dtype)
 *   a, b        [N, HV]        fp32  (raw gate inputs, before softplus / sigmoid)
 *   A_log       [HV]           fp32
 *   dt_bias     [HV]           fp32
 *   state_pool  [pool, HV, dv, dk] fp32, read and written in place
 *   cache_indices [B]          int64, distinct slots in [0, pool)
 *   cu_seqlens  [B + 1]        int64, cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = N
 * All of these are DEVICE pointers. The problem descriptor is a HOST pointer.
 *
 * Ownership: the caller allocates and owns every buffer, the workspace included
 * (size from gdn_prefill_workspace_size). The library allocates nothing, keeps no
 * pointer after returning, and holds no state: calls are re-entrant (the one exception is
 * gdn_prefill_fwd_noalloc, whose built-in workspace every call on a GPU shares). A call is
 * asynchronous on `stream` (a hipStream_t; NULL = the default stream); buffers
 * must stay valid until the stream reaches the call. `out` must not alias an input.
 * Calls that share a state_pool slot or a workspace must be ordered on one stream.
 *
 * Errors: every argument check on the host happens before any launch, so a call
 * that returns an error status has written nothing. Contents of device arrays
 * (cu_seqlens, cache_indices) are a precondition; gdn_validate_inputs checks them
 * (it copies them to the host and synchronises, so it is for debugging).
 * GDN_ERR_HIP means a launch failed; state_pool may then be partly updated.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null pointer, negative size, HV % H != 0, bad dtype */
  GDN_ERR_UNSUPPORTED = 2, /* a valid but unsupported shape (head dims, chunk size) */
  GDN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  GDN_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  GDN_ERR_BAD_INPUT = 5    /* gdn_validate_inputs found bad cu_seqlens / cache_indices */
} gdn_status_t;

typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype_t;

/* Shape of one call (host struct). */
typedef struct {
  int64_t total_tokens; /* N: rows of q, k, v, a, b, out; equals cu_seqlens[B]          */
  int64_t batch;        /* B: requests; cu_seqlens has B + 1 entries, cache_indices B  */
  int32_t num_qk_heads; /* H                                                          */
  int32_t num_v_heads;  /* HV, a multiple of H; value head hv uses q/k head hv/(HV/H) */
  int32_t head_k;       /* dk, one of 64, 128, 256                                    */
  int32_t head_v;       /* dv, one of 64, 128, 256                                    */
  int64_t pool_size;    /* slots in state_pool                                        */
  int32_t qkv_dtype;    /* gdn_dtype_t of q, k, v and out                             */
  int32_t flags;        /* GDN_FLAG_* bits (0 by default); gdn_prefill_fwd reads them  */
} gdn_problem_t;

/* gdn_problem_t.flags. GDN_FLAG_CHUNK_ALL: gdn_prefill_fwd evaluates every request in
 * chunks. By default, in a batch whose mean request length N / B is at most
 * GDN_SPLIT_MEAN_LENGTH tokens, requests of at most GDN_SHORT_REQUEST tokens are evaluated
 * by the token recurrence instead (the kernel of gdn_recurrent_fwd, in the same call and
 * on the same stream), which is faster for them: a request that short still costs the
 * chunked path a whole chunk of intermediates per value head. Any other bit is an error. */
#define GDN_FLAG_CHUNK_ALL 1
#define GDN_SHORT_REQUEST 10
#define GDN_SPLIT_MEAN_LENGTH 64

/* Bytes of device workspace gdn_prefill_fwd needs for this problem and chunk size,
 * or 0 if the problem or chunk size is invalid. Host only, no HIP calls. */
size_t gdn_prefill_workspace_size(const gdn_problem_t* prob, int32_t chunk_size);

/* The prefill forward (see the top of this file). chunk_size: 64, or 128 for bf16 inputs
 * with dk of 128 or 256 (the pymllm page's Torch function defaults to 128, its kernel entry
 * point to 64, Module Contents); any other value, or 128 with fp32 inputs or dk = 64,
 * returns GDN_ERR_UNSUPPORTED. The result does not depend on it beyond rounding; 64 is the
 * faster schedule on every measured shape (128 doubles the per-token work of the chunk
 * preparation and leaves the state pass's time per token unchanged), and the segment scan
 * of long requests runs at 64 only.
 * workspace: device memory of at least gdn_prefill_workspace_size bytes, 256-byte
 * aligned; its contents on entry do not matter. stream: a hipStream_t or NULL.
 * When N <= GDN_SPLIT_MEAN_LENGTH * B, requests of 1 .. GDN_SHORT_REQUEST tokens run
 * through the token recurrence (the kernel of gdn_recurrent_fwd, fp32) and longer ones
 * through the chunked kernels, unless prob->flags has GDN_FLAG_CHUNK_ALL or q, k, v, out
 * or state_pool is not 16-byte aligned; otherwise every request is chunked (the bf16
 * path requires that alignment anyway).
 *
 * Magnitude range of bf16 inputs. The state and every output are accumulated in fp32,
 * but the bf16 path rounds its per-chunk intermediates to fp16 for the matrix cores:
 * the decayed keys and queries, A_qk and W<- (all bounded by 1 in magnitude, whatever
 * the inputs), and U~, U and the state's operand copy, which scale with |v| and |state|.
 * fp16 holds magnitudes up to 65504 with 11 significant bits from 2^-14 (about 6.1e-5)
 * up; below that its spacing is a fixed 2^-24. So:
 *   - entries of v and of the initial states up to about 2^12 (4096) in magnitude keep
 *     every fp16 intermediate finite on inputs like the benchmarked workloads (U~ and the
 *     state can grow to several times |v|); beyond that an intermediate may overflow,
 *     the affected outputs and states become inf or NaN, and the call raises the flag
 *     that gdn_prefill_nonfinite reads;
 *   - at magnitudes down to about 2^-10 (1e-3) the results keep the bf16 accuracy
 *     (outputs within 2e-2 rms plus their own bf16 rounding, states within 1e-3 relative
 *     of the fp64 recurrence); smaller values lose relative precision in fp16's
 *     subnormal range, silently;
 *   - the read-out of a state takes fp16 copies of the state and of q, so an output also
 *     carries an absolute error of a few 1e-4 (at most about 1e-3) of the initial
 *     states' entry scale. That is within 2e-2 rms(o) while the outputs are not much
 *     smaller than the states (as on the benchmarked workloads). Where the initial states
 *     are about 50 times the outputs' rms or more (unit-scale states, small beta, strong
 *     decay), a request's first outputs can exceed that part of the bar by up to this
 *     error; the states keep their bar.
 * Inputs outside that range belong on the fp32 path (GDN_DTYPE_F32), which holds the
 * state, every intermediate and the output in fp32. */
gdn_status_t gdn_prefill_fwd(const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* A_log, const float* dt_bias,
                             float* state_pool, const int64_t* cache_indices,
                             const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                             const gdn_problem_t* prob, void* workspace, size_t workspace_bytes,
                             void* stream);

/* gdn_prefill_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same operation,
 * arguments, layouts and errors, without the workspace arguments. Its workspace is a
 * built-in array of GDN_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, created
 * when the library is loaded on that GPU and held until the process ends; the first call
 * on a device looks up that device's copy (hipGetSymbolAddress), and no call allocates or
 * frees memory. A problem whose workspace (gdn_prefill_workspace_size) exceeds
 * GDN_NOALLOC_SCRATCH_BYTES is refused with GDN_ERR_WORKSPACE before anything runs. Every
 * call on one GPU uses that GPU's one array, whose contents on entry do not matter: calls
 * that may overlap on one GPU (different streams, or concurrent host threads without
 * ordering) race on it and must be serialised by the caller. */
#define GDN_NOALLOC_SCRATCH_BYTES (64ull << 20)
gdn_status_t gdn_prefill_fwd_noalloc(const void* q, const void* k, const void* v, const float* a,
                                     const float* b, const float* A_log, const float* dt_bias,
                                     float* state_pool, const int64_t* cache_indices,
                                     const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                                     const gdn_problem_t* prob, void* stream);

/* Stages of one call, in launch order, for gdn_prefill_fwd_events. */
#define GDN_NUM_STAGES 5 /* 0: chunk table (and, for fp32 inputs, the gates and log
                            cumulative decay; for bf16 inputs of at most 64 requests at
                            C = 64 the chunk prep forms the table and this stage launches
                            nothing);
                            1: chunk prep (for bf16 inputs including the gates; Grams, the
                            one inverse, W<- and U~); 2: operator pass of the segment scan
                            (requests cut into segments: each segment's state from zero and
                            its transition operator); 3: combine (every segment's start
                            state); 4: state pass + outputs. Stages 2 and 3 launch nothing
                            when no request is cut. */

/* Whether the last gdn_prefill_fwd call that ran with `workspace` (and launched kernels:
 * N > 0 and B > 0) left a non-finite value in any final state it wrote: the sign of an
 * intermediate outside its range (see the magnitude range above). Each such call clears
 * the flag before its state pass and raises it if a final state is not finite; the flag
 * is the workspace's first 4 bytes. Copies it to *nonfinite (1 raised, 0 clear) after
 * synchronising `stream`, so call it after the prefill on the same stream. Debugging and
 * tests; GDN_OK, or GDN_ERR_INVALID_ARG / GDN_ERR_WORKSPACE / GDN_ERR_HIP. */
gdn_status_t gdn_prefill_nonfinite(const void* workspace, size_t workspace_bytes,
                                   int32_t* nonfinite, void* stream);

/* Which kernels run the sequential state pass (stages 2-4 below) of a prefill call of this
 * shape; a function of the descriptor only. Host only, no HIP calls. Returns -1 for an
 * invalid or unsupported descriptor or chunk size. For profiling and tests.
 *   GDN_SCHEDULE_COLUMN_SLICES  bf16 inputs: one workgroup per (request, value head, 16, 32
 *                               or 64 state rows: the widest that still fills the device),
 *                               each walking its request's chunks; used when the 32-row
 *                               workgroups alone fill the device, when dk = 256, above
 *                               64 requests and at chunk size 128.
 *   GDN_SCHEDULE_SEGMENTS       bf16 inputs: requests cut into segments of chunks (operator
 *                               pass, combine, output pass) with one workgroup per
 *                               (segment, value head, 128 state rows).
 *   GDN_SCHEDULE_FP32           fp32 inputs: fp32 arithmetic throughout. */
#define GDN_SCHEDULE_COLUMN_SLICES 0
#define GDN_SCHEDULE_SEGMENTS 1
#define GDN_SCHEDULE_FP32 2
int32_t gdn_prefill_state_schedule(const gdn_problem_t* prob, int32_t chunk_size);

/* gdn_prefill_fwd with timing marks: stage_events points to GDN_NUM_STAGES + 1
 * hipEvent_t handles created by the caller on the current device; event i is recorded
 * on `stream` just before stage i is launched, the last one after the last stage.
 * Arguments, results and errors are those of gdn_prefill_fwd; no event is recorded if
 * the call fails its host checks. For profiling. */
gdn_status_t gdn_prefill_fwd_events(const void* q, const void* k, const void* v, const float* a,
                                    const float* b, const float* A_log, const float* dt_bias,
                                    float* state_pool, const int64_t* cache_indices,
                                    const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                                    const gdn_problem_t* prob, void* workspace,
                                    size_t workspace_bytes, void* stream,
                                    void* const* stage_events);

/* Backward of the prefill forward: gradients of every input of a gdn_prefill_fwd call,
 * given the gradients of its outputs and of each request's final state. For the scalar
 *   L = sum_{t,hv} <dout[t,hv], out[t,hv]> + sum_{b,hv} <dstate[b,hv], S_b,hv(final)>
 * it writes dq, dk [N, H, dk], dv [N, HV, dv], da, db [N, HV], dA_log, ddt_bias [HV]
 * and dstate0 [B, HV, dv, dk] (the gradient of each request's initial state, in request
 * order), all fp32, DEVICE pointers, fully overwritten. The recurrence at the top of this
 * file is differentiated token by token (its chunked evaluation is the same map, pymllm
 * gdn_chunkwise page, Algorithm; awehrs.io "NRM training kernels", Results: the backward
 * is expensive because of the sequential structure): a forward sweep keeps each state
 * every 8 tokens, the reverse sweep recomputes from those and walks back.
 * Inputs: q, k, v, a, b, A_log, dt_bias, cache_indices, cu_seqlens and prob as for
 * gdn_prefill_fwd (q, k, v and dout in qkv_dtype); state_pool holds the INITIAL states
 * (the pool as it was before the forward call, which updates it in place; read only);
 * dout [N, HV, dv] in qkv_dtype; dstate [B, HV, dv, dk] fp32 in request order.
 * chunk_size must be 64. workspace: at least gdn_prefill_bwd_workspace_size bytes,
 * 256-byte aligned (checkpoints, about N/8 x HV x dv x dk x 4 bytes, and per-token sums
 * over blocks of 32 state rows, about N x HV x dv x (2 dk + 2) / 8 bytes).
 * Arithmetic in fp32 throughout (no matrix cores); deterministic. N == 0 writes
 * dstate0 = dstate and zero dA_log, ddt_bias; B == 0 is a no-op. Errors as for
 * gdn_prefill_fwd: host checks before any launch. */
size_t gdn_prefill_bwd_workspace_size(const gdn_problem_t* prob, int32_t chunk_size);
gdn_status_t gdn_prefill_bwd(const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* A_log, const float* dt_bias,
                             const float* state_pool, const int64_t* cache_indices,
                             const int64_t* cu_seqlens, int32_t chunk_size, const void* dout,
                             const float* dstate, float* dq, float* dk, float* dv, float* da,
                             float* db, float* dA_log, float* ddt_bias, float* dstate0,
                             const gdn_problem_t* prob, void* workspace, size_t workspace_bytes,
                             void* stream);

/* One decode step: every request b brings exactly one new token, row b of q, k, v, a, b,
 * and the token's step of the recurrence at the top of this file is applied to
 * S = state_pool[cache_indices[b], hv] in place, with out[b, hv] = S qh read after the
 * write (the step after a prefill in serving: pymllm gdn_chunkwise page, Module
 * Contents, where the pool and indices serve the later decoding; the step itself is the
 * state-transition equation of "Simple math to speed up GDN prefill", section Reminder).
 * It equals gdn_prefill_fwd with cu_seqlens = {0, 1, ..., B}, computed without chunks:
 *   u = beta (v - alpha S kh),  S <- alpha S + u kh^T,  out = alpha S_old qh + (kh . qh) u.
 * prob->total_tokens must equal prob->batch (GDN_ERR_INVALID_ARG otherwise); the other
 * fields, layouts, dtypes and head dims are those of gdn_prefill_fwd:
 *   q, k [B, H, dk]; v, out [B, HV, dv]; a, b [B, HV]; A_log, dt_bias [HV];
 *   state_pool [pool, HV, dv, dk] fp32; cache_indices [B] int64, distinct, in [0, pool).
 * All DEVICE pointers; q, k, v and state_pool 16-byte aligned. No workspace, no
 * allocation, asynchronous on `stream`; B == 0 is a no-op. Arithmetic in fp32. Errors as
 * for gdn_prefill_fwd: host checks before any launch. */
gdn_status_t gdn_decode_fwd(const void* q, const void* k, const void* v, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            float* state_pool, const int64_t* cache_indices, void* out,
                            const gdn_problem_t* prob, void* stream);

/* The same operation as gdn_prefill_fwd (same arguments, layouts, dtypes, head dims and
 * state-pool semantics), evaluated as the token recurrence itself (the state-transition
 * equation of "Simple math to speed up GDN prefill", section Reminder, applied to each
 * token of a request in order) rather than in chunks: each request's state
 * rows stay in registers from its first token to its last, so the state is read and
 * written once per call. No workspace and no chunk size. Meant for short requests
 * (speculative-decoding verification, a few tokens each), where 64-row chunks would be
 * mostly padding; correct for any length, but a request's tokens run one after another.
 * Arithmetic in fp32 (no matrix cores). q, k, v and state_pool 16-byte aligned; N == 0
 * or B == 0 is a no-op; errors as for gdn_prefill_fwd. cu_seqlens and cache_indices are
 * preconditions as for the prefill (gdn_validate_inputs checks them). Compared with the
 * chunked path the result differs only by rounding: the recurrence is applied in fp32
 * token by token instead of chunk by chunk (for bf16 inputs the chunked path also keeps
 * its per-chunk intermediates in fp16). */
gdn_status_t gdn_recurrent_fwd(const void* q, const void* k, const void* v, const float* a,
                               const float* b, const float* A_log, const float* dt_bias,
                               float* state_pool, const int64_t* cache_indices,
                               const int64_t* cu_seqlens, void* out, const gdn_problem_t* prob,
                               void* stream);

/* Shape of one Promote update scan (host struct). */
typedef struct {
  int64_t scans;    /* independent (batch, head) scans                                 */
  int32_t firings;  /* F: firings per scan                                             */
  int32_t pairs;    /* n: pairs per firing, a multiple of 16, at most head_k           */
  int32_t head_k;   /* dk: 64 or 128                                                   */
  int32_t head_v;   /* dv: 64, 128 or 256                                              */
  int32_t kv_dtype; /* gdn_dtype_t of K and V: GDN_DTYPE_BF16 (fp32 is unsupported)    */
  int32_t reserved; /* must be 0                                                       */
} gdn_promote_problem_t;

/* The update scan of one level of the nested model (awehrs.io "NRM training kernels",
 * section General implementation, the Promote algorithm; section Kernel, a scan over
 * firings). Each scan holds a memory M (dk x dv, fp32) updated in place; at firing f its
 * n pairs are written at once, all against the memory as it stood before the firing:
 *   M <- diag(exp(gamma_f)) M;  M <- M - K_f^T (beta_f o K_f) M;  M <- M + K_f^T (w_f o V_f)
 * (per-row decay, gated removal along the new keys, gated write; o scales the pairs' rows).
 * Layouts (dense, row-major, DEVICE pointers):
 *   K      [scans, F, n, dk]  bf16, unit rows (the probe's normalised write keys)
 *   V      [scans, F, n, dv]  bf16
 *   beta, w [scans, F, n]     fp32 erase and write gates
 *   gamma  [scans, F, dk]     fp32 log-decay, one entry per key row
 *   M      [scans, dk, dv]    fp32, in: the memory before the first firing; out: after the last
 *   states [scans, F, dk, dv] fp32 out: the memory after each firing; NULL to skip
 * K, V and states 16-byte aligned. Products on matrix cores with fp16 operands (the memory and
 * U = w o V - beta o K M rounded to fp16, keys converted exactly up to fp16 range) and fp32
 * accumulation; the memory itself stays fp32. No workspace, no allocation, asynchronous on
 * `stream`; scans == 0 is a no-op. Errors: host checks before any launch. */
gdn_status_t gdn_promote_scan(const void* K, const void* V, const float* beta, const float* w,
                              const float* gamma, float* M, float* states,
                              const gdn_promote_problem_t* prob, void* stream);

/* Debug check of the device-array preconditions: cu_seqlens[0] == 0, non-decreasing,
 * cu_seqlens[B] == N; cache_indices distinct and in [0, pool). Copies both arrays to
 * the host (16 bytes per request; at most 2^26 requests, GDN_ERR_UNSUPPORTED above that or
 * if the host copies cannot be allocated) and synchronises `stream`. GDN_OK or
 * GDN_ERR_BAD_INPUT. */
gdn_status_t gdn_validate_inputs(const int64_t* cu_seqlens, const int64_t* cache_indices,
                                 const gdn_problem_t* prob, void* stream);

/* Static text for a status code. */
const char* gdn_status_str(gdn_status_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
