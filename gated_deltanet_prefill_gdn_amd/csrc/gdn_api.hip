// C ABI of libgdn (declared in include/gdn.h): host-side argument checks, the
// workspace layout and the launch sequence plan -> gate -> chunk prep -> state pass of
// the prefill, the chunk-free recurrent path, the decode step and the Promote update scan.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"
#include "gdn_backward.h"

static_assert(gdn::kShortRequest == GDN_SHORT_REQUEST, "one threshold");
static_assert(gdn::kSplitMeanLength == GDN_SPLIT_MEAN_LENGTH, "one threshold");

namespace gdn {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

Path choose_path(const Shape& s) { return s.bf16 ? Path::kMfma : Path::kRef; }

WsLayout layout_for(const Shape& s, Path p) {
  WsLayout L;
  L.max_chunks = s.N / s.C + s.B;
  const size_t mc = (size_t)L.max_chunks;
  const size_t el = (p == Path::kRef) ? 4 : 2;
  size_t off = 0;
  L.flags = off;
  off = align256(off + sizeof(int32_t));
  L.chunk_off = off;
  off = align256(off + sizeof(int32_t) * (size_t)(s.B + 1));
  L.chunk_seq = off;
  off = align256(off + sizeof(int32_t) * mc);
  L.gcum = off;  // the MFMA chunk prep computes its gates itself
  if (p == Path::kRef) off = align256(off + sizeof(double) * mc * s.HV * s.C);
  L.beta = off;
  if (p == Path::kRef) off = align256(off + sizeof(float) * mc * s.HV * s.C);
  L.w = off;
  off = align256(off + el * mc * s.HV * s.C * s.dk);
  L.u = off;
  off = align256(off + el * mc * s.HV * s.C * s.dv);
  L.aqk = off;
  off = align256(off + el * mc * s.HV * s.C * s.C);
  L.eg = off;
  if (p == Path::kMfma) off = align256(off + sizeof(float) * mc * s.HV * s.C);
  L.kf = off;
  off = align256(off + el * mc * s.HV * s.C * s.dk);
  L.qf = off;  // per q/k head on the MFMA path, per value head (it carries e^G) on kRef
  off = align256(off + el * mc * (p == Path::kMfma ? s.H : s.HV) * s.C * s.dk);
  const ChainPlan cp = p == Path::kMfma ? chain_plan(s) : ChainPlan{};
  L.rp = off;
  off = align256(off + chain_rp_bytes(s, cp));
  L.sstart = off;
  off = align256(off + chain_sstart_bytes(s, cp));
  L.total = off;
  return L;
}

// Requests gdn_validate_inputs copies to the host at most (16 bytes each).
constexpr int64_t kMaxValidateRequests = (int64_t)1 << 26;

// A launch of `blocks` workgroups of `threads` work-items along x: the dispatch packet
// holds the grid size in work-items as 32 bits.
static bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 0 && blocks * (int64_t)threads <= (int64_t)0xFFFFFFFF;
}

// Every launch of a prefill call of shape s fits its grid limits.
static bool prefill_grids_fit(const Shape& s, Path path, int64_t max_chunks) {
  if (path == Path::kRef) {
    // gate: 4 (chunk, value head) pairs per 256-thread workgroup; ref prep: (chunk, value
    // head) grid; ref state: (request, value head) pairs rounded up to 8, times dv / 16
    return grid_fits((max_chunks * s.HV + 3) / 4, 256) && grid_fits(max_chunks, 256) &&
           s.HV <= 65535 && grid_fits((s.B * s.HV + 7) / 8 * 8 * (s.dv / 16), 256);
  }
  if (s.C == 128) {
    // prep: one 512-thread workgroup per (chunk, value head); state: eight waves per
    // (request, value head) pair rounded up to 8 and column block (at most dv / 16)
    return grid_fits(max_chunks * s.HV, 512) &&
           grid_fits((s.B * s.HV + 7) / 8 * 8 * (s.dv / 16), 512);
  }
  const ChainPlan cp = chain_plan(s);
  if (cp.use) {
    for (int stage = 0; stage < 3; ++stage)
      if (!grid_fits(chain_grid(s, cp, stage), chain_threads(stage))) return false;
    return true;
  }
  // column-slice state kernel: (request, value head) pairs rounded up to 8, times dv / 32
  // slices (dv / 16 where those would not fill the device, dv / 64 where those would),
  // workgroups of five waves; the bound below takes the most slices the rule can pick (the
  // prep kernel's grid is the device's resident capacity)
  const int64_t slices = s.B * s.HV * (s.dv / 32) < 256 ? s.dv / 16 : s.dv / 32;
  return grid_fits((s.B * s.HV + 7) / 8 * 8 * slices, 64 * 5);
}

// Descriptor checks shared by every entry point. Host only.
static gdn_status_t check_problem(const gdn_problem_t* p, int32_t chunk_size, Shape* s) {
  if (!p) return GDN_ERR_INVALID_ARG;
  if (p->total_tokens < 0 || p->batch < 0 || p->pool_size < 0) return GDN_ERR_INVALID_ARG;
  if (p->num_qk_heads <= 0 || p->num_v_heads <= 0) return GDN_ERR_INVALID_ARG;
  if (p->num_v_heads % p->num_qk_heads != 0) return GDN_ERR_INVALID_ARG;
  if (p->head_k <= 0 || p->head_v <= 0) return GDN_ERR_INVALID_ARG;
  if (p->qkv_dtype != GDN_DTYPE_F32 && p->qkv_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID_ARG;
  if ((p->flags & ~GDN_FLAG_CHUNK_ALL) != 0) return GDN_ERR_INVALID_ARG;
  if (chunk_size <= 0) return GDN_ERR_INVALID_ARG;
  if (p->batch > 0 && p->pool_size < 1) return GDN_ERR_INVALID_ARG;
  s->N = p->total_tokens;
  s->B = p->batch;
  s->H = p->num_qk_heads;
  s->HV = p->num_v_heads;
  s->dk = p->head_k;
  s->dv = p->head_v;
  s->C = chunk_size;
  s->pool = p->pool_size;
  s->bf16 = p->qkv_dtype == GDN_DTYPE_BF16;
  if (!head_dim_ok(p->head_k) || !head_dim_ok(p->head_v)) return GDN_ERR_UNSUPPORTED;
  // C = 64 on every path; C = 128 on the bf16 matrix-core path with dk of 128 or 256
  if (chunk_size != 64 && chunk_size != 128) return GDN_ERR_UNSUPPORTED;
  if (chunk_size == 128 && !(s->bf16 && s->dk >= 128)) return GDN_ERR_UNSUPPORTED;
  if (p->num_v_heads > 65535) return GDN_ERR_UNSUPPORTED;
  if (p->total_tokens > ((int64_t)1 << 31) - 1 - 64 * (p->batch + 1)) return GDN_ERR_UNSUPPORTED;
  if (p->batch > ((int64_t)1 << 30)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

int32_t gdn_version(void) { return 400; }

const char* gdn_status_str(gdn_status_t st) {
  switch (st) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape or chunk size";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime or launch failure";
    case GDN_ERR_BAD_INPUT: return "cu_seqlens or cache_indices violate their preconditions";
  }
  return "unknown status";
}

size_t gdn_prefill_workspace_size(const gdn_problem_t* prob, int32_t chunk_size) {
  Shape s;
  if (check_problem(prob, chunk_size, &s) != GDN_OK) return 0;
  return layout_for(s, choose_path(s)).total;
}

int32_t gdn_prefill_state_schedule(const gdn_problem_t* prob, int32_t chunk_size) {
  Shape s;
  if (check_problem(prob, chunk_size, &s) != GDN_OK) return -1;
  if (choose_path(s) == Path::kRef) return GDN_SCHEDULE_FP32;
  return chain_plan(s).use ? GDN_SCHEDULE_SEGMENTS : GDN_SCHEDULE_COLUMN_SLICES;
}

}  // extern "C"

namespace {

gdn_status_t run_prefill(const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* A_log, const float* dt_bias,
                         float* state_pool, const int64_t* cache_indices,
                         const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                         const gdn_problem_t* prob, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* events) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, chunk_size, &s);
  if (ps != GDN_OK) return ps;
  if (s.N == 0 || s.B == 0) return GDN_OK;  // no token: nothing is read or written
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state_pool || !cache_indices ||
      !cu_seqlens || !out)
    return GDN_ERR_INVALID_ARG;
  const Path path = choose_path(s);
  const WsLayout L = layout_for(s, path);
  if (!prefill_grids_fit(s, path, L.max_chunks)) return GDN_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return GDN_ERR_WORKSPACE;
  bool aligned = true;  // 16-byte vector loads and stores
  for (const void* ptr : {q, k, v, (const void*)out, (const void*)state_pool})
    aligned = aligned && ((uintptr_t)ptr & 15) == 0;
  if (path == Path::kMfma && !aligned) return GDN_ERR_INVALID_ARG;
  // Short requests go to the token recurrence (its 16-byte loads need the alignment; the
  // fp32 chunked kernels do not, and take every request otherwise).
  const bool split = (prob->flags & GDN_FLAG_CHUNK_ALL) == 0 && s.N <= kSplitMeanLength * s.B;
  s.short_len = (split && aligned && decode_blocks(s) <= 0x7FFFFFFF) ? kShortRequest : 0;
  if (events) {
    for (int i = 0; i <= GDN_NUM_STAGES; ++i)
      if (!events[i]) return GDN_ERR_INVALID_ARG;
  }
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord((hipEvent_t)events[i], st) == hipSuccess;
  };
  // the requests of at most s.short_len tokens, in the state stage
  auto short_pass = [&]() -> bool {
    return s.short_len == 0 ||
           launch_recurrent(q, k, v, a, b, A_log, dt_bias, cache_indices, cu_seqlens, s,
                            s.short_len, state_pool, out, st) == hipSuccess;
  };
  char* ws = (char*)workspace;
  int32_t* chunk_off = (int32_t*)(ws + L.chunk_off);
  int32_t* chunk_seq = (int32_t*)(ws + L.chunk_seq);
  double* gcum = (double*)(ws + L.gcum);
  float* beta = (float*)(ws + L.beta);
  int32_t* nonfinite = (int32_t*)(ws + L.flags);

  // Up to 64 requests the MFMA chunk prep at C = 64 forms the chunk table itself (one scan
  // per workgroup) and writes chunk_off for the state pass: one launch fewer. The C = 128
  // prep reads the plan kernel's table.
  const bool self_plan = path == Path::kMfma && s.B <= kMaxSelfPlanRequests && s.C == 64;
  if (!mark(0)) return GDN_ERR_HIP;
  if (!self_plan &&
      launch_plan(cu_seqlens, s, chunk_off, chunk_seq, L.max_chunks, st) != hipSuccess)
    return GDN_ERR_HIP;
  if (path == Path::kRef &&
      launch_gate(a, b, A_log, dt_bias, cu_seqlens, chunk_off, chunk_seq, s, L.max_chunks, gcum,
                  beta, nonfinite, st) != hipSuccess)
    return GDN_ERR_HIP;
  if (!mark(1)) return GDN_ERR_HIP;
  void* w = ws + L.w;
  void* u = ws + L.u;
  if (path == Path::kMfma) {
    void* aqk = ws + L.aqk;
    float* eg = (float*)(ws + L.eg);
    void* kf = ws + L.kf;
    void* qf = ws + L.qf;
    if (launch_mfma_prep(q, k, v, cu_seqlens, chunk_off, chunk_seq, self_plan, a, b, A_log,
                         dt_bias, s, L.max_chunks, w, u, aqk, eg, kf, qf, nonfinite,
                         st) != hipSuccess)
      return GDN_ERR_HIP;
    const ChainPlan cp = chain_plan(s);
    if (cp.use) {
      float* rp = (float*)(ws + L.rp);
      float* sstart = (float*)(ws + L.sstart);
      for (int stage = 0; stage < 3; ++stage) {
        if (!mark(2 + stage)) return GDN_ERR_HIP;
        if (stage == 2 && !short_pass()) return GDN_ERR_HIP;
        if ((stage < 2 && !cp.segmented)) continue;  // nothing is cut: one pass
        if (launch_chain(cp, s, qf, kf, cu_seqlens, cache_indices, chunk_off, w, u, aqk, eg, rp,
                         sstart, state_pool, out, nonfinite, stage, st) != hipSuccess)
          return GDN_ERR_HIP;
      }
    } else {
      if (!mark(2) || !mark(3) || !mark(4) || !short_pass()) return GDN_ERR_HIP;
      if (launch_mfma_state(qf, kf, cu_seqlens, cache_indices, chunk_off, w, u, aqk, eg, s,
                            state_pool, out, nonfinite, st) != hipSuccess)
        return GDN_ERR_HIP;
    }
  } else {
    float* aqk = (float*)(ws + L.aqk);
    float* kf = (float*)(ws + L.kf);
    float* qf = (float*)(ws + L.qf);
    if (launch_ref_prep(q, k, v, cu_seqlens, chunk_off, chunk_seq, gcum, beta, s, L.max_chunks,
                        (float*)w, (float*)u, aqk, kf, qf, st) != hipSuccess)
      return GDN_ERR_HIP;
    if (!mark(2) || !mark(3) || !mark(4) || !short_pass()) return GDN_ERR_HIP;
    if (launch_ref_state(cu_seqlens, cache_indices, chunk_off, gcum, (const float*)w,
                         (const float*)u, aqk, kf, qf, s, state_pool, out, nonfinite,
                         st) != hipSuccess)
      return GDN_ERR_HIP;
  }
  if (!mark(5)) return GDN_ERR_HIP;
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status_t gdn_prefill_fwd(const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* A_log, const float* dt_bias,
                             float* state_pool, const int64_t* cache_indices,
                             const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                             const gdn_problem_t* prob, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return run_prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                     chunk_size, out, prob, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// Built-in workspace of gdn_prefill_fwd_noalloc: one array per GPU the library runs on,
// held until the process ends. In host code `scratch` names a host-side stand-in only; the
// device address comes from hipGetSymbolAddress, once per device, and only that address is
// ever passed to a kernel.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's scratch address (resolved on the first call on that device), or
// nullptr on a HIP error.
void* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

gdn_status_t gdn_prefill_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const float* a, const float* b, const float* A_log,
                                     const float* dt_bias, float* state_pool,
                                     const int64_t* cache_indices, const int64_t* cu_seqlens,
                                     int32_t chunk_size, void* out, const gdn_problem_t* prob,
                                     void* stream) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, chunk_size, &s);
  if (ps != GDN_OK) return ps;
  if (s.N == 0 || s.B == 0) return GDN_OK;
  // the call's workspace must fit the built-in array
  if (layout_for(s, choose_path(s)).total > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return GDN_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return GDN_ERR_HIP;
  return run_prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                     chunk_size, out, prob, ws, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream,
                     nullptr);
}

gdn_status_t gdn_prefill_fwd_events(const void* q, const void* k, const void* v, const float* a,
                                    const float* b, const float* A_log, const float* dt_bias,
                                    float* state_pool, const int64_t* cache_indices,
                                    const int64_t* cu_seqlens, int32_t chunk_size, void* out,
                                    const gdn_problem_t* prob, void* workspace,
                                    size_t workspace_bytes, void* stream,
                                    void* const* stage_events) {
  if (!stage_events) return GDN_ERR_INVALID_ARG;
  return run_prefill(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                     chunk_size, out, prob, workspace, workspace_bytes, stream, stage_events);
}

gdn_status_t gdn_decode_fwd(const void* q, const void* k, const void* v, const float* a,
                            const float* b, const float* A_log, const float* dt_bias,
                            float* state_pool, const int64_t* cache_indices, void* out,
                            const gdn_problem_t* prob, void* stream) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, 64, &s);  // the chunk size plays no part
  if (ps != GDN_OK) return ps;
  if (s.N != s.B) return GDN_ERR_INVALID_ARG;  // exactly one token per request
  if (s.B == 0) return GDN_OK;
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state_pool || !cache_indices || !out)
    return GDN_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)state_pool})  // 16-byte vector loads
    if (((uintptr_t)ptr & 15) != 0) return GDN_ERR_INVALID_ARG;
  if (decode_blocks(s) > 0x7FFFFFFF) return GDN_ERR_UNSUPPORTED;
  if (launch_decode(q, k, v, a, b, A_log, dt_bias, cache_indices, s, state_pool, out,
                    (hipStream_t)stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

gdn_status_t gdn_recurrent_fwd(const void* q, const void* k, const void* v, const float* a,
                               const float* b, const float* A_log, const float* dt_bias,
                               float* state_pool, const int64_t* cache_indices,
                               const int64_t* cu_seqlens, void* out, const gdn_problem_t* prob,
                               void* stream) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, 64, &s);  // the chunk size plays no part
  if (ps != GDN_OK) return ps;
  if (s.N == 0 || s.B == 0) return GDN_OK;
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state_pool || !cache_indices ||
      !cu_seqlens || !out)
    return GDN_ERR_INVALID_ARG;
  for (const void* ptr : {q, k, v, (const void*)state_pool})  // 16-byte vector loads
    if (((uintptr_t)ptr & 15) != 0) return GDN_ERR_INVALID_ARG;
  if (decode_blocks(s) > 0x7FFFFFFF) return GDN_ERR_UNSUPPORTED;
  if (launch_recurrent(q, k, v, a, b, A_log, dt_bias, cache_indices, cu_seqlens, s, INT64_MAX,
                       state_pool, out, (hipStream_t)stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

gdn_status_t gdn_promote_scan(const void* K, const void* V, const float* beta, const float* w,
                              const float* gamma, float* M, float* states,
                              const gdn_promote_problem_t* prob, void* stream) {
  if (!prob || prob->reserved != 0) return GDN_ERR_INVALID_ARG;
  if (prob->scans < 0 || prob->firings < 0 || prob->pairs <= 0 || prob->head_k <= 0 ||
      prob->head_v <= 0)
    return GDN_ERR_INVALID_ARG;
  if (prob->kv_dtype != GDN_DTYPE_F32 && prob->kv_dtype != GDN_DTYPE_BF16)
    return GDN_ERR_INVALID_ARG;
  if (prob->kv_dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
  if (prob->head_k != 64 && prob->head_k != 128) return GDN_ERR_UNSUPPORTED;
  if (prob->head_v % 64 != 0 || prob->head_v > 256) return GDN_ERR_UNSUPPORTED;
  if (prob->pairs % 16 != 0 || prob->pairs > prob->head_k) return GDN_ERR_UNSUPPORTED;
  if (prob->scans > ((int64_t)1 << 28)) return GDN_ERR_UNSUPPORTED;
  if (prob->scans == 0) return GDN_OK;
  if (!M) return GDN_ERR_INVALID_ARG;
  if (prob->firings > 0 && (!K || !V || !beta || !w || !gamma)) return GDN_ERR_INVALID_ARG;
  for (const void* ptr : {K, V, (const void*)states})  // 16-byte vector loads and stores
    if (((uintptr_t)ptr & 15) != 0) return GDN_ERR_INVALID_ARG;
  PromoteShape s{prob->scans, prob->firings, prob->pairs, prob->head_k, prob->head_v};
  if (launch_promote(s, K, V, beta, w, gamma, M, states, (hipStream_t)stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

size_t gdn_prefill_bwd_workspace_size(const gdn_problem_t* prob, int32_t chunk_size) {
  Shape s;
  if (check_problem(prob, chunk_size, &s) != GDN_OK || chunk_size != 64) return 0;
  return bwd_layout_for(s).total;
}

gdn_status_t gdn_prefill_bwd(const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* A_log, const float* dt_bias,
                             const float* state_pool, const int64_t* cache_indices,
                             const int64_t* cu_seqlens, int32_t chunk_size, const void* dout,
                             const float* dstate, float* dq, float* dk, float* dv, float* da,
                             float* db, float* dA_log, float* ddt_bias, float* dstate0,
                             const gdn_problem_t* prob, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, chunk_size, &s);
  if (ps != GDN_OK) return ps;
  if (chunk_size != 64) return GDN_ERR_UNSUPPORTED;  // the backward's schedule is fixed
  if (s.B == 0) return GDN_OK;
  if (!A_log || !dt_bias || !state_pool || !cache_indices || !cu_seqlens || !dstate ||
      !dA_log || !ddt_bias || !dstate0)
    return GDN_ERR_INVALID_ARG;
  if (s.N > 0 && (!q || !k || !v || !a || !b || !dout || !dq || !dk || !dv || !da || !db))
    return GDN_ERR_INVALID_ARG;
  if (!bwd_grids_fit(s)) return GDN_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout_for(s);
  if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255) != 0) return GDN_ERR_WORKSPACE;
  if (launch_backward(s, L, (char*)workspace, q, k, v, a, b, A_log, dt_bias, state_pool,
                      cache_indices, cu_seqlens, dout, dstate, dq, dk, dv, da, db, dA_log,
                      ddt_bias, dstate0, (hipStream_t)stream) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

gdn_status_t gdn_prefill_nonfinite(const void* workspace, size_t workspace_bytes,
                                   int32_t* nonfinite, void* stream) {
  if (!workspace || !nonfinite) return GDN_ERR_INVALID_ARG;
  if (workspace_bytes < sizeof(int32_t)) return GDN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess)
    return GDN_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return GDN_ERR_HIP;
  *nonfinite = v != 0;
  return GDN_OK;
}

gdn_status_t gdn_validate_inputs(const int64_t* cu_seqlens, const int64_t* cache_indices,
                                 const gdn_problem_t* prob, void* stream) {
  Shape s;
  const gdn_status_t ps = check_problem(prob, 64, &s);
  if (ps != GDN_OK && ps != GDN_ERR_UNSUPPORTED) return ps;
  if (s.B == 0) return GDN_OK;
  if (!cu_seqlens || !cache_indices) return GDN_ERR_INVALID_ARG;
  if (s.B > kMaxValidateRequests) return GDN_ERR_UNSUPPORTED;
  // host copies of both arrays (16 bytes per request); a descriptor whose arrays cannot be
  // held on the host is refused rather than thrown through the C ABI
  std::vector<int64_t> cu, idx;
  try {
    cu.resize((size_t)s.B + 1);
    idx.resize((size_t)s.B);
  } catch (...) {  // std::bad_alloc or std::length_error
    return GDN_ERR_UNSUPPORTED;
  }
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int64_t) * cu.size(), hipMemcpyDeviceToHost,
                     st) != hipSuccess)
    return GDN_ERR_HIP;
  if (hipMemcpyAsync(idx.data(), cache_indices, sizeof(int64_t) * idx.size(),
                     hipMemcpyDeviceToHost, st) != hipSuccess)
    return GDN_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return GDN_ERR_HIP;
  if (cu[0] != 0 || cu[(size_t)s.B] != s.N) return GDN_ERR_BAD_INPUT;
  for (int64_t i = 0; i < s.B; ++i)
    if (cu[(size_t)i + 1] < cu[(size_t)i]) return GDN_ERR_BAD_INPUT;
  for (int64_t i = 0; i < s.B; ++i)
    if (idx[(size_t)i] < 0 || idx[(size_t)i] >= s.pool) return GDN_ERR_BAD_INPUT;
  // distinct slots: sort the host copy (O(B) memory, whatever the pool size)
  std::sort(idx.begin(), idx.end());
  if (std::adjacent_find(idx.begin(), idx.end()) != idx.end()) return GDN_ERR_BAD_INPUT;
  return GDN_OK;
}

}  // extern "C"
