// Internal declarations of the prefill's backward: workspace layout and launcher.
// Not part of the public C ABI (include/gdn.h).
#pragma once

#include "gdn_internal.h"

namespace gdn {

// Backward of the prefill (fp32 arithmetic): workspace layout and launcher.
struct BwdLayout {
  int64_t max_chunks = 0;  // N / 8 + B: checkpoints per value head at most
  size_t chunk_off = 0;    // int32 [B + 1]
  size_t chunk_seq = 0;    // int32 [max_chunks]
  size_t ck = 0;           // float [max_chunks][HV][dv][dk]: state every 8 tokens
  size_t part = 0;         // float [dv / 32][N][HV][2 dk + 2]: per-row-block token sums
  size_t dal = 0;          // float [N][HV]
  size_t qn = 0, kn = 0;   // float [N][H][dk]: normalised q and k
  size_t ab = 0;           // float [N][HV][2]: alpha, beta
  size_t total = 0;
};
BwdLayout bwd_layout_for(const Shape& s);
bool bwd_grids_fit(const Shape& s);
hipError_t launch_backward(const Shape& s, const BwdLayout& L, char* ws, const void* q,
                           const void* k, const void* v, const float* a, const float* b,
                           const float* A_log, const float* dt_bias, const float* state_pool,
                           const int64_t* cache_indices, const int64_t* cu_seqlens,
                           const void* dout, const float* dstate, float* dq, float* dk,
                           float* dv, float* da, float* db, float* dA_log, float* ddt_bias,
                           float* dstate0, hipStream_t st);

}  // namespace gdn
