// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

// After a kernel launch: map a launch error to DSA_ERR_HIP.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int ceil_div(long a, long b) { return int((a + b - 1) / b); }

// Filtered scores -> top-k (index_scores.hip, topk_pools.hip): the score
// pass that keeps per (row, pool range) a list of candidate keys instead of
// the scores, and the top-k over those lists.
int filter_supported(int Q, int H, int D, int dtype);
int filter_ranges(int Q, int P_max, int max_ranges);
int index_scores_filter(const void* q, const float* w, float scale, const void* k_pool, const int32_t* pool_start,
                        const uint8_t* pool_valid, const float* ln_gamma, const float* ln_beta, float ln_eps,
                        const int32_t* row_seq, const int32_t* row_pos, int Q, int H, int B, int P_max, int kpool,
                        int K, int cap, int max_ranges, uint64_t* keys, uint32_t* counts, hipStream_t s);
int topk_lists(const uint64_t* keys, const uint32_t* counts, int nseg, int cap, int Q, int P_max, int K,
               int32_t* pool_ids, const int32_t* row_seq, const int32_t* pool_start, int B, int kpool,
               int32_t* token_ids, int W, hipStream_t s);

}  // namespace dsa
