// index_topk_pools_expand: index scores, top-k and expansion for many rows
// without the [Q, P] score tensor (page "Module glm5next_dsa", "Shape of the
// pipeline": index_scores -> [Q, P] scores -> topk_pools -> expand_selection;
// the operations are those of dsa_index_scores and dsa_topk_pools_expand).
//
// Filtered path (bf16 keys, D = 128, 16 or 32 heads, more than 64 rows: the
// shapes of the many-row score kernel; and lists that fit, filter_fits).  The
// score kernel does not store the
// scores: each wave keeps, for its row and its workgroup's pool range, a list
// of the candidate keys that can still be among the row's K largest (a key is
// dropped only when K larger keys of the same range have been seen; the list
// is shrunk by a radix select whenever it fills up).  A top-k over the lists
// then selects and expands.  The scores are computed by the same code as in
// dsa_index_scores and the selection is exact, so the outputs are
// bit-identical to the two calls; the workspace holds the lists (cap keys of 8
// bytes per row and range, 64 MiB at 4096 rows and K = 512) instead of 4*P
// bytes of scores per row.
//
// Row-blocked path (every other shape).  The rows are taken in blocks whose
// fp32 scores fit a fixed budget (64 MiB: inside the last-level cache, so the
// top-k reads them back from there rather than from HBM).  For each block the
// score kernel writes the block's scores into the workspace and the top-k +
// expansion kernel consumes them before the next block overwrites them.
#include <climits>

#include "dsa_host.hpp"

namespace dsa {

constexpr long kBlockScoreBytes = 64L << 20;  // fp32 scores held at once

static int block_rows(int Q, int P_max) {
  long r = kBlockScoreBytes / (4L * P_max);
  if (r >= Q) r = Q;
  else if (r >= 8) r = r / 8 * 8;
  if (r < 1) r = 1;
  if (r > 65535) r = 65535;
  return int(r);
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Filtered path: list capacity (a power of two with room for K keys, one
// score stage of 256 and as much again, so that shrinks are rare).  The path
// is taken when the score kernel's pool ranges give a row at most min(32768,
// P_max) list slots (the final top-k reads a row's slots in one workgroup, and
// the lists are to be smaller than the row's scores) and all lists fit
// kFilterListBytes.
constexpr size_t kFilterListBytes = size_t(256) << 20;

static int list_cap(int K) {
  int c = 2048;
  while (c < 2 * K + 512) c <<= 1;
  return c;
}

static bool filter_fits(int Q, int P_max, int K) {
  if (Q <= 64 || Q > 65535 || K > DSA_MAX_SELECT_K) return false;
  const long slots = long(filter_ranges(Q, P_max, INT_MAX)) * list_cap(K);
  return slots <= 32768 && slots <= P_max && size_t(Q) * slots * sizeof(uint64_t) <= kFilterListBytes;
}

// Filtered workspace: the top-k counter block, left untouched (so that a
// row-blocked call on the same workspace still finds it zero), then the lists,
// then their lengths.
static size_t filter_keys_bytes(int Q, int P_max, int K) {
  return align256(size_t(Q) * filter_ranges(Q, P_max, INT_MAX) * list_cap(K) * sizeof(uint64_t));
}
static size_t filter_bytes(int Q, int P_max, int K) {
  return DSA_TOPK_COUNTER_BYTES + filter_keys_bytes(Q, P_max, K) +
         size_t(Q) * filter_ranges(Q, P_max, INT_MAX) * sizeof(uint32_t);
}

static size_t block_topk_bytes(int Q, int P_max, int K) {
  const int R = block_rows(Q, P_max);
  size_t t = dsa_topk_workspace_bytes(R, P_max, K);
  const int rem = Q % R;
  if (rem) {
    const size_t t2 = dsa_topk_workspace_bytes(rem, P_max, K);
    t = t2 > t ? t2 : t;
  }
  return t;
}

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_index_topk_workspace_bytes(int Q, int P_max, int K) {
  if (Q <= 0 || P_max <= 0 || K <= 0) return 0;
  const int R = block_rows(Q, P_max);
  const size_t blocked = align256(block_topk_bytes(Q, P_max, K)) + size_t(R) * P_max * sizeof(float);
  if (!filter_fits(Q, P_max, K)) return blocked;
  const size_t filtered = filter_bytes(Q, P_max, K);
  return filtered > blocked ? filtered : blocked;
}

extern "C" int dsa_index_topk_pools_expand(const void* q, const float* w, float scale, const void* k_pool,
                                           const int32_t* pool_start, const uint8_t* pool_valid,
                                           const float* ln_gamma, const float* ln_beta, float ln_eps,
                                           const int32_t* row_seq, const int32_t* row_pos, int Q, int H, int D,
                                           int B, int P_max, int kpool, int dtype, int K, int32_t* pool_ids,
                                           int32_t* token_ids, int W, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  // every check of the two stages first, so that a negative status means
  // that nothing was launched
  if (!q || !w || !k_pool || !pool_start || !pool_valid || !ln_gamma || !ln_beta || !row_seq || !row_pos ||
      !pool_ids || !token_ids)
    return DSA_ERR_NULL;
  if (Q <= 0 || H <= 0 || D <= 0 || B <= 0 || P_max <= 0 || kpool <= 0 || K <= 0 || W <= 0)
    return DSA_ERR_SHAPE;
  if (long(W) < long(K) * kpool) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL || K > DSA_MAX_SELECT_K) return DSA_ERR_UNSUPPORTED;
  if (H > 64 || (D != 32 && D != 64 && D != 128)) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  if (long(P_max) > 32768L * 16) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_index_topk_workspace_bytes(Q, P_max, K);
  if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  if (filter_supported(Q, H, D, dtype) && filter_fits(Q, P_max, K)) {
    const int cap = list_cap(K), max_ranges = INT_MAX;
    const int nseg = filter_ranges(Q, P_max, max_ranges);
    char* base = static_cast<char*>(workspace) + DSA_TOPK_COUNTER_BYTES;
    uint64_t* keys = reinterpret_cast<uint64_t*>(base);
    uint32_t* counts = reinterpret_cast<uint32_t*>(base + filter_keys_bytes(Q, P_max, K));
    const int st = index_scores_filter(q, w, scale, k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq,
                                       row_pos, Q, H, B, P_max, kpool, K, cap, max_ranges, keys, counts, s);
    if (st) return st;
    return topk_lists(keys, counts, nseg, cap, Q, P_max, K, pool_ids, row_seq, pool_start, B, kpool, token_ids, W, s);
  }
  const int R = block_rows(Q, P_max);
  const size_t tk_bytes = block_topk_bytes(Q, P_max, K);
  void* tk_ws = tk_bytes ? workspace : nullptr;
  float* sc = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(tk_bytes));
  const size_t elt = dtype == DSA_BF16 ? 2 : 4;
  for (int r0 = 0; r0 < Q; r0 += R) {
    const int Rb = Q - r0 < R ? Q - r0 : R;
    int st = dsa_index_scores(static_cast<const char*>(q) + size_t(r0) * H * D * elt, w + size_t(r0) * H, scale,
                              k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq + r0, row_pos + r0,
                              Rb, H, D, B, P_max, kpool, dtype, sc, stream);
    if (st) return st;
    st = dsa_topk_pools_expand(sc, Rb, P_max, K, pool_ids + size_t(r0) * K, row_seq + r0, pool_start, B, P_max,
                               kpool, token_ids + size_t(r0) * W, W, tk_ws, tk_bytes, stream);
    if (st) return st;
  }
  return DSA_OK;
}
