// index_topk_pools_expand: index scores, top-k and expansion for many rows
// without holding the whole [Q, P] score tensor (page "Module glm5next_dsa",
// "Shape of the pipeline": index_scores -> [Q, P] scores -> topk_pools ->
// expand_selection; the stages themselves are those of dsa_index_scores and
// dsa_topk_pools_expand).
//
// The rows are taken in blocks whose fp32 scores fit a fixed budget (64 MiB:
// inside the last-level cache, so the top-k reads them back from there rather
// than from HBM).  For each block the score kernel writes the block's scores
// into the workspace and the top-k + expansion kernel consumes them before the
// next block overwrites them.  The kernels and their arithmetic are the
// unfused ones, so the outputs are bit-identical to dsa_index_scores followed
// by dsa_topk_pools_expand; only the score storage is bounded.
#include "dsa_host.hpp"

namespace dsa {

constexpr long kStreamScoreBytes = 64L << 20;  // fp32 scores held at once

static int stream_rows(int Q, int P_max) {
  long r = kStreamScoreBytes / (4L * P_max);
  if (r >= Q) r = Q;
  else if (r >= 8) r = r / 8 * 8;
  if (r < 1) r = 1;
  if (r > 65535) r = 65535;
  return int(r);
}

static size_t stream_align(size_t v) { return (v + 255) & ~size_t(255); }

static size_t stream_topk_bytes(int Q, int P_max, int K) {
  const int R = stream_rows(Q, P_max);
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
  const int R = stream_rows(Q, P_max);
  return stream_align(stream_topk_bytes(Q, P_max, K)) + size_t(R) * P_max * sizeof(float);
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
  const int R = stream_rows(Q, P_max);
  const size_t tk_bytes = stream_topk_bytes(Q, P_max, K);
  void* tk_ws = tk_bytes ? workspace : nullptr;
  float* sc = reinterpret_cast<float*>(static_cast<char*>(workspace) + stream_align(tk_bytes));
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
