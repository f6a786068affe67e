/*
 * dsa.h -- C ABI of libdsa.so: DeepSeek-Sparse-Attention token selection and
 * attention over the selected tokens for one GLM-5.3 DSA layer, on one
 * MI355X (gfx950) GPU.
 *
 * The five stage entry points follow the pipeline on the "Module
 * glm5next_dsa" API page, section "Shape of the pipeline":
 *
 *   k, gate, valid, ape -> dsa_kpool_compress   -> pool keys / starts / valid
 *                       -> dsa_index_scores     -> [Q, P] scores + candidate validity
 *                       -> dsa_topk_pools       -> [Q, select_k] pool ids
 *                       -> dsa_expand_selection -> [Q, out_width] token ids (-1 = invalid)
 *                       -> dsa_sparse_mla_decode (NoPE MLA restricted to those tokens)
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a caller-owned DEVICE pointer to a dense,
 *     row-major array (innermost index last, no padding), with one exception:
 *     the pool cache k_pool is tile-interleaved and padded to whole 16-pool
 *     tiles (layout below, DSA_POOL_CACHE_POOLS).  Scalars are by value.
 *   - The library allocates nothing and keeps no pointer after it returns.
 *     Calls that need scratch take a caller-sized workspace (device memory);
 *     its size comes from the matching *_workspace_bytes function, which is a
 *     pure host computation.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the default stream) and
 *     the call returns without synchronising the host.  Calls keep no state
 *     and may run concurrently on different streams with disjoint outputs and
 *     workspaces, with one exception: the counter block of a top-k workspace
 *     (see dsa_topk_pools) carries state from call to call, so calls that
 *     share one top-k workspace must not overlap.
 *   - Geometry is never defaulted: every dimension is an argument.
 *   - Every call checks its arguments on the host first.  On a negative status
 *     nothing was launched and no output was touched.
 *   - `dtype` selects the activation type (DSA_F32 or DSA_BF16) of the tensors
 *     marked "act"; parameters (ape, w, gamma, beta) and scores are always fp32.
 *   - Preconditions NOT checked on the device (callers guarantee them):
 *     finite inputs; row_seq[q] in [0, B); token ids < T_max; pool ids < P_max.
 *     Kernels still bounds-check indices they dereference, so a violation gives
 *     a wrong value (-1 / -inf / zero), never an out-of-bounds access.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DSA_OK                0
#define DSA_ERR_NULL         -1  /* a required pointer is NULL */
#define DSA_ERR_SHAPE        -2  /* a dimension is non-positive or inconsistent */
#define DSA_ERR_UNSUPPORTED  -3  /* a dimension outside what the kernels implement */
#define DSA_ERR_WORKSPACE    -4  /* workspace missing or too small */
#define DSA_ERR_HIP          -5  /* the HIP runtime reported an error at launch */
#define DSA_ERR_TOO_LARGE    -6  /* the call needs more scratch than a fixed-size buffer holds */

/* Size of the counter block at the start of a dsa_topk_pools workspace: the
 * same for every shape. */
#define DSA_TOPK_COUNTER_BYTES 262144

/* activation dtypes */
#define DSA_F32   0
#define DSA_BF16  1
/* latent-cache code type of dsa_sparse_mla_decode_paged only: OCP FP8 E4M3
 * bytes with one fp32 scale per token row */
#define DSA_FP8_E4M3  2

/*
 * The pool cache.  dsa_kpool_compress writes the pooled keys k_pool[b,p,c]
 * (b < B, p < P_max, c < D) tile-interleaved, and dsa_index_scores reads them
 * in that layout: pools are grouped in tiles of 16 (P_tiles = ceil(P_max/16)
 * tiles per sequence) and a tile stores the 16-byte pieces of its 16 pools
 * piece-major.  With E = 16 / sizeof(act) elements per piece (8 for bf16, 4 for
 * fp32), k_pool[b,p,c] sits at element
 *     (((b*P_tiles + p/16) * (D/E) + c/E) * 16 + p%16) * E + c%E
 * of a buffer of B * P_tiles * 16 * D elements (DSA_POOL_CACHE_POOLS(P_max)
 * pools per sequence; the padding pools of the last tile are zeros).  For
 * bf16 keys with D = 128 each wave-wide 16-byte load of the score kernel then
 * reads 1 KiB of contiguous memory straight into the matrix-core operand layout.
 */
#define DSA_POOL_CACHE_POOLS(P_max) ((((P_max) + 15) / 16) * 16)

/* Most pool slots (kpool) accepted.  The "Module glm5next_dsa" page, section
 * "Constants" (KERNEL_MAX_KPOOL), states that the reference compression kernel
 * holds at most 8 slots and silently truncates more; here a larger kpool is
 * refused with DSA_ERR_UNSUPPORTED. */
#define DSA_MAX_KPOOL 8

/* Largest select_k accepted by dsa_topk_pools. */
#define DSA_MAX_SELECT_K 2048

/* Human-readable text for a status code (static storage, never NULL). */
const char* dsa_status_string(int status);

/* ABI version of this header (bumped on any signature change). */
int dsa_abi_version(void);
#define DSA_ABI_VERSION 2

/*
 * dsa_kpool_compress -- pooled index keys.
 * "Module glm5next_dsa", "Shape of the pipeline" (k, gate, valid, ape ->
 * pool keys / indices / valid) and "Traps carried from Slice 8": the pool
 * softmax runs over the pool-slot axis, per channel; pooling starts at the
 * first valid token (left padding is skipped, not pooled); a pool counts only
 * if every kpool slot is valid (a trailing partial pool is not a pool).
 *
 * For sequence b with first valid token f_b (among its first seq_len[b]
 * tokens), pool p < n_pools[b] = (seq_len[b] - f_b) / kpool covers tokens
 * t_s = f_b + p*kpool + s, s < kpool, and per channel c
 *     a_s = softmax_s(gate[b,t_s,c] + ape[s,c]),  k_pool[b,p,c] = sum_s a_s k[b,t_s,c].
 * pool_valid[b,p] = 1 iff all kpool slot tokens are valid (a hole invalidates
 * its pool).  Rows p >= n_pools[b] are written as k_pool = 0,
 * pool_start = -1, pool_valid = 0: the whole output is written (k_pool
 * including the padding pools of the pool-cache layout).  A sequence with no
 * valid token gets n_pools = 0 and first_valid = seq_len[b].
 *
 *   k, gate      [B, T_max, D] act        valid [B, T_max] uint8 (nonzero = valid)
 *   ape          [kpool, D] fp32          seq_len [B] int32, each in [0, T_max]
 *   k_pool       pool cache (out): B * DSA_POOL_CACHE_POOLS(P_max) * D act
 *   pool_start   [B, P_max] int32 (out)   pool_valid [B, P_max] uint8 (out)
 *   n_pools, first_valid [B] int32 (out)
 * Requires 1 <= kpool <= DSA_MAX_KPOOL, D % 8 == 0 and D <= 1024,
 * P_max >= T_max / kpool.  Computes in fp32; bf16 outputs are rounded to
 * nearest even once.
 */
int dsa_kpool_compress(const void* k, const void* gate, const uint8_t* valid, const float* ape,
                       const int32_t* seq_len, int B, int T_max, int D, int kpool, int P_max,
                       int dtype, void* k_pool, int32_t* pool_start, uint8_t* pool_valid,
                       int32_t* n_pools, int32_t* first_valid, void* stream);

/*
 * dsa_kpool_append -- the per-sequence indexer state, advanced after tokens
 * are appended.  "Module glm5next_dsa", module list ("state": the per-sequence
 * DSA indexer state, the cache the selector reads every decode step) and the
 * compress rules quoted above dsa_kpool_compress.
 *
 * The state of sequence b is first_valid[b], n_pools[b] and its rows of
 * k_pool / pool_start / pool_valid.  On entry they must be exactly what
 * dsa_kpool_compress (or earlier calls of this function) left for a length
 * L_old <= seq_len[b], with the token data k, gate, valid of rows t < L_old
 * unchanged since.  A fresh sequence starts from dsa_kpool_compress with
 * seq_len = 0 (or the same bytes: k_pool 0, pool_start -1, pool_valid 0,
 * n_pools 0, first_valid 0).  The call moves the anchor over tokens that are
 * still invalid, forms the pools that became whole (at most max_new_pools
 * per sequence; later calls continue where this one stopped) and updates
 * first_valid and n_pools in place.  When no pool is left pending, the state
 * equals the output of dsa_kpool_compress at the new lengths bit for bit (the
 * same per-pool arithmetic).  Tensors, layouts, dtype and the limits on
 * kpool, D and P_max are those of dsa_kpool_compress; max_new_pools >= 1.
 * One workgroup per sequence: meant for decode steps that add a few tokens.
 * A length that shrank is a precondition violation; the rows past the new
 * pool count are then cleared.
 *
 *   n_pools, first_valid [B] int32: in/out state
 *   k_pool, pool_start, pool_valid: in/out (only changed rows are written)
 */
int dsa_kpool_append(const void* k, const void* gate, const uint8_t* valid, const float* ape,
                     const int32_t* seq_len, int B, int T_max, int D, int kpool, int P_max,
                     int max_new_pools, int dtype, void* k_pool, int32_t* pool_start,
                     uint8_t* pool_valid, int32_t* n_pools, int32_t* first_valid, void* stream);

/*
 * dsa_index_scores -- indexer scores with candidate validity.
 * "Module glm5next_dsa", "Shape of the pipeline" (-> [Q, P] scores + candidate
 * validity) and "Traps carried from Slice 8" (indexer.k_norm is a LayerNorm:
 * mean-subtracting, with bias); "Module tp", "Why the indexer is REPLICATED,
 * not sharded" (the score is a plain sum over heads of w[h]*relu(scale*dot)).
 *
 * For row q of sequence b = row_seq[q] and pool p (k_pool in the pool-cache
 * layout described above):
 *   kn = LayerNorm(k_pool[b,p,:]; gamma, beta, eps)   (biased variance)
 *   scores[q,p] = sum_h w[q,h] * max(0, scale * <q[q,h,:], kn>)
 * when p is a candidate -- pool_valid[b,p] != 0 and
 * pool_start[b,p] + kpool - 1 <= row_pos[q] (causal: the pool ends at or
 * before the row's position) -- and -inf otherwise.  All Q*P_max scores are
 * written.
 *
 *   q [Q, H, D] act     w [Q, H] fp32     gamma, beta [D] fp32
 *   k_pool: pool cache, B * DSA_POOL_CACHE_POOLS(P_max) * D act
 *   pool_start [B, P_max] int32 as dsa_kpool_compress / dsa_kpool_append
 *              write it: a valid pool p starts at pool_start[b,0] + p*kpool
 *              (pool p begins kpool*p tokens after the anchor); the decode
 *              kernel relies on this and reads pool_start[b,0] only
 *   pool_valid [B, P_max] uint8           row_seq, row_pos [Q] int32
 *   scores [Q, P_max] fp32 (out)
 * Requires D in {32, 64, 128} and 1 <= H <= 64.
 * Accuracy: |score - exact| <= 1e-3 |exact| + 1e-5 sum_h |w| |scale|
 * sum_c |q kn|.  The bf16 matrix-core path (D = 128, H in {16, 32}) forms
 * the LayerNorm mean and variance from sum_c x and sum_c x^2 in fp32, which
 * holds that bound for pooled keys whose mean over the D channels is at most
 * 100 standard deviations from zero (|mean| <= 100 sigma); keys further off
 * centre lose accuracy in the variance (about 3e-3 relative at 300 sigma).
 */
int dsa_index_scores(const void* q, const float* w, float scale, const void* k_pool,
                     const int32_t* pool_start, const uint8_t* pool_valid, const float* ln_gamma,
                     const float* ln_beta, float ln_eps, const int32_t* row_seq,
                     const int32_t* row_pos, int Q, int H, int D, int B, int P_max, int kpool,
                     int dtype, float* scores, void* stream);

/*
 * dsa_topk_pools -- deterministic per-row top-k of the scores.
 * "Module glm5next_dsa", "Shape of the pipeline" (-> [Q, select_k] pool ids);
 * "Module tp", "Why the indexer is REPLICATED, not sharded" (tiebreak: higher
 * score first, then the smaller pool index).
 *
 * Candidates of row q are the p with scores[q,p] != -inf.  pool_ids[q,j] is
 * the j-th candidate in (score descending, pool index ascending) order, with
 * +0.0 and -0.0 comparing equal; when a row has fewer than K candidates the
 * rest of its row is -1.  The whole [Q, K] output is written.  Scores must not
 * be NaN.
 *
 *   scores [Q, P] fp32     pool_ids [Q, K] int32 (out)
 *   workspace: device buffer of dsa_topk_workspace_bytes(Q, P, K) bytes
 *              (may be NULL when that is 0).  Its first
 *              DSA_TOPK_COUNTER_BYTES bytes are per-row merge counters, the
 *              one piece of state a call carries: the chunk workgroups of a
 *              split row count themselves in, and the last to arrive merges
 *              the row and sets its counter back to zero.  So:
 *                - before the first use, zero the counter block with
 *                  dsa_topk_workspace_init (or any zero fill);
 *                - every call that runs to completion leaves the counters
 *                  at zero, so one buffer then serves calls of any shape
 *                  that fit it (the rest of it is scratch);
 *                - calls that share a workspace must not overlap (they
 *                  would count into the same counters);
 *                - a call that did not run to completion (its stream failed
 *                  or the process was stopped while it ran) may leave
 *                  counters non-zero, after which the next call on that
 *                  workspace would merge too early or never: zero the
 *                  counter block again before reusing the workspace.
 * Requires 1 <= K <= DSA_MAX_SELECT_K and P <= 524288.
 */
size_t dsa_topk_workspace_bytes(int Q, int P, int K);
/* Zero the counter block (the first min(workspace_bytes,
 * DSA_TOPK_COUNTER_BYTES) bytes) of a top-k workspace with a fill kernel
 * queued on `stream` (no memset node, so it may be captured in a HIP graph).
 * For a new workspace, and after a call on it did not complete. */
int dsa_topk_workspace_init(void* workspace, size_t workspace_bytes, void* stream);
int dsa_topk_pools(const float* scores, int Q, int P, int K, int32_t* pool_ids, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * dsa_expand_selection -- pool ids to token ids.
 * "Module glm5next_dsa", "Shape of the pipeline" (-> [Q, out_width] token ids,
 * -1 = invalid) and "Traps carried from Slice 8" (the -1 sentinel destination
 * must be fully written).
 *
 * token_ids[q, j*kpool + s] = pool_start[b, pool_ids[q,j]] + s for j < K,
 * s < kpool, b = row_seq[q]; it is -1 where pool_ids[q,j] is -1 or names a
 * pool that does not exist (pool_start = -1), and every column >= K*kpool is -1.
 *
 *   pool_ids [Q, K] int32    row_seq [Q] int32    pool_start [B, P_max] int32
 *   token_ids [Q, W] int32 (out)
 * Requires W >= K*kpool and 1 <= kpool <= DSA_MAX_KPOOL.
 */
int dsa_expand_selection(const int32_t* pool_ids, int Q, int K, const int32_t* row_seq,
                         const int32_t* pool_start, int B, int P_max, int kpool,
                         int32_t* token_ids, int W, void* stream);

/*
 * dsa_topk_pools_expand -- dsa_topk_pools followed by dsa_expand_selection, in
 * one launch.  "Module glm5next_dsa", "Shape of the pipeline" (the selected
 * [Q, select_k] pool ids become [Q, out_width] token ids) and "Traps carried
 * from Slice 8" (the -1 sentinel destination fully written).
 *
 * Writes exactly what the two calls write: pool_ids [Q, K] as dsa_topk_pools
 * and token_ids [Q, W] as dsa_expand_selection applied to those pool ids.  The
 * workgroup that finishes a row's selection also expands it, so the decode
 * path saves one launch.  Arguments, workspace (dsa_topk_workspace_bytes, with
 * its counter block) and requirements are those of the two calls.
 */
int dsa_topk_pools_expand(const float* scores, int Q, int P, int K, int32_t* pool_ids,
                          const int32_t* row_seq, const int32_t* pool_start, int B, int P_max,
                          int kpool, int32_t* token_ids, int W, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode -- absorbed NoPE MLA decode over the selected tokens.
 * "Module glm5next_dsa", "Shape of the pipeline" (NoPE MLA restricted to the
 * selected tokens) and "Traps carried from Slice 8" (NoPE: the rotary slice is
 * zero-width); "Module tp", "Traps this module encodes" (kv_a_proj_with_mqa
 * yields one shared latent per token with no head axis, so the cache is
 * [B, T_max, Dl] and, absorbed, keys and values are the latent itself).
 *
 * For row q (b = row_seq[q]) and head h, over the ids j = token_ids[q,c] >= 0:
 *   l_j = sm_scale * <q_lat[q,h,:], kv[b,j,:]>
 *   out[q,h,:] = sum_j softmax(l)_j kv[b,j,:],   lse[q,h] = log sum_j exp(l_j)
 * A row with no id gets out = 0 and lse = -inf.  Ids are expected unique
 * (dsa_expand_selection produces unique ids); each listed entry is one term.
 *
 *   q_lat [Q, Hm, Dl] act    kv [B, T_max, Dl] act    token_ids [Q, W] int32
 *   out [Q, Hm, Dl] act (out)    lse [Q, Hm] fp32 (out, may be NULL)
 *   workspace: device buffer of dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W,
 *              dtype) bytes (may be NULL when that is 0), scratch for the
 *              split partials; calls that share it must not overlap.
 * Requires Dl in {64, 128, 256, 512}, 1 <= Hm <= 128 and W <= 16384; the bf16
 * MFMA path is taken for Dl == 512 with Hm % 16 == 0.
 */
size_t dsa_sparse_mla_workspace_bytes(int Q, int Hm, int Dl, int W, int dtype);
int dsa_sparse_mla_decode(const void* q_lat, const void* kv, const int32_t* row_seq,
                          const int32_t* token_ids, int Q, int Hm, int Dl, int B, int T_max,
                          int W, float sm_scale, int dtype, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Outputs, arguments, checks and errors are those of dsa_sparse_mla_decode
 * (the same kernels, so the same bits).  The split partials go to a buffer of
 * DSA_MLA_SCRATCH_BYTES bytes inside the library instead of a workspace:
 *   - each GPU has its own copy, held until the process ends; its address is
 *     looked up on the first call on that GPU (no allocation at any time);
 *   - a call that needs more, i.e. dsa_sparse_mla_workspace_bytes(Q, Hm, Dl,
 *     W, dtype) > DSA_MLA_SCRATCH_BYTES, returns DSA_ERR_TOO_LARGE and
 *     launches nothing;
 *   - every call on one GPU uses that GPU's buffer: calls that overlap on one
 *     GPU (different streams, or host threads) race on it, so the caller must
 *     order them (each call writes every partial it reads; nothing needs
 *     clearing between calls).
 */
#define DSA_MLA_SCRATCH_BYTES 33554432
int dsa_sparse_mla_decode_noalloc(const void* q_lat, const void* kv, const int32_t* row_seq,
                                  const int32_t* token_ids, int Q, int Hm, int Dl, int B, int T_max,
                                  int W, float sm_scale, int dtype, void* out, float* lse, void* stream);

/*
 * dsa_index_topk_pools_expand -- dsa_index_scores, then dsa_topk_pools_expand,
 * for many rows (a prefill chunk) without the [Q, P_max] score tensor.  Same
 * operations as those two calls ("Module glm5next_dsa", "Shape of the
 * pipeline": index_scores -> topk_pools -> expand_selection; see them for the
 * arguments); pool_ids [Q, K] and token_ids [Q, W] are bit-identical to the
 * two calls.  Two paths:
 *   filtered     bf16 q and keys, D = 128, H = 16 or 32, Q > 64, when the
 *                lists below fit (at most min(32768, P_max) slots per row,
 *                256 MiB in all): the score kernel stores no scores.  Each
 *                of its waves keeps, for one row and one pool range, a list
 *                of the candidates that can still be among the row's K best
 *                (one is left out only once K better ones of the same range
 *                have been seen), and a top-k over the lists selects and
 *                expands.  The lists hold 2048 keys of 8 bytes per row and
 *                range for K <= 768 (64 MiB at Q = 4096, one range per row).
 *   row-blocked  every other call: the rows are taken in blocks whose fp32
 *                scores fit 64 MiB, each block's scores written into the
 *                workspace and consumed by its top-k before the next block.
 *   workspace  dsa_index_topk_workspace_bytes(Q, P_max, K) bytes: enough for
 *              either path (the sizer does not know H, D or dtype).  No state
 *              is kept in it between calls, except the top-k counter block
 *              that it may start with (the row-blocked top-k uses it when it
 *              splits rows; the filtered path leaves it untouched): its first
 *              DSA_TOPK_COUNTER_BYTES must be zero before the first use, and
 *              every call leaves them zero (as for dsa_topk_pools).
 * Every argument check of both stages is made before any launch.
 */
size_t dsa_index_topk_workspace_bytes(int Q, int P_max, int K);
int dsa_index_topk_pools_expand(const void* q, const float* w, float scale, const void* k_pool,
                                const int32_t* pool_start, const uint8_t* pool_valid, const float* ln_gamma,
                                const float* ln_beta, float ln_eps, const int32_t* row_seq, const int32_t* row_pos,
                                int Q, int H, int D, int B, int P_max, int kpool, int dtype, int K,
                                int32_t* pool_ids, int32_t* token_ids, int W, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode_paged -- dsa_sparse_mla_decode over a paged latent
 * cache, optionally stored as fp8.  "Module glm5next_dsa", module list
 * ("attend": the launcher of the selected-index NoPE MLA *paged* decode) and
 * "Constants" (the reference's mla_paged_decode and mla_paged_decode_fp8
 * kernels).  The pages name the paged and fp8 variants but print no layout;
 * this one is:
 *   kv_pages     [num_pages, page_size, Dl]: bf16 (kv_dtype DSA_BF16) or OCP
 *                FP8 E4M3 codes, one byte each (kv_dtype DSA_FP8_E4M3)
 *   kv_scale     [num_pages, page_size] fp32: the latent value of an fp8 code
 *                is decode(code) * scale of its row; NULL for bf16 pages
 *   block_table  [B, max_pages] int32: physical page of page j of sequence b
 * Token t of sequence b (the ids of token_ids, as in dsa_sparse_mla_decode)
 * is row t % page_size of page block_table[b, t / page_size]; a token whose
 * page index is >= max_pages or whose table entry is outside [0, num_pages)
 * counts as absent, like -1.  fp8 codes are widened to bf16 exactly as they
 * are gathered (an E4M3 value is a bf16 value) and the row's scale is applied
 * to the token's logit and to its softmax weight in the value sum, which in
 * exact arithmetic is the attention of dsa_sparse_mla_decode over the rows
 * decode(code) * scale.  q_lat and out are bf16; Dl must be 512, Hm a
 * multiple of 16 up to 128.  Every row runs the split-ids path, so W > 64
 * needs the workspace sized by dsa_sparse_mla_paged_workspace_bytes.  Other
 * arguments, ownership and errors as for dsa_sparse_mla_decode.
 */
size_t dsa_sparse_mla_paged_workspace_bytes(int Q, int Hm, int Dl, int W);
int dsa_sparse_mla_decode_paged(const void* q_lat, const void* kv_pages, const float* kv_scale,
                                const int32_t* block_table, int max_pages, int page_size, int num_pages,
                                const int32_t* row_seq, const int32_t* token_ids, int Q, int Hm, int Dl,
                                int B, int W, float sm_scale, int kv_dtype, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
