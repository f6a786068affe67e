// kpool_compress: pooled index keys (page "Module glm5next_dsa", "Shape of the
// pipeline" and "Traps carried from Slice 8": slot-axis softmax per channel,
// anchored at the first valid token, full pools only; kpool <= 8 per
// "Constants", KERNEL_MAX_KPOOL).
//
// Two launches: an anchor kernel (one workgroup per sequence finds the first
// valid token and the number of whole pools), then a pool kernel with one
// thread per (pool, 8-channel group).  The pool kernel is HBM-bound: it reads
// kpool token rows of k and gate (2 * kpool * 2 B per channel for bf16) and
// writes one pooled row; the kpool <= 8 slot logits of each channel live in
// registers.  The pooled keys go to the tile-interleaved pool-cache layout
// (KpLayout); the padding pools of the last tile are written as zeros.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kAnchorThreads = 256;
constexpr int kAnchorBytes = 16;  // valid bytes examined per thread per window

__global__ __launch_bounds__(kAnchorThreads) void anchor_kernel(const uint8_t* __restrict__ valid,
                                                                const int32_t* __restrict__ seq_len,
                                                                int T_max, int kp,
                                                                int32_t* __restrict__ n_pools,
                                                                int32_t* __restrict__ first_valid) {
  const int b = blockIdx.x;
  int L = seq_len[b];
  L = L < 0 ? 0 : (L > T_max ? T_max : L);
  const uint8_t* v = valid + size_t(b) * T_max;
  __shared__ int s_first;
  if (threadIdx.x == 0) s_first = L;
  __syncthreads();
  // Windows of kAnchorThreads * kAnchorBytes tokens, front to back; stop at the
  // first window that holds a valid token (the smallest index in it wins).
  for (int base = 0; base < L; base += kAnchorThreads * kAnchorBytes) {
    const int t0 = base + threadIdx.x * kAnchorBytes;
    int found = L;
    for (int i = 0; i < kAnchorBytes; ++i) {
      const int t = t0 + i;
      if (t < L && v[t] != 0) { found = t; break; }
    }
    if (found < L) atomicMin(&s_first, found);
    __syncthreads();
    const int f = s_first;
    __syncthreads();
    if (f < L) break;  // uniform: every thread read the same value
  }
  if (threadIdx.x == 0) {
    const int f = s_first;
    first_valid[b] = f;
    n_pools[b] = f < L ? (L - f) / kp : 0;
  }
}

// 8 channels c0 .. c0+7 of pool p into the pool cache: one 16-byte piece for
// bf16, two for fp32
__device__ __forceinline__ void store_kp(uint16_t* k_pool, int b, int p, int c0, int P_tiles, int D,
                                         const float (&v)[8]) {
  store8(k_pool + KpLayout<uint16_t>::index(b, p, c0, P_tiles, D), v);
}
__device__ __forceinline__ void store_kp(float* k_pool, int b, int p, int c0, int P_tiles, int D,
                                         const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(k_pool + KpLayout<float>::index(b, p, c0, P_tiles, D)) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(k_pool + KpLayout<float>::index(b, p, c0 + 4, P_tiles, D)) = f32x4{v[4], v[5], v[6], v[7]};
}

// One pooled row piece: channels c0 .. c0+7 of the pool whose first slot token
// is row0 (a row index into [B*T_max]), written to the pool cache with its
// start and validity (by the c0 == 0 thread).  KP (the kpool) is a template
// argument so that all 2*KP row loads of a thread are issued before the first
// is used.  Shared by the full compress and the incremental append, so both
// produce the same bits for the same pool.
template <typename T, int KP>
__device__ __forceinline__ void pool_piece(const T* __restrict__ k, const T* __restrict__ gate,
                                           const uint8_t* __restrict__ valid,
                                           const float* __restrict__ ape, size_t row0, int t0, int b,
                                           int p, int c0, int P_tiles, int D, int P_max,
                                           T* __restrict__ k_pool, int32_t* __restrict__ pool_start,
                                           uint8_t* __restrict__ pool_valid) {
  float lg[KP][8], kv[KP][8], acc[8];
#pragma unroll
  for (int s = 0; s < KP; ++s) {
    load8(gate + (row0 + s) * D + c0, lg[s]);
    load8(k + (row0 + s) * D + c0, kv[s]);
  }
  // slot logits gate + ape and their max over the slot axis, per channel
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = -INFINITY;
#pragma unroll
  for (int s = 0; s < KP; ++s) {
    float a[8];
    load8(ape + size_t(s) * D + c0, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lg[s][e] += a[e];
      mx[e] = fmaxf(mx[e], lg[s][e]);
    }
  }
  float den[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { den[e] = 0.f; acc[e] = 0.f; }
#pragma unroll
  for (int s = 0; s < KP; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = expf(lg[s][e] - mx[e]);
      den[e] += w;
      acc[e] = fmaf(w, kv[s][e], acc[e]);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] / den[e];
  store_kp(k_pool, b, p, c0, P_tiles, D, acc);
  if (c0 == 0) {
    int all = 1;
#pragma unroll
    for (int s = 0; s < KP; ++s) all &= (valid[row0 + s] != 0);
    pool_start[size_t(b) * P_max + p] = t0;
    pool_valid[size_t(b) * P_max + p] = uint8_t(all);
  }
}

// The empty row of pool p (p >= n_pools): zero keys, start -1, not valid.
template <typename T>
__device__ __forceinline__ void empty_piece(int b, int p, int c0, int P_tiles, int D, int P_max,
                                            T* __restrict__ k_pool, int32_t* __restrict__ pool_start,
                                            uint8_t* __restrict__ pool_valid) {
  float z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = 0.f;
  store_kp(k_pool, b, p, c0, P_tiles, D, z);
  if (c0 == 0 && p < P_max) {
    pool_start[size_t(b) * P_max + p] = -1;
    pool_valid[size_t(b) * P_max + p] = 0;
  }
}

template <typename T, int KP>
__global__ __launch_bounds__(256) void pool_kernel(
    const T* __restrict__ k, const T* __restrict__ gate, const uint8_t* __restrict__ valid,
    const float* __restrict__ ape, int T_max, int D, int P_max,
    const int32_t* __restrict__ n_pools, const int32_t* __restrict__ first_valid,
    T* __restrict__ k_pool, int32_t* __restrict__ pool_start, uint8_t* __restrict__ pool_valid) {
  const int b = blockIdx.y;
  const int groups = D >> 3;
  const int P_tiles = pool_tiles(P_max);
  const long gid = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= long(P_tiles) * 16 * groups) return;
  const int p = int(gid / groups);
  const int c0 = int(gid % groups) * 8;
  if (p >= n_pools[b]) {
    empty_piece<T>(b, p, c0, P_tiles, D, P_max, k_pool, pool_start, pool_valid);
    return;
  }
  const int t0 = first_valid[b] + p * KP;
  pool_piece<T, KP>(k, gate, valid, ape, size_t(b) * T_max + t0, t0, b, p, c0, P_tiles, D, P_max, k_pool,
                    pool_start, pool_valid);
}

// Incremental pool cache: the per-sequence indexer state that the selector
// reads every decode step (page "Module glm5next_dsa", module "state").  The
// state of sequence b is (first_valid[b], n_pools[b]) plus its rows of the pool
// cache, exactly as dsa_kpool_compress leaves them for some earlier length.
// After tokens are appended (seq_len[b] grows), only the pools that became
// whole are formed; the arithmetic per pool is pool_piece, so the result is
// bit-identical to a full compress at the new length.  One workgroup per
// sequence: it moves the anchor forward over still-invalid tokens (all tokens
// before the anchor are invalid, so the scan starts there), then forms pools
// [start, end) with end - start <= max_new, and publishes the new state.  A
// length that shrank (a precondition violation) clears the rows past the new
// pool count instead, so the state stays that of a full compress.
constexpr int kAppendThreads = 256;

template <typename T, int KP>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const T* __restrict__ k, const T* __restrict__ gate, const uint8_t* __restrict__ valid,
    const float* __restrict__ ape, const int32_t* __restrict__ seq_len, int T_max, int D, int P_max,
    int max_new, T* __restrict__ k_pool, int32_t* __restrict__ pool_start,
    uint8_t* __restrict__ pool_valid, int32_t* __restrict__ n_pools, int32_t* __restrict__ first_valid) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ int s_f;
  int L = seq_len[b];
  L = L < 0 ? 0 : (L > T_max ? T_max : L);
  int f0 = first_valid[b];
  int n0 = n_pools[b];  // read with the other state, not after the scan
  f0 = f0 < 0 ? 0 : (f0 > L ? L : f0);
  n0 = n0 < 0 ? 0 : (n0 > P_max ? P_max : n0);
  const uint8_t* v = valid + size_t(b) * T_max;
  int f = f0;
  if (!(f0 < L && v[f0] != 0)) {  // uniform; a still-valid anchor (the usual case) needs no scan
    if (tid == 0) s_f = L;
    __syncthreads();
    // first valid token at or after f0 (windows of 16 tokens per thread)
    for (int base = f0; base < L; base += kAppendThreads * 16) {
      const int t0 = base + tid * 16;
      int found = L;
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + i;
        if (t < L && v[t] != 0) { found = t; break; }
      }
      if (found < L) atomicMin(&s_f, found);
      __syncthreads();
      const int fw = s_f;
      __syncthreads();
      if (fw < L) break;  // uniform
    }
    f = s_f;
  }
  // the pools to form (or, for a length that shrank, to clear); the same
  // values in every thread
  const int start = (f == f0) ? n0 : 0;  // a new anchor: no pool existed before it
  const int P_new = f < L ? (L - f) / KP : 0;
  const int form = P_new >= start ? 1 : 0;
  const int lo = form ? start : P_new;
  const int hi = form ? min(P_new, start + max_new) : start;
  const int groups = D >> 3;
  const int P_tiles = pool_tiles(P_max);
  const long items = long(hi - lo) * groups;
  for (long it = tid; it < items; it += kAppendThreads) {
    const int p = lo + int(it / groups);
    const int c0 = int(it % groups) * 8;
    if (form) {
      const int t0 = f + p * KP;
      pool_piece<T, KP>(k, gate, valid, ape, size_t(b) * T_max + t0, t0, b, p, c0, P_tiles, D, P_max, k_pool,
                        pool_start, pool_valid);
    } else {
      empty_piece<T>(b, p, c0, P_tiles, D, P_max, k_pool, pool_start, pool_valid);
    }
  }
  __syncthreads();  // every wave has read the old state
  if (tid == 0) {
    first_valid[b] = f;
    n_pools[b] = form ? hi : lo;
  }
}

template <typename T>
static void launch_append(int kp, int B, hipStream_t s, const void* k, const void* gate,
                          const uint8_t* valid, const float* ape, const int32_t* seq_len, int T_max,
                          int D, int P_max, int max_new, void* k_pool, int32_t* pool_start,
                          uint8_t* pool_valid, int32_t* n_pools, int32_t* first_valid) {
#define DSA_APPEND(KP)                                                                              \
  hipLaunchKernelGGL((append_kernel<T, KP>), dim3(B), dim3(kAppendThreads), 0, s, (const T*)k,       \
                     (const T*)gate, valid, ape, seq_len, T_max, D, P_max, max_new, (T*)k_pool,       \
                     pool_start, pool_valid, n_pools, first_valid)
  switch (kp) {
    case 1: DSA_APPEND(1); break;
    case 2: DSA_APPEND(2); break;
    case 3: DSA_APPEND(3); break;
    case 4: DSA_APPEND(4); break;
    case 5: DSA_APPEND(5); break;
    case 6: DSA_APPEND(6); break;
    case 7: DSA_APPEND(7); break;
    default: DSA_APPEND(8); break;
  }
#undef DSA_APPEND
}

template <typename T>
static void launch_pool(int kp, dim3 grid, hipStream_t s, const void* k, const void* gate,
                        const uint8_t* valid, const float* ape, int T_max, int D, int P_max,
                        const int32_t* n_pools, const int32_t* first_valid, void* k_pool,
                        int32_t* pool_start, uint8_t* pool_valid) {
#define DSA_POOL(KP)                                                                           \
  hipLaunchKernelGGL((pool_kernel<T, KP>), grid, dim3(256), 0, s, (const T*)k, (const T*)gate, \
                     valid, ape, T_max, D, P_max, n_pools, first_valid, (T*)k_pool, pool_start, \
                     pool_valid)
  switch (kp) {
    case 1: DSA_POOL(1); break;
    case 2: DSA_POOL(2); break;
    case 3: DSA_POOL(3); break;
    case 4: DSA_POOL(4); break;
    case 5: DSA_POOL(5); break;
    case 6: DSA_POOL(6); break;
    case 7: DSA_POOL(7); break;
    default: DSA_POOL(8); break;
  }
#undef DSA_POOL
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_kpool_compress(const void* k, const void* gate, const uint8_t* valid,
                                  const float* ape, const int32_t* seq_len, int B, int T_max,
                                  int D, int kpool, int P_max, int dtype, void* k_pool,
                                  int32_t* pool_start, uint8_t* pool_valid, int32_t* n_pools,
                                  int32_t* first_valid, void* stream) {
  if (!k || !gate || !valid || !ape || !seq_len || !k_pool || !pool_start || !pool_valid ||
      !n_pools || !first_valid)
    return DSA_ERR_NULL;
  if (B <= 0 || T_max <= 0 || D <= 0 || kpool <= 0 || P_max <= 0) return DSA_ERR_SHAPE;
  if (P_max < T_max / kpool) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL) return DSA_ERR_UNSUPPORTED;
  if (D % 8 != 0 || D > 1024) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  if (long(B) > 65535) return DSA_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(anchor_kernel, dim3(B), dim3(kAnchorThreads), 0, s, valid, seq_len, T_max,
                     kpool, n_pools, first_valid);
  int st = launch_status();
  if (st) return st;
  const long work = long(pool_tiles(P_max)) * 16 * (D / 8);
  dim3 grid(ceil_div(work, 256), B);
  if (dtype == DSA_BF16)
    launch_pool<uint16_t>(kpool, grid, s, k, gate, valid, ape, T_max, D, P_max, n_pools, first_valid,
                          k_pool, pool_start, pool_valid);
  else
    launch_pool<float>(kpool, grid, s, k, gate, valid, ape, T_max, D, P_max, n_pools, first_valid,
                       k_pool, pool_start, pool_valid);
  return launch_status();
}

extern "C" int dsa_kpool_append(const void* k, const void* gate, const uint8_t* valid,
                                const float* ape, const int32_t* seq_len, int B, int T_max, int D,
                                int kpool, int P_max, int max_new_pools, int dtype, void* k_pool,
                                int32_t* pool_start, uint8_t* pool_valid, int32_t* n_pools,
                                int32_t* first_valid, void* stream) {
  if (!k || !gate || !valid || !ape || !seq_len || !k_pool || !pool_start || !pool_valid ||
      !n_pools || !first_valid)
    return DSA_ERR_NULL;
  if (B <= 0 || T_max <= 0 || D <= 0 || kpool <= 0 || P_max <= 0 || max_new_pools <= 0)
    return DSA_ERR_SHAPE;
  if (P_max < T_max / kpool) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL) return DSA_ERR_UNSUPPORTED;
  if (D % 8 != 0 || D > 1024) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (dtype == DSA_BF16)
    launch_append<uint16_t>(kpool, B, s, k, gate, valid, ape, seq_len, T_max, D, P_max, max_new_pools,
                            k_pool, pool_start, pool_valid, n_pools, first_valid);
  else
    launch_append<float>(kpool, B, s, k, gate, valid, ape, seq_len, T_max, D, P_max, max_new_pools,
                         k_pool, pool_start, pool_valid, n_pools, first_valid);
  return launch_status();
}
