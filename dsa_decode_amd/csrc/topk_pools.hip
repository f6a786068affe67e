// topk_pools: deterministic per-row top-k (page "Module glm5next_dsa", "Shape
// of the pipeline": -> [Q, select_k] pool ids; page "Module tp", "Why the
// indexer is REPLICATED, not sharded": higher score first, then the smaller
// pool index).
//
// Every candidate becomes one 64-bit key: the high word maps the fp32 score to
// an unsigned integer with the same order (-0 folded onto +0), the low word is
// 0xffffffff - pool index.  Larger key = earlier in the output, and all keys of
// a row are distinct, so "the K largest keys" is exactly the wanted set and
// "keys descending" exactly the wanted order.  Key 0 means "no candidate".
//
// Selection is a radix select inside one workgroup over keys held in
// registers: the bits common to the row's largest and smallest key are
// skipped, then 8-bit digits are histogrammed (one LDS histogram per wave)
// until the bin holding the K-th key is exactly consumed.  Long rows are split
// into chunks whose K largest keys go to a workspace; a merge launch selects
// the K largest of the chunk winners (the K largest of a union are among the
// K largest of each part, so this is exact).  The final K keys are sorted with
// a bitonic network in LDS and written as pool ids, -1 padded.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkMaxChunk = 32768;  // keys per workgroup (kTkThreads * 32)
constexpr int kTkMaxSplit = 16;     // chunks merged by one merge launch

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float f, uint32_t idx) {
  return (uint64_t(score_key(f)) << 32) | uint64_t(0xffffffffu - idx);
}

struct TkShared {
  uint32_t hist[kTkWaves][256];
  uint64_t sel[DSA_MAX_SELECT_K];
  uint64_t red[kTkWaves][2];
  uint32_t cnt[kTkWaves];
  uint64_t bound[2];
  uint32_t bin_info[3];
  uint32_t nsel;
};

template <int KPT>
__device__ __forceinline__ uint32_t block_count_valid(const uint64_t (&key)[KPT], TkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) c += key[j] != 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
  if (lane == 0) sh.cnt[wave] = c;
  __syncthreads();
  uint32_t tot = 0;
  for (int w = 0; w < kTkWaves; ++w) tot += sh.cnt[w];
  __syncthreads();
  return tot;
}

// Returns (prefix, lo): the selected keys are exactly those != 0 with
// (key >> lo) >= (prefix >> lo).  Requires n_valid > K.
template <int KPT>
__device__ void radix_select(const uint64_t (&key)[KPT], int K, TkShared& sh, uint64_t& prefix_out,
                             int& lo_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block max / min of the valid keys
  uint64_t mx = 0, mn = ~uint64_t(0);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (key[j] != 0) {
      mx = key[j] > mx ? key[j] : mx;
      mn = key[j] < mn ? key[j] : mn;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t a = __shfl_xor(mx, o, kWave), b = __shfl_xor(mn, o, kWave);
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
  if (lane == 0) { sh.red[wave][0] = mx; sh.red[wave][1] = mn; }
  __syncthreads();
  mx = 0; mn = ~uint64_t(0);
  for (int w = 0; w < kTkWaves; ++w) {
    mx = sh.red[w][0] > mx ? sh.red[w][0] : mx;
    mn = sh.red[w][1] < mn ? sh.red[w][1] : mn;
  }
  // n_valid > K >= 1 and keys are distinct, so mx != mn
  const int top = 63 - __clzll(mx ^ mn);      // highest differing bit
  uint64_t prefix = (top == 63) ? 0 : (mx >> (top + 1)) << (top + 1);
  uint32_t need = uint32_t(K);
  int hi = top;
  int lo = 0;
  while (true) {
    lo = hi >= 7 ? hi - 7 : 0;
    const int width = hi - lo + 1;
    const uint64_t dmask = (uint64_t(1) << width) - 1;
    // zero the per-wave histograms
    for (int u = tid; u < kTkWaves * 256; u += kTkThreads) (&sh.hist[0][0])[u] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t k = key[j];
      const bool match = k != 0 && (hi == 63 || (k >> (hi + 1)) == (prefix >> (hi + 1)));
      if (match) atomicAdd(&sh.hist[wave][uint32_t((k >> lo) & dmask)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 4*lane .. 4*lane+3; suffix sums over bins (high to low)
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t s = 0;
        for (int w = 0; w < kTkWaves; ++w) s += sh.hist[w][4 * lane + i];
        c[i] = s;
      }
      const uint32_t lane_tot = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = lane_tot;  // sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(incl, o, kWave);
        if (lane + o < 64) incl += v;
      }
      uint32_t above = incl - lane_tot;  // keys in bins of higher lanes
      int found = -1;
      uint32_t f_above = 0, f_cnt = 0;
      for (int i = 3; i >= 0; --i) {
        if (found < 0 && above + c[i] >= need) { found = 4 * lane + i; f_above = above; f_cnt = c[i]; }
        above += c[i];
      }
      // exactly one lane holds the bin where the running count first reaches need
      if (found >= 0 && f_above < need) {
        sh.bin_info[0] = uint32_t(found);
        sh.bin_info[1] = f_above;
        sh.bin_info[2] = f_cnt;
      }
    }
    __syncthreads();
    const uint32_t d = sh.bin_info[0], above = sh.bin_info[1], cnt = sh.bin_info[2];
    __syncthreads();
    prefix |= uint64_t(d) << lo;
    need -= above;
    if (cnt == need || lo == 0) break;
    hi = lo - 1;
  }
  prefix_out = prefix;
  lo_out = lo;
}

// Sort sh.sel[0..n) descending (n <= kp2 <= DSA_MAX_SELECT_K, entries past n are 0).
__device__ void bitonic_desc(TkShared& sh, int kp2) {
  for (int k = 2; k <= kp2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < kp2; i += kTkThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = sh.sel[i], b = sh.sel[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) { sh.sel[i] = b; sh.sel[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
}

// One workgroup: select the K largest keys of its KPT*kTkThreads keys and
// either write them unsorted to the workspace (partial) or sort and write ids.
template <int KPT, bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores,
                                                          const uint64_t* __restrict__ keys_in,
                                                          int P, int chunk, int nsplit_in, int K,
                                                          uint64_t* __restrict__ keys_out,
                                                          int32_t* __restrict__ pool_ids) {
  __shared__ TkShared sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  uint64_t key[KPT];
  if (FROM_SCORES) {
    const float* s = scores + size_t(row) * P;
    const int base = c * chunk;
    const int end = min(P, base + chunk);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = base + j * kTkThreads + tid;
      key[j] = 0;
      if (p < end) {
        const float v = s[p];
        if (v != -INFINITY) key[j] = make_key(v, uint32_t(p));
      }
    }
  } else {
    const uint64_t* src = keys_in + size_t(row) * nsplit_in * K;
    const int n = nsplit_in * K;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = j * kTkThreads + tid;
      key[j] = i < n ? src[i] : 0;
    }
  }
  if (tid == 0) sh.nsel = 0;
  const uint32_t nvalid = block_count_valid<KPT>(key, sh);  // has barriers
  uint64_t prefix = 1;
  int lo = 0;
  if (nvalid > uint32_t(K)) radix_select<KPT>(key, K, sh, prefix, lo);
  const uint64_t thr = prefix >> lo;
  const uint32_t nsel = nvalid < uint32_t(K) ? nvalid : uint32_t(K);
  int kp2 = 1;
  while (kp2 < K) kp2 <<= 1;
  if (FINAL)
    for (int i = tid; i < kp2; i += kTkThreads) sh.sel[i] = 0;
  __syncthreads();
  uint64_t* out = FINAL ? nullptr : keys_out + (size_t(row) * gridDim.x + c) * K;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t k = key[j];
    if (k != 0 && (k >> lo) >= thr) {
      const uint32_t at = atomicAdd(&sh.nsel, 1u);
      if (FINAL) sh.sel[at] = k;
      else out[at] = k;
    }
  }
  if (!FINAL) {
    for (int i = int(nsel) + tid; i < K; i += kTkThreads) out[i] = 0;
    return;
  }
  __syncthreads();
  bitonic_desc(sh, kp2);
  int32_t* dst = pool_ids + size_t(row) * K;
  for (int i = tid; i < K; i += kTkThreads) {
    const uint64_t k = sh.sel[i];
    dst[i] = (i < int(nsel) && k != 0) ? int32_t(0xffffffffu - uint32_t(k)) : -1;
  }
}

struct TkPlan {
  int nsplit;  // chunks per row (1: single launch)
  int chunk;   // pools per chunk
  int kpt;     // keys per thread in the first launch
  int kpt_merge;
};

static int pow2_at_least(long v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

static TkPlan tk_plan(int Q, int P, int K) {
  TkPlan pl{1, P, 1, 0};
  int nsplit = 1;
  if (P > kTkMaxChunk) nsplit = int((P + kTkMaxChunk - 1) / kTkMaxChunk);
  if (Q < 256) {
    // few rows: spread each row over chunks of >= 4096 pools (and >= 4K) so
    // that enough workgroups run; the merge then sees nsplit*K keys
    const int min_chunk = K * 4 > 4096 ? K * 4 : 4096;
    int want = (P + min_chunk - 1) / min_chunk;
    if (want > kTkMaxSplit) want = kTkMaxSplit;
    if (want > nsplit) nsplit = want;
  }
  pl.nsplit = nsplit;
  pl.chunk = (P + nsplit - 1) / nsplit;
  pl.kpt = pow2_at_least((pl.chunk + kTkThreads - 1) / kTkThreads);
  pl.kpt_merge = nsplit > 1 ? pow2_at_least((long(nsplit) * K + kTkThreads - 1) / kTkThreads) : 0;
  return pl;
}

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_topk_workspace_bytes(int Q, int P, int K) {
  if (Q <= 0 || P <= 0 || K <= 0) return 0;
  const TkPlan pl = tk_plan(Q, P, K);
  return pl.nsplit > 1 ? size_t(Q) * pl.nsplit * K * sizeof(uint64_t) : 0;
}

extern "C" int dsa_topk_pools(const float* scores, int Q, int P, int K, int32_t* pool_ids,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !pool_ids) return DSA_ERR_NULL;
  if (Q <= 0 || P <= 0 || K <= 0) return DSA_ERR_SHAPE;
  if (K > DSA_MAX_SELECT_K) return DSA_ERR_UNSUPPORTED;
  if (long(P) > long(kTkMaxChunk) * kTkMaxSplit) return DSA_ERR_UNSUPPORTED;
  if (Q > 65535) return DSA_ERR_UNSUPPORTED;
  const TkPlan pl = tk_plan(Q, P, K);
  if (pl.nsplit > kTkMaxSplit || pl.kpt > 32 || pl.kpt_merge > 32) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_topk_workspace_bytes(Q, P, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  dim3 g1(pl.nsplit, Q);
#define DSA_TK1(KPT)                                                                              \
  do {                                                                                            \
    if (pl.nsplit == 1)                                                                           \
      hipLaunchKernelGGL((topk_kernel<KPT, true, true>), g1, dim3(kTkThreads), 0, s, scores,      \
                         nullptr, P, pl.chunk, 0, K, nullptr, pool_ids);                          \
    else                                                                                          \
      hipLaunchKernelGGL((topk_kernel<KPT, true, false>), g1, dim3(kTkThreads), 0, s, scores,     \
                         nullptr, P, pl.chunk, 0, K, ws, nullptr);                                \
  } while (0)
  switch (pl.kpt) {
    case 1: DSA_TK1(1); break;
    case 2: DSA_TK1(2); break;
    case 4: DSA_TK1(4); break;
    case 8: DSA_TK1(8); break;
    case 16: DSA_TK1(16); break;
    default: DSA_TK1(32); break;
  }
#undef DSA_TK1
  int st = launch_status();
  if (st || pl.nsplit == 1) return st;
  dim3 g2(1, Q);
#define DSA_TK2(KPT)                                                                               \
  hipLaunchKernelGGL((topk_kernel<KPT, false, true>), g2, dim3(kTkThreads), 0, s, nullptr, ws, P, \
                     0, pl.nsplit, K, nullptr, pool_ids)
  switch (pl.kpt_merge) {
    case 1: DSA_TK2(1); break;
    case 2: DSA_TK2(2); break;
    case 4: DSA_TK2(4); break;
    case 8: DSA_TK2(8); break;
    case 16: DSA_TK2(16); break;
    default: DSA_TK2(32); break;
  }
#undef DSA_TK2
  return launch_status();
}
