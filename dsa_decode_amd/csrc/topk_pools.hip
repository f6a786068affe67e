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
// skipped, then 11-bit digits are histogrammed in LDS until the bin holding the
// K-th key is exactly consumed (about three passes for distinct scores).  Long rows are split
// into chunks whose K largest keys go to a workspace; a merge launch selects
// the K largest of the chunk winners (the K largest of a union are among the
// K largest of each part, so this is exact).  The final K keys are sorted with
// a bitonic network in LDS and written as pool ids, -1 padded.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kTkMaxChunk = 32768;  // keys per workgroup (1024 threads x 32)
constexpr int kTkMaxSplit = 16;     // chunks merged by one merge launch

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float f, uint32_t idx) {
  return (uint64_t(score_key(f)) << 32) | uint64_t(0xffffffffu - idx);
}

constexpr int kDig = 11;              // radix digit width
constexpr int kBins = 1 << kDig;      // 2048 bins, 32 per lane of the scanning wave

template <int NT>
struct TkShared {
  static constexpr int NW = NT / kWave;
  uint32_t hist[kBins];
  uint64_t sel[DSA_MAX_SELECT_K];
  uint64_t red[NW][2];
  uint32_t cnt[NW];
  uint64_t bound[2];
  uint32_t bin_info[3];
  uint32_t nsel;
};

// Number of valid keys and their max / min over the workgroup (one barrier;
// the LDS slots are not rewritten before the caller's next barrier).
template <int NT, int KPT>
__device__ __forceinline__ uint32_t block_stats(const uint64_t (&key)[KPT], TkShared<NT>& sh, uint64_t& mx,
                                                uint64_t& mn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t c = 0;
  mx = 0;
  mn = ~uint64_t(0);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (key[j] != 0) {
      ++c;
      mx = key[j] > mx ? key[j] : mx;
      mn = key[j] < mn ? key[j] : mn;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    c += __shfl_xor(c, o, kWave);
    const uint64_t a = __shfl_xor(mx, o, kWave), b = __shfl_xor(mn, o, kWave);
    mx = a > mx ? a : mx;
    mn = b < mn ? b : mn;
  }
  if (lane == 0) {
    sh.cnt[wave] = c;
    sh.red[wave][0] = mx;
    sh.red[wave][1] = mn;
  }
  __syncthreads();
  uint32_t tot = 0;
  mx = 0;
  mn = ~uint64_t(0);
  for (int w = 0; w < TkShared<NT>::NW; ++w) {
    tot += sh.cnt[w];
    mx = sh.red[w][0] > mx ? sh.red[w][0] : mx;
    mn = sh.red[w][1] < mn ? sh.red[w][1] : mn;
  }
  return tot;
}

// Returns (prefix, lo): the selected keys are exactly those != 0 with
// (key >> lo) >= (prefix >> lo).  Requires n_valid > K; mx / mn are the largest
// and smallest valid keys.
template <int NT, int KPT>
__device__ void radix_select(const uint64_t (&key)[KPT], int K, TkShared<NT>& sh, uint64_t mx, uint64_t mn,
                             uint64_t& prefix_out, int& lo_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // n_valid > K >= 1 and keys are distinct, so mx != mn
  const int top = 63 - __clzll(mx ^ mn);      // highest differing bit
  uint64_t prefix = (top == 63) ? 0 : (mx >> (top + 1)) << (top + 1);
  uint32_t need = uint32_t(K);
  int hi = top;
  int lo = 0;
  for (int u = tid; u < kBins; u += NT) sh.hist[u] = 0;
  __syncthreads();
  while (true) {
    lo = hi >= kDig - 1 ? hi - (kDig - 1) : 0;
    const int width = hi - lo + 1;
    const uint64_t dmask = (uint64_t(1) << width) - 1;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t k = key[j];
      const bool match = k != 0 && (hi == 63 || (k >> (hi + 1)) == (prefix >> (hi + 1)));
      if (match) atomicAdd(&sh.hist[uint32_t((k >> lo) & dmask)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins 32*lane .. 32*lane+31 (read, then cleared for the next
      // pass); suffix sums over bins (high to low)
      u32x4* hv = reinterpret_cast<u32x4*>(&sh.hist[32 * lane]);
      u32x4 cv[8];
      uint32_t lane_tot = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cv[i] = hv[i];
        lane_tot += (cv[i][0] + cv[i][1]) + (cv[i][2] + cv[i][3]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) hv[i] = u32x4{0u, 0u, 0u, 0u};
      uint32_t incl = lane_tot;  // sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(incl, o, kWave);
        if (lane + o < 64) incl += v;
      }
      uint32_t above = incl - lane_tot;  // keys in bins of higher lanes
      int found = -1;
      uint32_t f_above = 0, f_cnt = 0;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          if (found < 0 && above + cv[i][e] >= need) { found = 32 * lane + 4 * i + e; f_above = above; f_cnt = cv[i][e]; }
          above += cv[i][e];
        }
      }
      // exactly one lane holds the bin where the running count first reaches need
      if (found >= 0 && f_above < need) {
        sh.bin_info[0] = uint32_t(found);
        sh.bin_info[1] = f_above;
        sh.bin_info[2] = f_cnt;
      }
    }
    __syncthreads();
    // bin_info is rewritten only after the next pass's barrier
    const uint32_t d = sh.bin_info[0], above = sh.bin_info[1], cnt = sh.bin_info[2];
    prefix |= uint64_t(d) << lo;
    need -= above;
    if (cnt == need || lo == 0) break;
    hi = lo - 1;
  }
  prefix_out = prefix;
  lo_out = lo;
}

// Exclusive prefix sum of one value per thread over the workgroup.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, TkShared<NT>& sh, uint32_t& total) {
  constexpr int NW = TkShared<NT>::NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh.cnt[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = sh.cnt[w];
    base += w < wave ? c : 0u;
    total += c;
  }
  __syncthreads();
  return base + incl - v;
}

// value of lane (lane ^ TJ) for TJ < 32: DPP for 1, 2, 4, 8 (quad permutes,
// row shifts and the 8-lane row rotate), ds_swizzle (xor mode) for 16
template <int TJ>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (TJ == 1) {
    return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (TJ == 2) {
    return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (TJ == 4) {
    const uint32_t up = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0xF, false);  // row_shl:4 (lane + 4)
    const uint32_t dn = __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false);  // row_shr:4 (lane - 4)
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (TJ == 8) {
    return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else {
    static_assert(TJ == 16, "in-wave xor distance");
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);                     // xor 16 within 32 lanes
  }
}

template <int TJ>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  if constexpr (TJ < 32) {
    const uint32_t lo = xor_lane<TJ>(uint32_t(v)), hi = xor_lane<TJ>(uint32_t(v >> 32));
    return (uint64_t(hi) << 32) | lo;
  } else {
    return __shfl_xor(v, TJ, kWave);
  }
}

// one compare-exchange step of the bitonic network: element pair distance j =
// 2*TJ (thread distance TJ), sort direction from k
template <int NT, int TJ>
__device__ __forceinline__ void bitonic_step(uint64_t& a0, uint64_t& a1, int k, TkShared<NT>& sh) {
  const int t = threadIdx.x;
  const bool act = t < 256;
  const bool desc = ((2 * t) & k) == 0;
  uint64_t b0 = 0, b1 = 0;
  if constexpr (TJ < 64) {
    b0 = xor_lane64<TJ>(a0);
    b1 = xor_lane64<TJ>(a1);
  } else {
    if (act) { sh.sel[2 * t] = a0; sh.sel[2 * t + 1] = a1; }
    __syncthreads();
    if (act) { b0 = sh.sel[2 * (t ^ TJ)]; b1 = sh.sel[2 * (t ^ TJ) + 1]; }
    __syncthreads();
  }
  const bool keep_max = ((t & TJ) == 0) == desc;
  a0 = keep_max ? (a0 > b0 ? a0 : b0) : (a0 < b0 ? a0 : b0);
  a1 = keep_max ? (a1 > b1 ? a1 : b1) : (a1 < b1 ? a1 : b1);
}

// Sort 512 keys descending, two per thread: thread t < 256 holds elements 2t
// (a0) and 2t+1 (a1).  Bitonic network: the j = 1 exchanges stay in a thread,
// in-wave partners are exchanged with DPP / swizzle / shuffles, and the three
// cross-wave steps go through LDS.  Threads >= 256 only take part in barriers
// (their results are discarded).
template <int NT>
__device__ __forceinline__ void sort512_desc(uint64_t& a0, uint64_t& a1, TkShared<NT>& sh) {
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 2; k <= 512; k <<= 1) {
    const bool desc = ((2 * t) & k) == 0;
    if (k >= 512) bitonic_step<NT, 128>(a0, a1, k, sh);
    if (k >= 256) bitonic_step<NT, 64>(a0, a1, k, sh);
    if (k >= 128) bitonic_step<NT, 32>(a0, a1, k, sh);
    if (k >= 64) bitonic_step<NT, 16>(a0, a1, k, sh);
    if (k >= 32) bitonic_step<NT, 8>(a0, a1, k, sh);
    if (k >= 16) bitonic_step<NT, 4>(a0, a1, k, sh);
    if (k >= 8) bitonic_step<NT, 2>(a0, a1, k, sh);
    if (k >= 4) bitonic_step<NT, 1>(a0, a1, k, sh);
    // j = 1: the thread's own pair
    const bool sw = desc ? (a0 < a1) : (a0 > a1);
    const uint64_t x = sw ? a1 : a0, y = sw ? a0 : a1;
    a0 = x;
    a1 = y;
  }
}

// Sort sh.sel[0..kp2) descending in LDS (kp2 a power of two <= DSA_MAX_SELECT_K;
// used when select_k > 512).
template <int NT>
__device__ void bitonic_desc(TkShared<NT>& sh, int kp2) {
  for (int k = 2; k <= kp2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < kp2; i += NT) {
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

// One workgroup: select the K largest keys of its KPT*NT keys and
// either write them unsorted to the workspace (partial) or sort and write ids.
template <int NT, int KPT, bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                          const uint64_t* __restrict__ keys_in,
                                                          int P, int chunk, int nsplit_in, int K,
                                                          uint64_t* __restrict__ keys_out,
                                                          int32_t* __restrict__ pool_ids) {
  __shared__ TkShared<NT> sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  uint64_t key[KPT];
  // all loads are issued before any is used (clamped, in-bounds addresses),
  // so that they are in flight together
  if (FROM_SCORES) {
    const float* s = scores + size_t(row) * P;
    const int base = c * chunk;
    const int end = min(P, base + chunk);
    float v[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = base + j * NT + tid;
      v[j] = s[p < end ? p : P - 1];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = base + j * NT + tid;
      key[j] = (p < end && v[j] != -INFINITY) ? make_key(v[j], uint32_t(p)) : 0;
    }
  } else {
    const uint64_t* src = keys_in + size_t(row) * nsplit_in * K;
    const int n = nsplit_in * K;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = j * NT + tid;
      key[j] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j * NT + tid >= n) key[j] = 0;
  }
  uint64_t kmax, kmin;
  const uint32_t nvalid = block_stats<NT, KPT>(key, sh, kmax, kmin);  // one barrier
  uint64_t prefix = 1;
  int lo = 0;
  if (nvalid > uint32_t(K)) radix_select<NT, KPT>(key, K, sh, kmax, kmin, prefix, lo);
  const uint64_t thr = prefix >> lo;
  uint32_t selmask = 0;  // bit j: key[j] is selected (KPT <= 32)
#pragma unroll
  for (int j = 0; j < KPT; ++j) selmask |= (key[j] != 0 && (key[j] >> lo) >= thr) ? (1u << j) : 0u;
  uint32_t nsel = 0;
  uint32_t at = block_excl_scan<NT>(uint32_t(__builtin_popcount(selmask)), sh, nsel);  // nsel = min(K, nvalid)
  if (!FINAL) {
    uint64_t* out = keys_out + (size_t(row) * gridDim.x + c) * K;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if ((selmask >> j) & 1u) out[at++] = key[j];
    for (int i = int(nsel) + tid; i < K; i += NT) out[i] = 0;
    return;
  }
  int kp2 = 1;
  while (kp2 < K) kp2 <<= 1;
  if (kp2 < 512) kp2 = 512;
  for (int i = tid; i < kp2; i += NT) sh.sel[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((selmask >> j) & 1u) sh.sel[at++] = key[j];
  __syncthreads();
  int32_t* dst = pool_ids + size_t(row) * K;
  if (kp2 == 512) {
    uint64_t a0 = 0, a1 = 0;
    if (tid < 256) { a0 = sh.sel[2 * tid]; a1 = sh.sel[2 * tid + 1]; }
    __syncthreads();
    sort512_desc<NT>(a0, a1, sh);
    if (tid < 256) {
      const int e0 = 2 * tid, e1 = 2 * tid + 1;
      if (e0 < K) dst[e0] = (e0 < int(nsel) && a0 != 0) ? int32_t(0xffffffffu - uint32_t(a0)) : -1;
      if (e1 < K) dst[e1] = (e1 < int(nsel) && a1 != 0) ? int32_t(0xffffffffu - uint32_t(a1)) : -1;
    }
    return;
  }
  bitonic_desc<NT>(sh, kp2);
  for (int i = tid; i < K; i += NT) {
    const uint64_t k = sh.sel[i];
    dst[i] = (i < int(nsel) && k != 0) ? int32_t(0xffffffffu - uint32_t(k)) : -1;
  }
}

struct TkPlan {
  int nsplit;  // chunks per row (1: single launch)
  int chunk;   // pools per chunk
  int nt1, kpt1;  // first launch: threads and keys per thread
  int nt2, kpt2;  // merge launch
};

static int pow2_at_least(long v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// threads and keys per thread for n keys: 256 threads while that needs at most
// 32 keys each, else 1024 threads
static void tk_shape(long n, int& nt, int& kpt) {
  nt = n <= 256L * 32 ? 256 : 1024;
  kpt = pow2_at_least((n + nt - 1) / nt);
}

static TkPlan tk_plan(int Q, int P, int K) {
  TkPlan pl{1, P, 256, 1, 256, 0};
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
  tk_shape(pl.chunk, pl.nt1, pl.kpt1);
  if (nsplit > 1) tk_shape(long(nsplit) * K, pl.nt2, pl.kpt2);
  return pl;
}

template <int NT, bool FROM_SCORES, bool FINAL>
static void launch_tk(int kpt, dim3 grid, hipStream_t s, const float* scores, const uint64_t* keys_in,
                      int P, int chunk, int nsplit_in, int K, uint64_t* keys_out, int32_t* pool_ids) {
#define DSA_TK(KPT)                                                                                \
  hipLaunchKernelGGL((topk_kernel<NT, KPT, FROM_SCORES, FINAL>), grid, dim3(NT), 0, s, scores,    \
                     keys_in, P, chunk, nsplit_in, K, keys_out, pool_ids)
  switch (kpt) {
    case 1: DSA_TK(1); break;
    case 2: DSA_TK(2); break;
    case 4: DSA_TK(4); break;
    case 8: DSA_TK(8); break;
    case 16: DSA_TK(16); break;
    default: DSA_TK(32); break;
  }
#undef DSA_TK
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
  if (pl.nsplit > kTkMaxSplit || pl.kpt1 > 32 || pl.kpt2 > 32) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_topk_workspace_bytes(Q, P, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  dim3 g1(pl.nsplit, Q);
  if (pl.nsplit == 1) {
    if (pl.nt1 == 256) launch_tk<256, true, true>(pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, nullptr, pool_ids);
    else launch_tk<1024, true, true>(pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, nullptr, pool_ids);
    return launch_status();
  }
  if (pl.nt1 == 256) launch_tk<256, true, false>(pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, ws, nullptr);
  else launch_tk<1024, true, false>(pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, ws, nullptr);
  int st = launch_status();
  if (st) return st;
  dim3 g2(1, Q);
  if (pl.nt2 == 256) launch_tk<256, false, true>(pl.kpt2, g2, s, nullptr, ws, P, 0, pl.nsplit, K, nullptr, pool_ids);
  else launch_tk<1024, false, true>(pl.kpt2, g2, s, nullptr, ws, P, 0, pl.nsplit, K, nullptr, pool_ids);
  return launch_status();
}
