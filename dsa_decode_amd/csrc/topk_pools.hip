// topk_pools: deterministic per-row top-k (page "Module glm5next_dsa", "Shape
// of the pipeline": -> [Q, select_k] pool ids; page "Module tp", "Why the
// indexer is REPLICATED, not sharded": higher score first, then the smaller
// pool index).
//
// Order.  Every candidate is the pair (hi, lo): hi maps the fp32 score to a
// nonzero u32 with the same order (-0 folded onto +0; 0 marks a non-candidate),
// lo = 0xffffffff - pool index.  The 64-bit key (hi << 32 | lo) is larger
// exactly when the pool comes earlier in the output, and all keys of a row are
// distinct, so "the K largest keys" is the wanted set and "keys descending"
// the wanted order.
//
// Selection runs inside one workgroup over keys held in registers, latency
// first (a decode row has only a few workgroups in flight):
//  * a first pass histograms the candidates into bins of equal width between
//    the smallest and the largest score (512 to 2048 bins, about 4 keys per
//    bin on average; the map is monotone, so the bins keep the key order and
//    tied scores share a bin); one wave scans the histogram with DPP prefix
//    sums and finds the bin of the K-th key;
//  * when every bin from that one up holds at most 256 keys, those keys are
//    scattered bin by bin into LDS and each is placed directly: output
//    position = keys in higher bins + its rank among its bin mates;
//  * otherwise (a large tie, or scores spread too widely for equal bins) a
//    radix select on 11-bit digits of the key bits below those common to all
//    candidates finds the K-th key; a tie at the K-th score is broken by
//    position (ballot ranks) for raw scores and by the lo bits for chunk
//    winners; the selected keys are then sorted by a bitonic network.
// Long rows are split into chunks whose K largest keys (sorted) go to a
// workspace; the K largest of the chunk winners are the row's (the K largest
// of a union are among the K largest of each part, so this is exact).  For
// the decode shapes this runs in one launch: the chunk workgroups publish
// their winners and the last one to finish merges them, first from the heads
// of the sorted lists (exact whenever no list can hold winners past its head)
// and else from the full lists.  Otherwise a second launch merges.
#include "dsa_common.hpp"
#include "dsa_host.hpp"
#include "dsa_select.hpp"

namespace dsa {

constexpr int kTkMaxChunk = 32768;  // keys per workgroup (1024 threads x 32)
constexpr int kTkMaxSplit = 16;     // chunks merged by one merge launch

constexpr int kDig = 11;              // radix digit width
constexpr int kBins = 1 << kDig;      // 2048 bins, 32 per lane of the scanning wave
constexpr int kRankCap = 256;         // largest bin that is ordered by pairwise ranks

// Bins of the first (linear) pass for n keys: about 4 keys per bin on average,
// between 512 and kBins (the single-wave scan of the histogram is on the
// critical path, and its cost follows the number of bins).
template <int N>
constexpr int first_pass_bins() {
  return N <= 2048 ? 512 : (N <= 4096 ? 1024 : kBins);
}

template <int NT>
struct TkShared {
  static constexpr int NW = NT / kWave;
  alignas(16) uint32_t hist[kBins];
  alignas(16) uint32_t sfx[kBins];  // first pass: keys in higher bins, per bin
  uint64_t sel[DSA_MAX_SELECT_K + kRankCap];
  int32_t sel_ps[DSA_MAX_SELECT_K + kRankCap];  // merge with expansion: pool_start of sel[i]
  uint32_t red[NW][4];
  uint32_t tie[32 * NW];  // per (key slot, wave): tied keys, then their exclusive prefix
  uint32_t info[4];
  uint32_t slot;
  uint32_t ticket;
  uint32_t flag;
};

// Valid keys (hi != 0): their number, largest and smallest hi (one barrier;
// the LDS slots are not rewritten before the caller's next barrier).
template <int NT, int KPT>
__device__ __forceinline__ void block_stats(const uint32_t (&hi)[KPT], TkShared<NT>& sh, uint32_t& n,
                                            uint32_t& mx, uint32_t& mn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t c = 0, a = 0, b = 0;  // count, max hi, max ~hi (= ~min hi)
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool v = hi[j] != 0;
    c += v ? 1u : 0u;
    a = max(a, hi[j]);
    b = max(b, v ? ~hi[j] : 0u);
  }
  c = __builtin_amdgcn_readlane(wave_incl_sum(c), 63);
  a = wave_max_u32(a);
  b = wave_max_u32(b);
  if (lane == 0) {
    sh.red[wave][0] = c;
    sh.red[wave][1] = a;
    sh.red[wave][2] = b;
  }
  __syncthreads();
  if constexpr (TkShared<NT>::NW > 8) {
    // lane w of every wave takes wave w's partials and the wave reductions
    // combine them: three registers, where reading all 16 waves' partials at
    // once held 48 and pushed the 32-key kernel into spills (the histogram
    // loop then reloaded its key mask from scratch for every key)
    uint32_t c2 = 0, a2 = 0, b2 = 0;
    if (lane < TkShared<NT>::NW) {
      c2 = sh.red[lane][0];
      a2 = sh.red[lane][1];
      b2 = sh.red[lane][2];
    }
    n = __builtin_amdgcn_readlane(wave_incl_sum(c2), 63);
    mx = wave_max_u32(a2);
    mn = ~wave_max_u32(b2);
  } else {
    // up to 8 waves: every lane reads all the partials (shorter latency)
    n = 0;
    mx = 0;
    b = 0;
#pragma unroll
    for (int w = 0; w < TkShared<NT>::NW; ++w) {
      n += sh.red[w][0];
      mx = max(mx, sh.red[w][1]);
      b = max(b, sh.red[w][2]);
    }
    mn = ~b;
  }
}

// Wave 0: scans the histogram from the highest bin down and finds the bin where
// the running count reaches need (need >= 1, and the histogram holds at least
// need keys).  Writes (bin, keys in higher bins, keys in the bin) to sh.info
// and clears the histogram for the next pass.
// With SFX it also writes, for every bin, the number of keys in higher bins
// to sh.sfx, and the largest count of a bin at or above the found one to
// sh.info[3].
template <int NT, bool SFX = false, int NB = kBins>
__device__ __forceinline__ void scan_find(TkShared<NT>& sh, uint32_t need) {
  static_assert(NB == 512 || NB == 1024 || NB == 2048, "bins scanned");
  constexpr int BPL = NB / kWave;  // bins per lane
  constexpr int V = BPL / 4;
  const int lane = threadIdx.x & 63;
  u32x4* hv = reinterpret_cast<u32x4*>(&sh.hist[BPL * lane]);  // bins BPL*lane .. BPL*lane+BPL-1
  u32x4 cv[V];
  uint32_t tot = 0, lmax = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    cv[i] = hv[i];
    tot += (cv[i][0] + cv[i][1]) + (cv[i][2] + cv[i][3]);
    if (SFX) lmax = max(lmax, max(max(cv[i][0], cv[i][1]), max(cv[i][2], cv[i][3])));
  }
  const uint32_t incl = wave_incl_sum(tot);
  const uint32_t above = __builtin_amdgcn_readlane(incl, 63) - incl;  // keys in higher lanes' bins
  // lanes 0..L satisfy this (the count from the top is non-increasing in lane)
  const uint64_t b = __ballot(above + tot >= need);
  const int L = 63 - __builtin_clzll(b);
  const uint32_t aboveL = __builtin_amdgcn_readlane(above, L);
  // lane L's BPL bins, highest first, over lanes 0..BPL-1
  const uint32_t x = lane < BPL ? sh.hist[BPL * L + BPL - 1 - lane] : 0u;
  const uint32_t xin = wave_incl_sum(x);
  const uint64_t b2 = __ballot(aboveL + xin >= need);
  const int i = __builtin_ctzll(b2);
  const uint32_t xi = __builtin_amdgcn_readlane(x, i);
  const uint32_t xin_i = __builtin_amdgcn_readlane(xin, i);
  uint32_t maxc = 0;
  if (SFX) {
    u32x4* sv = reinterpret_cast<u32x4*>(&sh.sfx[BPL * lane]);
    uint32_t run = above;
#pragma unroll
    for (int k = V - 1; k >= 0; --k) {
      u32x4 o;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        o[e] = run;
        run += cv[k][e];
      }
      sv[k] = o;
    }
    // lanes above L hold only bins above the found one; lanes 0..i hold lane
    // L's bins down to the found one
    maxc = wave_max_u32(max(lane > L ? lmax : 0u, lane <= i ? x : 0u));
  }
#pragma unroll
  for (int k = 0; k < V; ++k) hv[k] = u32x4{0u, 0u, 0u, 0u};
  if (lane == 0) {
    sh.info[0] = uint32_t(BPL * L + BPL - 1 - i);
    sh.info[1] = aboveL + xin_i - xi;
    sh.info[2] = xi;
    sh.info[3] = maxc;
  }
}

struct RadixResult {
  uint32_t prefix;  // decided bits (bits >= lo)
  int lo;           // lowest decided bit
  uint32_t cnt;     // keys whose bits >= lo equal prefix's
  uint32_t need;    // of those, how many are selected
};

// Radix select over the 32-bit values v[j] with bit j of vmask set.  Bits above
// h are already decided (equal to prefix's for every key in vmask).  The
// histogram is zero on entry and on return.  On return the selected keys are
// those with (v >> lo) > (prefix >> lo), plus `need` of the cnt keys with
// (v >> lo) == (prefix >> lo) (all of them when cnt == need).
template <int NT, int KPT>
__device__ __forceinline__ RadixResult radix_on(const uint32_t (&v)[KPT], uint32_t vmask, int h, uint32_t prefix,
                                uint32_t need, TkShared<NT>& sh) {
  while (true) {
    const int lo = h >= kDig - 1 ? h - (kDig - 1) : 0;
    const uint32_t hmask = h >= 31 ? 0u : (0xffffffffu << (h + 1));
    const uint32_t want = prefix & hmask;
    const uint32_t dmask = (2u << (h - lo)) - 1u;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (((vmask >> j) & 1u) && (v[j] & hmask) == want) atomicAdd(&sh.hist[(v[j] >> lo) & dmask], 1u);
    __syncthreads();
    if ((threadIdx.x >> 6) == 0) scan_find<NT>(sh, need);
    __syncthreads();
    // sh.info is rewritten only after the next pass's first barrier
    const uint32_t d = sh.info[0], above = sh.info[1], cnt = sh.info[2];
    prefix = want | (d << lo);
    need -= above;
    if (cnt == need || lo == 0) return {prefix, lo, cnt, need};
    h = lo - 1;
  }
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
__device__ __forceinline__ void bitonic_desc(TkShared<NT>& sh, int kp2) {
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

// Tied keys (bit j of eqm) at the K-th score, taken in position order: key
// slot j of thread t is position base + j*NT + t.  Returns the mask of the
// first `need` of them (two barriers).
template <int NT, int KPT>
__device__ __forceinline__ uint32_t tie_by_position(uint32_t eqm, uint32_t need, TkShared<NT>& sh) {
  constexpr int NW = TkShared<NT>::NW;
  constexpr int NE = KPT * NW;                       // (slot, wave) counters
  constexpr int PER = (NE + kWave - 1) / kWave;      // counters per lane of wave 0
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t m = __ballot((eqm >> j) & 1u);
    if (lane == 0) sh.tie[j * NW + wave] = uint32_t(__builtin_popcountll(m));
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t c[PER], s = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = lane * PER + e;
      c[e] = i < NE ? sh.tie[i] : 0u;
      s += c[e];
    }
    uint32_t run = wave_incl_sum(s) - s;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = lane * PER + e;
      if (i < NE) sh.tie[i] = run;
      run += c[e];
    }
  }
  __syncthreads();
  uint32_t take = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t m = __ballot((eqm >> j) & 1u);  // recomputed: cheaper than holding KPT ranks
    if (((eqm >> j) & 1u) && sh.tie[j * NW + wave] + lane_rank(m) < need) take |= 1u << j;
  }
  return take;
}

// One workgroup: select the K largest keys of its KPT*NT keys and either write
// them unsorted to the workspace (partial) or sort them and write pool ids.
// A chunk winner for the merge: an agent-scope store (written through to the
// device's coherence point, so the merging workgroup can read it without
// whole-cache writeback and invalidation).
__device__ __forceinline__ void publish(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Selection followed by expansion (dsa_topk_pools_expand): the thread that
// places a row's j-th pool id also writes that pool's token ids, with the
// rules of dsa_expand_selection (kpool consecutive ids from pool_start, -1 for
// an absent or nonexistent pool); the columns past K*kpool are written -1.
struct ExpandArgs {
  const int32_t* row_seq;
  const int32_t* pool_start;
  int B, P_max, kp;
  int32_t* token_ids;  // nullptr: no expansion
  int W;
  int seq;  // the sequence of the workgroup's row (row_seq, read once at kernel entry)
};

// ex with seq set for row: one uniform load at kernel entry, so that a pool's
// start is a single load once the pool is known (not behind a load of the
// row's sequence in every lane that expands)
__device__ __forceinline__ ExpandArgs expand_for_row(const ExpandArgs& ex, int row) {
  ExpandArgs r = ex;
  r.seq = ex.token_ids ? ex.row_seq[row] : -1;
  return r;
}

// pool_start of pool pid for the row's sequence (-1: absent or nonexistent)
__device__ __forceinline__ int32_t expand_start(int32_t pid, const ExpandArgs& ex) {
  const int b = ex.seq;
  int32_t ps = -1;
  if (pid >= 0 && pid < ex.P_max && b >= 0 && b < ex.B) ps = ex.pool_start[size_t(b) * ex.P_max + pid];
  return ps;
}

__device__ __forceinline__ void expand_write(int row, int j, int32_t ps, const ExpandArgs& ex) {
  int32_t* t = ex.token_ids + size_t(row) * ex.W + size_t(j) * ex.kp;
  for (int sl = 0; sl < ex.kp; ++sl) t[sl] = ps >= 0 ? ps + sl : -1;
}

__device__ __forceinline__ void expand_one(int row, int j, int32_t pid, const ExpandArgs& ex) {
  expand_write(row, j, expand_start(pid, ex), ex);
}

template <int NT>
__device__ __forceinline__ void expand_pad(int row, int K, const ExpandArgs& ex) {
  for (int col = K * ex.kp + int(threadIdx.x); col < ex.W; col += NT) ex.token_ids[size_t(row) * ex.W + col] = -1;
}

// One workgroup's selection: chunk c of row `row` (FROM_SCORES: pools c*chunk
// .. of the scores; otherwise the nsplit_in chunk winner lists of the row) ->
// its K largest keys, written to chunk slot c of keys_out (partial) or sorted
// to pool_ids (FINAL).  nchunk: chunk slots per row of keys_out.
// With lcounts (and FROM_SCORES false) the input is instead the row's
// nsplit_in candidate lists of the filtering score pass, lcap keys apart (lcap
// a power of two), list l holding lcounts[row * nsplit_in + l] keys.
template <int NT, int KPT, bool FROM_SCORES, bool FINAL>
__device__ __forceinline__ void topk_block(TkShared<NT>& sh, int row, int c, int nchunk, const float* __restrict__ scores,
                           const uint64_t* __restrict__ keys_in, int P, int chunk, int nsplit_in, int K,
                           uint64_t* __restrict__ keys_out, int32_t* __restrict__ pool_ids,
                           const ExpandArgs& ex, const uint32_t* __restrict__ lcounts = nullptr, int lcap = 0) {
  static_assert(KPT <= 32, "selection masks are 32-bit");
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t hi[KPT];
  uint32_t lo[FROM_SCORES ? 1 : KPT];
  const int base = c * chunk;
  // all loads are issued before any is used, so that they are in flight
  // together; buffer loads past the chunk's end return 0
  if constexpr (FROM_SCORES) {
    const int end = min(P, base + chunk);
    const auto rs = make_rsrc(scores + size_t(row) * P + base, uint32_t(max(end - base, 0)) * 4u);
    float v[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (j * NT + tid) * 4, 0, 0));
    // The range test is an AND with a mask the compiler cannot see through:
    // as a select it becomes a branch per key, with the load sunk into it.
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      uint32_t in = base + j * NT + tid < end ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(in));
      hi[j] = score_key(v[j]) & in;
    }
  } else if (lcounts) {
    // candidate lists: only each list's first lcounts keys are loaded
    const int n = nsplit_in * lcap;
    const int lsh = __builtin_ctz(uint32_t(lcap));
    const uint64_t* src = keys_in + size_t(row) * n;
    uint32_t len[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = j * NT + tid;
      len[j] = i < n ? lcounts[size_t(row) * nsplit_in + (i >> lsh)] : 0u;
    }
    uint64_t k[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = j * NT + tid;
      k[j] = uint32_t(i & (lcap - 1)) < len[j] ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                : 0ull;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      hi[j] = uint32_t(k[j] >> 32);  // 0 past a list's end
      lo[j] = uint32_t(k[j]);
    }
  } else {
    // chunk winners published by other workgroups of this launch: agent-scope
    // loads (coherent with their agent-scope stores, no cache maintenance)
    const int n = nsplit_in * K;
    const uint64_t* src = keys_in + size_t(row) * n;
    uint64_t k[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = j * NT + tid;
      k[j] = __hip_atomic_load(src + (i < n ? i : n - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool in = j * NT + tid < n;
      hi[j] = in ? uint32_t(k[j] >> 32) : 0u;  // 0 for padding keys and past the end
      lo[j] = uint32_t(k[j]);
    }
  }
  if (tid == 0) sh.slot = 0;
  for (int u = tid; u < kBins; u += NT) sh.hist[u] = 0;
  uint32_t nvalid, kmax, kmin;
  block_stats<NT, KPT>(hi, sh, nvalid, kmax, kmin);  // its barrier also publishes the cleared LDS
  const uint32_t nsel = min(nvalid, uint32_t(K));

  uint32_t vmask = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) vmask |= hi[j] != 0 ? (1u << j) : 0u;
  // the 64-bit key of slot j
  auto key_of = [&](int j) -> uint64_t {
    const uint32_t l = FROM_SCORES ? 0xffffffffu - uint32_t(base + j * NT + tid) : lo[FROM_SCORES ? 0 : j];
    return (uint64_t(hi[j]) << 32) | l;
  };
  uint32_t selmask = vmask;
  if (nvalid > uint32_t(K)) {
    RadixResult st;
    if (kmax == kmin) {
      st = {kmax, 0, nvalid, uint32_t(K)};  // every candidate has the same score
    } else {
      // First pass: NB1 bins of equal width in score between the smallest
      // and the largest candidate (fp32 subtraction and scaling are monotone,
      // so bins keep the key order, ties included).  It also leaves, per bin,
      // the number of keys in higher bins.
      const float fmn = key_float(kmin);
      constexpr int NB1 = first_pass_bins<NT * KPT>();
      const float scale = float(NB1) / (key_float(kmax) - fmn);  // 0 if the range overflows
      auto bin_of = [&](uint32_t k) -> uint32_t {
        return min(uint32_t((key_float(k) - fmn) * scale), uint32_t(NB1 - 1));
      };
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if ((vmask >> j) & 1u) atomicAdd(&sh.hist[bin_of(hi[j])], 1u);
      __syncthreads();
      if ((tid >> 6) == 0) scan_find<NT, true, NB1>(sh, uint32_t(K));
      __syncthreads();
      const uint32_t t = sh.info[0], above = sh.info[1], cnt = sh.info[2], maxc = sh.info[3];
      if (maxc <= uint32_t(kRankCap)) {
        // Every bin from the K-th key's bin up holds at most kRankCap keys:
        // output position = keys in higher bins + rank inside the own bin.
        // Keys are gathered per bin in LDS (the cleared histogram counts the
        // slots), then ranked against their bin mates.
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t d = bin_of(hi[j]);
          if (((vmask >> j) & 1u) && d >= t) sh.sel[sh.sfx[d] + atomicAdd(&sh.hist[d], 1u)] = key_of(j);
        }
        __syncthreads();
        // slots [0, above + cnt) now hold the keys of those bins, bin by bin;
        // one thread per slot ranks its key (bin mates read four at a time)
        uint64_t* out = FINAL ? nullptr : keys_out + (size_t(row) * nchunk + c) * K;
        int32_t* dst = FINAL ? pool_ids + size_t(row) * K : nullptr;
        for (uint32_t sl = tid; sl < above + cnt; sl += NT) {
          const uint64_t me = sh.sel[sl];
          const uint32_t d = bin_of(uint32_t(me >> 32));
          const uint32_t r0 = sh.sfx[d], n = sh.hist[d];
          uint32_t pos = r0;
          for (uint32_t i = 0; i < n; i += 4) {
            const uint64_t a0 = sh.sel[r0 + i];
            const uint64_t a1 = sh.sel[r0 + min(i + 1, n - 1)];
            const uint64_t a2 = sh.sel[r0 + min(i + 2, n - 1)];
            const uint64_t a3 = sh.sel[r0 + min(i + 3, n - 1)];
            pos += (a0 > me ? 1u : 0u) + (i + 1 < n && a1 > me ? 1u : 0u) + (i + 2 < n && a2 > me ? 1u : 0u) +
                   (i + 3 < n && a3 > me ? 1u : 0u);
          }
          if (pos < uint32_t(K)) {
            if constexpr (FINAL) {
              dst[pos] = int32_t(0xffffffffu - uint32_t(me));
              if (ex.token_ids) expand_one(row, int(pos), int32_t(0xffffffffu - uint32_t(me)), ex);
            } else {
              publish(out + pos, me);
            }
          }
        }
        return;
      }
      // a bin at or above the K-th key's is large (ties, or scores spread
      // over many orders of magnitude): radix select on the key bits below
      // those common to every candidate (the histogram is clear again)
      const int top = 31 - __builtin_clz(kmax ^ kmin);
      const uint32_t pre = top >= 31 ? 0u : (kmax & (0xffffffffu << (top + 1)));
      st = radix_on<NT, KPT>(hi, vmask, top, pre, uint32_t(K), sh);
    }
    const uint32_t thr = st.prefix >> st.lo;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      gt |= ((vmask >> j) & 1u) && (hi[j] >> st.lo) > thr ? (1u << j) : 0u;
      eq |= ((vmask >> j) & 1u) && (hi[j] >> st.lo) == thr ? (1u << j) : 0u;
    }
    if (st.cnt == st.need) {
      selmask = gt | eq;
    } else if constexpr (FROM_SCORES) {
      // the K-th score is tied: smaller positions first
      selmask = gt | tie_by_position<NT, KPT>(eq, st.need, sh);
    } else {
      // the K-th score is tied: radix select on lo among the tied keys.  lo =
      // ~index with index < P, so the bits above P-1's top bit are all ones.
      const int h2 = P > 1 ? 31 - __builtin_clz(uint32_t(P - 1)) : 0;
      const uint32_t pre2 = h2 >= 31 ? 0u : (0xffffffffu << (h2 + 1));
      const RadixResult s2 = radix_on<NT, KPT>(lo, eq, h2, pre2, st.need, sh);
      const uint32_t thr2 = s2.prefix >> s2.lo;
      uint32_t take = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) take |= ((eq >> j) & 1u) && (lo[j] >> s2.lo) >= thr2 ? (1u << j) : 0u;
      selmask = gt | take;
    }
  }

  // output slots: a DPP scan of the per-thread counts and one LDS atomic per wave
  const uint32_t mine = uint32_t(__builtin_popcount(selmask));
  const uint32_t incl = wave_incl_sum(mine);
  uint32_t wbase = 0;
  if (lane == 63) wbase = atomicAdd(&sh.slot, incl);
  uint32_t at = __builtin_amdgcn_readlane(wbase, 63) + incl - mine;

  // sort the selected keys (0-padded) in LDS; chunk winners (partial) are
  // written sorted too, as the merge reads only the head of each list first
  int kp2 = 1;
  while (kp2 < K) kp2 <<= 1;
  if (kp2 < 512) kp2 = 512;
  for (int i = int(nsel) + tid; i < kp2; i += NT) sh.sel[i] = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((selmask >> j) & 1u) sh.sel[at++] = key_of(j);
  __syncthreads();
  uint64_t* out = FINAL ? nullptr : keys_out + (size_t(row) * nchunk + c) * K;
  int32_t* dst = FINAL ? pool_ids + size_t(row) * K : nullptr;
  auto emit = [&](int e, uint64_t k) {
    if constexpr (FINAL) {
      const int32_t pid = (e < int(nsel) && k != 0) ? int32_t(0xffffffffu - uint32_t(k)) : -1;
      dst[e] = pid;
      if (ex.token_ids) expand_one(row, e, pid, ex);
    } else {
      publish(out + e, e < int(nsel) ? k : 0);
    }
  };
  if (kp2 == 512) {
    uint64_t a0 = 0, a1 = 0;
    if (tid < 256) { a0 = sh.sel[2 * tid]; a1 = sh.sel[2 * tid + 1]; }
    __syncthreads();
    sort512_desc<NT>(a0, a1, sh);
    if (tid < 256) {
      if (2 * tid < K) emit(2 * tid, a0);
      if (2 * tid + 1 < K) emit(2 * tid + 1, a1);
    }
    return;
  }
  bitonic_desc<NT>(sh, kp2);
  for (int i = tid; i < K; i += NT) emit(i, sh.sel[i]);
}

// Merge of a row's S sorted chunk-winner lists (stride K) from their first m
// keys each (S*m keys, m < K).  The row's K winners are exactly the K largest
// of these when no list could hold further winners past its first m, which is
// certain when the m-th key of every full list lies below the bin of the K-th
// largest key.  Takes the first-pass/rank path; returns false, having written
// nothing, when a list may hold more winners or the first pass does not apply
// (the caller then merges the full lists).
template <int NT, int KPT>
__device__ __forceinline__ bool merge_heads(TkShared<NT>& sh, int row, int S, int m, int K,
                                            const uint64_t* __restrict__ keys, int32_t* __restrict__ pool_ids,
                                            const ExpandArgs& ex) {
  static_assert(KPT <= 32, "selection masks are 32-bit");
  const int tid = threadIdx.x;
  const int n = S * m;
  const uint64_t* src = keys + size_t(row) * S * K;
  uint64_t k[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = j * NT + tid;
    const int ii = i < n ? i : n - 1;
    k[j] = __hip_atomic_load(src + size_t(ii / m) * K + ii % m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  uint32_t hi[KPT], lo[KPT];
  uint32_t vmask = 0, lastmask = 0;  // valid keys; keys that end a list's head
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = j * NT + tid;
    const bool in = i < n;
    hi[j] = in ? uint32_t(k[j] >> 32) : 0u;
    lo[j] = uint32_t(k[j]);
    vmask |= hi[j] != 0 ? (1u << j) : 0u;
    lastmask |= (in && i % m == m - 1) ? (1u << j) : 0u;
  }
  // with expansion: every winner is among these keys, so their pool starts
  // are requested now and arrive while the selection runs
  int32_t ps[KPT];
  if (ex.token_ids) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) ps[j] = (vmask >> j) & 1u ? expand_start(int32_t(0xffffffffu - lo[j]), ex) : -1;
  }
  if (tid == 0) sh.flag = 0;
  for (int u = tid; u < kBins; u += NT) sh.hist[u] = 0;
  uint32_t nvalid, kmax, kmin;
  block_stats<NT, KPT>(hi, sh, nvalid, kmax, kmin);
  if (nvalid <= uint32_t(K) || kmax == kmin) return false;
  const float fmn = key_float(kmin);
  constexpr int NB1 = first_pass_bins<NT * KPT>();
  const float scale = float(NB1) / (key_float(kmax) - fmn);
  auto bin_of = [&](uint32_t key) -> uint32_t {
    return min(uint32_t((key_float(key) - fmn) * scale), uint32_t(NB1 - 1));
  };
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((vmask >> j) & 1u) atomicAdd(&sh.hist[bin_of(hi[j])], 1u);
  __syncthreads();
  if ((tid >> 6) == 0) scan_find<NT, true, NB1>(sh, uint32_t(K));
  __syncthreads();
  const uint32_t t = sh.info[0], above = sh.info[1], cnt = sh.info[2], maxc = sh.info[3];
  if (maxc > uint32_t(kRankCap)) return false;
  // scatter the keys of bins >= t; flag a full list head that reaches bin t
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t d = bin_of(hi[j]);
    if (((vmask >> j) & 1u) && d >= t) {
      const uint32_t at = sh.sfx[d] + atomicAdd(&sh.hist[d], 1u);
      sh.sel[at] = (uint64_t(hi[j]) << 32) | lo[j];
      if (ex.token_ids) sh.sel_ps[at] = ps[j];
      if ((lastmask >> j) & 1u) sh.flag = 1;
    }
  }
  __syncthreads();
  if (sh.flag) return false;
  int32_t* dst = pool_ids + size_t(row) * K;
  for (uint32_t sl = tid; sl < above + cnt; sl += NT) {
    const uint64_t me = sh.sel[sl];
    const uint32_t d = bin_of(uint32_t(me >> 32));
    const uint32_t r0 = sh.sfx[d], nb = sh.hist[d];
    uint32_t pos = r0;
    for (uint32_t i = 0; i < nb; i += 4) {
      const uint64_t a0 = sh.sel[r0 + i];
      const uint64_t a1 = sh.sel[r0 + min(i + 1, nb - 1)];
      const uint64_t a2 = sh.sel[r0 + min(i + 2, nb - 1)];
      const uint64_t a3 = sh.sel[r0 + min(i + 3, nb - 1)];
      pos += (a0 > me ? 1u : 0u) + (i + 1 < nb && a1 > me ? 1u : 0u) + (i + 2 < nb && a2 > me ? 1u : 0u) +
             (i + 3 < nb && a3 > me ? 1u : 0u);
    }
    if (pos < uint32_t(K)) {
      dst[pos] = int32_t(0xffffffffu - uint32_t(me));
      if (ex.token_ids) expand_write(row, int(pos), sh.sel_ps[sl], ex);
    }
  }
  return true;
}

template <int NT, int KPT, bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                  const uint64_t* __restrict__ keys_in,
                                                  int P, int chunk, int nsplit_in, int K,
                                                  uint64_t* __restrict__ keys_out,
                                                  int32_t* __restrict__ pool_ids, ExpandArgs ex,
                                                  const uint32_t* __restrict__ lcounts, int lcap) {
  __shared__ TkShared<NT> sh;
  const ExpandArgs exr = expand_for_row(ex, blockIdx.y);
  if constexpr (FINAL)
    if (ex.token_ids) expand_pad<NT>(blockIdx.y, K, ex);
  topk_block<NT, KPT, FROM_SCORES, FINAL>(sh, blockIdx.y, blockIdx.x, gridDim.x, scores, keys_in, P, chunk,
                                          nsplit_in, K, keys_out, pool_ids, exr, lcounts, lcap);
}

// Split rows in one launch: workgroup (c, row) selects chunk c's K winners,
// publishes them (agent-scope stores, complete before it moves on), and takes
// a ticket from the row's counter; the workgroup that takes the last ticket
// (all chunks of the row are then published) resets the counter to zero and
// merges the row's winner lists.  A counter that starts at zero is zero again
// after every call.
template <int NT, int KPT1, int KPTH, int KPT2>
__global__ __launch_bounds__(NT) void topk_split_kernel(const float* __restrict__ scores, int P, int chunk,
                                                        int nsplit, int K, int m, uint64_t* __restrict__ keys,
                                                        uint32_t* __restrict__ counters,
                                                        int32_t* __restrict__ pool_ids, ExpandArgs ex) {
  __shared__ TkShared<NT> sh;
  const int row = blockIdx.y;
  const ExpandArgs exr = expand_for_row(ex, row);
  topk_block<NT, KPT1, true, false>(sh, row, blockIdx.x, nsplit, scores, nullptr, P, chunk, 0, K, keys, nullptr,
                                    ExpandArgs{});
  // Ordering of the hand-over (what release / acquire at agent scope would
  // give, built from its parts).  On gfx950 an agent-scope release is a
  // write-back of the L2's dirty lines followed by a wait for the workgroup's
  // stores to complete, and an agent-scope acquire invalidates the caches that
  // are not coherent across the XCDs.  Here the only data handed over are the
  // winners, and they are stored with agent-scope atomics, which write through
  // to the device's coherence point and leave no dirty line of theirs in the
  // L2: the write-back has nothing of this hand-over to do, and the wait below
  // (every thread's stores acknowledged, then the workgroup barrier) is the
  // rest of the release.  The ticket is an agent-scope atomic at that same
  // point, so it moves only after the winners are there.  On the other side
  // the merging workgroup reads the winners only with agent-scope atomic loads,
  // which are served at the coherence point and never from a stale cache line,
  // which is what the acquire's invalidation would otherwise ensure.
  // (Measured: the full release + acquire cost ~12 µs per launch here.)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    sh.ticket = __hip_atomic_fetch_add(&counters[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sh.ticket != uint32_t(nsplit - 1)) return;
  // the last ticket: every chunk's winners are published; reset the counter
  // for the next call and merge
  if (threadIdx.x == 0) __hip_atomic_store(&counters[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (ex.token_ids) expand_pad<NT>(row, K, ex);
  if (m < K && merge_heads<NT, KPTH>(sh, row, nsplit, m, K, keys, pool_ids, exr)) return;
  __syncthreads();
  topk_block<NT, KPT2, false, true>(sh, row, 0, 1, nullptr, keys, P, 0, nsplit, K, nullptr, pool_ids, exr);
}

struct TkPlan {
  int nsplit;  // chunks per row (1: single launch)
  int chunk;   // pools per chunk
  int nt1, kpt1;  // first launch: threads and keys per thread
  int nt2, kpt2;  // merge launch
  bool fused;     // split rows in one launch (512 threads, 8 keys per thread per chunk)
  int kpt_m;      // fused: merge keys per thread (full lists)
  int head;       // fused: keys taken first from the head of each sorted winner list
  int kpt_h;      // fused: keys per thread of that first merge
};

constexpr int kFusedThreads = 512;
constexpr int kFusedKpt = 8;  // chunk keys per thread in the fused launch (chunks <= 4096)

static int pow2_at_least(long v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// threads and keys per thread for n keys: 256 threads for up to 2K keys, 512
// up to 4K, else 1024 (more waves shorten each pass's instruction stream)
static void tk_shape(long n, int& nt, int& kpt) {
  nt = n <= 2048 ? 256 : (n <= 4096 ? 512 : 1024);
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
  pl.fused = false;
  pl.kpt_m = 0;
  if (nsplit > 1) {
    tk_shape(long(nsplit) * K, pl.nt2, pl.kpt2);
    const long merge = long(nsplit) * K;
    if (pl.chunk <= kFusedThreads * kFusedKpt && merge <= kFusedThreads * 32) {
      pl.fused = true;
      pl.kpt_m = pow2_at_least((merge + kFusedThreads - 1) / kFusedThreads);
      if (pl.kpt_m < 2) pl.kpt_m = 2;
      // twice a list's expected share of the K winners, at least 32
      int head = pow2_at_least((2L * K + nsplit - 1) / nsplit);
      if (head < 32) head = 32;
      pl.head = head < K ? head : K;
      pl.kpt_h = pow2_at_least((long(nsplit) * pl.head + kFusedThreads - 1) / kFusedThreads);
      if (pl.kpt_h < 2) pl.kpt_h = 2;
      if (pl.kpt_h > 4) pl.head = K;  // heads of more than 2048 keys: merge the full lists
    }
  }
  return pl;
}

// workspace: a block of merge counters of fixed size (one per row, for every
// Q the entry point accepts, so that the block sits at the same place for
// every shape), then the chunk winner lists
static_assert(DSA_TOPK_COUNTER_BYTES >= 65535 * sizeof(uint32_t), "one counter per row");

template <int NT, bool FROM_SCORES, bool FINAL>
static void launch_tk(int kpt, dim3 grid, hipStream_t s, const float* scores, const uint64_t* keys_in,
                      int P, int chunk, int nsplit_in, int K, uint64_t* keys_out, int32_t* pool_ids,
                      const ExpandArgs& ex, const uint32_t* lcounts, int lcap) {
#define DSA_TK(KPT)                                                                                \
  hipLaunchKernelGGL((topk_kernel<NT, KPT, FROM_SCORES, FINAL>), grid, dim3(NT), 0, s, scores,    \
                     keys_in, P, chunk, nsplit_in, K, keys_out, pool_ids, ex, lcounts, lcap)
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

template <bool FROM_SCORES, bool FINAL>
static void launch_tk_nt(int nt, int kpt, dim3 grid, hipStream_t s, const float* scores,
                         const uint64_t* keys_in, int P, int chunk, int nsplit_in, int K,
                         uint64_t* keys_out, int32_t* pool_ids, const ExpandArgs& ex,
                         const uint32_t* lcounts = nullptr, int lcap = 0) {
  if (nt == 256)
    launch_tk<256, FROM_SCORES, FINAL>(kpt, grid, s, scores, keys_in, P, chunk, nsplit_in, K, keys_out, pool_ids, ex,
                                       lcounts, lcap);
  else if (nt == 512)
    launch_tk<512, FROM_SCORES, FINAL>(kpt, grid, s, scores, keys_in, P, chunk, nsplit_in, K, keys_out, pool_ids, ex,
                                       lcounts, lcap);
  else
    launch_tk<1024, FROM_SCORES, FINAL>(kpt, grid, s, scores, keys_in, P, chunk, nsplit_in, K, keys_out, pool_ids, ex,
                                        lcounts, lcap);
}

// The row's K largest keys from the candidate lists of the filtering score
// pass (nseg lists of cap keys per row), sorted to pool ids and expanded.
int topk_lists(const uint64_t* keys, const uint32_t* counts, int nseg, int cap, int Q, int P_max, int K,
               int32_t* pool_ids, const int32_t* row_seq, const int32_t* pool_start, int B, int kpool,
               int32_t* token_ids, int W, hipStream_t s) {
  const ExpandArgs ex{row_seq, pool_start, B, P_max, kpool, token_ids, W};
  // 512 threads up to 4096 slots (measured on 4096 rows of 2048-key lists:
  // 512 x 4 beat 256 x 8 and 1024 x 2), then 1024
  const long n = long(nseg) * cap;
  const int nt = n <= 4096 ? 512 : 1024;
  const int kpt = pow2_at_least((n + nt - 1) / nt);
  if (kpt > 32 || Q > 65535) return DSA_ERR_UNSUPPORTED;
  launch_tk_nt<false, true>(nt, kpt, dim3(1, Q), s, nullptr, keys, P_max, 0, nseg, K, nullptr, pool_ids, ex, counts,
                            cap);
  return launch_status();
}

}  // namespace dsa

using namespace dsa;

// zero-fills the counter block of a top-k workspace (a plain fill kernel, so
// that the call can sit in a captured HIP graph)
__global__ __launch_bounds__(256) void topk_counter_fill(uint32_t* __restrict__ counters, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) counters[i] = 0u;
}

extern "C" int dsa_topk_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return DSA_ERR_NULL;
  const size_t n = (workspace_bytes < DSA_TOPK_COUNTER_BYTES ? workspace_bytes : DSA_TOPK_COUNTER_BYTES) / 4;
  if (n == 0) return DSA_OK;
  hipLaunchKernelGGL(topk_counter_fill, dim3(64), dim3(256), 0, as_stream(stream), static_cast<uint32_t*>(workspace),
                     int(n));
  return launch_status();
}

extern "C" size_t dsa_topk_workspace_bytes(int Q, int P, int K) {
  if (Q <= 0 || P <= 0 || K <= 0) return 0;
  const TkPlan pl = tk_plan(Q, P, K);
  return pl.nsplit > 1 ? DSA_TOPK_COUNTER_BYTES + size_t(Q) * pl.nsplit * K * sizeof(uint64_t) : 0;
}

// The selection launches shared by dsa_topk_pools and dsa_topk_pools_expand
// (ex.token_ids == nullptr: selection only).
static int topk_run(const float* scores, int Q, int P, int K, int32_t* pool_ids, void* workspace,
                    size_t workspace_bytes, hipStream_t s, const ExpandArgs& ex) {
  if (!scores || !pool_ids) return DSA_ERR_NULL;
  if (Q <= 0 || P <= 0 || K <= 0) return DSA_ERR_SHAPE;
  if (K > DSA_MAX_SELECT_K) return DSA_ERR_UNSUPPORTED;
  if (long(P) > long(kTkMaxChunk) * kTkMaxSplit) return DSA_ERR_UNSUPPORTED;
  if (Q > 65535) return DSA_ERR_UNSUPPORTED;
  const TkPlan pl = tk_plan(Q, P, K);
  if (pl.nsplit > kTkMaxSplit || pl.kpt1 > 32 || pl.kpt2 > 32) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_topk_workspace_bytes(Q, P, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  dim3 g1(pl.nsplit, Q);
  if (pl.nsplit == 1) {
    launch_tk_nt<true, true>(pl.nt1, pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, nullptr, pool_ids, ex);
    return launch_status();
  }
  uint32_t* counters = static_cast<uint32_t*>(workspace);
  uint64_t* ws = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + DSA_TOPK_COUNTER_BYTES);
  if (pl.fused) {
#define DSA_TKF(KH, KM)                                                                                  \
  hipLaunchKernelGGL((topk_split_kernel<kFusedThreads, kFusedKpt, KH, KM>), g1, dim3(kFusedThreads), 0, s, \
                     scores, P, pl.chunk, pl.nsplit, K, pl.head, ws, counters, pool_ids, ex)
#define DSA_TKF_H(KM)       \
  if (pl.kpt_h <= 2)        \
    DSA_TKF(2, KM);         \
  else                      \
    DSA_TKF(4, KM)
    switch (pl.kpt_m) {
      case 2: DSA_TKF_H(2); break;
      case 4: DSA_TKF_H(4); break;
      case 8: DSA_TKF_H(8); break;
      case 16: DSA_TKF_H(16); break;
      default: DSA_TKF_H(32); break;
    }
#undef DSA_TKF_H
#undef DSA_TKF
    return launch_status();
  }
  const ExpandArgs none{};
  launch_tk_nt<true, false>(pl.nt1, pl.kpt1, g1, s, scores, nullptr, P, pl.chunk, 0, K, ws, nullptr, none);
  int st = launch_status();
  if (st) return st;
  dim3 g2(1, Q);
  launch_tk_nt<false, true>(pl.nt2, pl.kpt2, g2, s, nullptr, ws, P, 0, pl.nsplit, K, nullptr, pool_ids, ex);
  return launch_status();
}

extern "C" int dsa_topk_pools(const float* scores, int Q, int P, int K, int32_t* pool_ids,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return topk_run(scores, Q, P, K, pool_ids, workspace, workspace_bytes, as_stream(stream), ExpandArgs{});
}

extern "C" int dsa_topk_pools_expand(const float* scores, int Q, int P, int K, int32_t* pool_ids,
                                     const int32_t* row_seq, const int32_t* pool_start, int B, int P_max,
                                     int kpool, int32_t* token_ids, int W, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!row_seq || !pool_start || !token_ids) return DSA_ERR_NULL;
  if (B <= 0 || P_max <= 0 || kpool <= 0 || W <= 0) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL) return DSA_ERR_UNSUPPORTED;
  if (K > 0 && long(W) < long(K) * kpool) return DSA_ERR_SHAPE;
  const ExpandArgs ex{row_seq, pool_start, B, P_max, kpool, token_ids, W};
  return topk_run(scores, Q, P, K, pool_ids, workspace, workspace_bytes, as_stream(stream), ex);
}
