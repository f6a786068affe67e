// Selection keys and wave-level helpers shared by the top-k kernels and the
// score kernel's candidate filter (page "Module tp", "Why the indexer is
// REPLICATED, not sharded": higher score first, then the smaller pool index).
//
// A candidate pool is the 64-bit key (hi << 32 | lo): hi maps the fp32 score
// to a nonzero u32 with the same order (-0 folded onto +0; 0 marks a
// non-candidate), lo = 0xffffffff - pool index.  A larger key comes earlier in
// the output, and a row's keys are distinct.
#pragma once

#include "dsa_common.hpp"

namespace dsa {

// Order-preserving map of a score to a nonzero u32; 0 for a non-candidate
// (-inf, and NaN, which the interface excludes).
// Written with selects only, so that a loop of them stays branch-free.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u << 1) == 0u ? 0u : u;  // -0 -> +0
  const uint32_t k = int32_t(u) < 0 ? ~u : (u | 0x80000000u);
  return f > -INFINITY ? k : 0u;
}

// The score a key stands for (inverse of score_key for candidates).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float(int32_t(k) < 0 ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- wave helpers
// v from lane (lane - n) of the same row of 16 lanes, 0 for the first n lanes
template <int N>
__device__ __forceinline__ uint32_t row_shr(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x110 + N, 0xF, 0xF, true));
}

// inclusive prefix sum over the wave: DPP shifts within rows of 16, then the
// row broadcasts (lane 15 of a row into the next row, lane 31 into rows 2, 3)
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// maximum over the wave (wave-uniform result)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, row_shr<1>(v));
  v = max(v, row_shr<2>(v));
  v = max(v, row_shr<4>(v));
  v = max(v, row_shr<8>(v));
  return max(max(uint32_t(__builtin_amdgcn_readlane(v, 15)), uint32_t(__builtin_amdgcn_readlane(v, 31))),
             max(uint32_t(__builtin_amdgcn_readlane(v, 47)), uint32_t(__builtin_amdgcn_readlane(v, 63))));
}

// bitwise OR over the wave (wave-uniform result)
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v |= row_shr<1>(v);
  v |= row_shr<2>(v);
  v |= row_shr<4>(v);
  v |= row_shr<8>(v);
  return (uint32_t(__builtin_amdgcn_readlane(v, 15)) | uint32_t(__builtin_amdgcn_readlane(v, 31))) |
         (uint32_t(__builtin_amdgcn_readlane(v, 47)) | uint32_t(__builtin_amdgcn_readlane(v, 63)));
}

// number of set bits of m below this lane
__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// ------------------------------------------------- per-wave candidate lists
// A wave that produces the keys of one row over a range of pools keeps a
// list of them in global memory, buf[0, n), with a key threshold thr: a key
// below thr is left out.  Exactness: thr only ever takes values below which
// at least K keys of the range already seen lie at or above it, so a key
// below thr has K larger keys in the row and is not among the row's K
// largest; every key of the row's top K therefore ends up in the list.
//
// A list is written and read back only by the wave that owns it, and read
// after a wait for that wave's own stores: workgroup-scope loads (the
// workgroup's waves share one CU and its write-through L1) are coherent with
// those stores and may be served by the XCD's L2.  (Agent-scope loads, served
// at the device's coherence point, made the filtering score kernel 1.5 %
// slower at the prefill chunk.)
__device__ __forceinline__ uint64_t list_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

constexpr int kListChunk = 16;  // keys per lane per read round of a list

// Shrinks the list buf[0, n) (n > K) to its keys at or above a new threshold,
// which it returns: a radix select over 8-bit digits of the keys, starting
// below the bits that every listed key shares, that stops at the first digit
// where the keys at or above the threshold number at most `target` (exactly
// K when it reaches the last bit, as the keys are distinct).  The kept keys
// stay in list order.  hist: this wave's 256 LDS counters.  Wave-uniform
// control flow; every lane returns the same threshold and n.
__device__ __forceinline__ uint64_t list_compact(uint64_t* buf, uint32_t& n, uint32_t K, uint32_t target,
                                              uint32_t* hist, uint64_t& lor, uint64_t& land) {
  const int lane = threadIdx.x & 63;
  const uint32_t cnt_in = n;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's appends have left it
  // bits shared by every listed key: the OR and AND of the lanes' running
  // OR / AND of the keys they listed
  const uint64_t kor = (uint64_t(wave_or_u32(uint32_t(lor >> 32))) << 32) | wave_or_u32(uint32_t(lor));
  const uint64_t kand = ~((uint64_t(wave_or_u32(~uint32_t(land >> 32))) << 32) | wave_or_u32(~uint32_t(land)));
  int h = 63 - __builtin_clzll(kor ^ kand);  // keys are distinct and n >= 2: some bit differs
  uint64_t pre = h >= 63 ? 0ull : (kor & ~((2ull << h) - 1ull));
  uint32_t need = K, above_tot = 0;
  while (true) {
    const int lo = h >= 7 ? h - 7 : 0;
    const uint64_t hmask = h >= 63 ? 0ull : (~0ull << (h + 1));
    const uint64_t want = pre & hmask;
    const uint32_t dmask = (2u << (h - lo)) - 1u;
    *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (uint32_t c0 = 0; c0 < cnt_in; c0 += 64 * kListChunk) {
      uint64_t k[kListChunk];
#pragma unroll
      for (int j = 0; j < kListChunk; ++j) {
        const uint32_t i = c0 + j * 64 + lane;
        k[j] = i < cnt_in ? list_load(buf + i) : 0ull;
      }
#pragma unroll
      for (int j = 0; j < kListChunk; ++j)
        if (c0 + j * 64 + lane < cnt_in && (k[j] & hmask) == want)
          atomicAdd(&hist[uint32_t(k[j] >> lo) & dmask], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // the digit whose count from the top reaches `need`: lane l holds digits
    // 4l .. 4l+3, and the count of digits >= 4l is non-increasing in l
    const u32x4 cv = *reinterpret_cast<const u32x4*>(hist + 4 * lane);
    const uint32_t tot = (cv[0] + cv[1]) + (cv[2] + cv[3]);
    const uint32_t incl = wave_incl_sum(tot);
    const uint32_t above_l = __builtin_amdgcn_readlane(incl, 63) - incl;
    const uint64_t b = __ballot(above_l + tot >= need);
    const int L = 63 - __builtin_clzll(b);
    uint32_t run = __builtin_amdgcn_readlane(above_l, L);
    const uint32_t c3 = __builtin_amdgcn_readlane(cv[3], L), c2 = __builtin_amdgcn_readlane(cv[2], L);
    const uint32_t c1 = __builtin_amdgcn_readlane(cv[1], L), c0v = __builtin_amdgcn_readlane(cv[0], L);
    uint32_t d, above, cnt;
    if (run + c3 >= need) {
      d = 4 * L + 3; above = run; cnt = c3;
    } else if (run + c3 + c2 >= need) {
      d = 4 * L + 2; above = run + c3; cnt = c2;
    } else if (run + c3 + c2 + c1 >= need) {
      d = 4 * L + 1; above = run + c3 + c2; cnt = c1;
    } else {
      d = 4 * L; above = run + c3 + c2 + c1; cnt = c0v;
    }
    pre = want | (uint64_t(d) << lo);
    if (above_tot + above + cnt <= target || lo == 0) break;
    above_tot += above;
    need -= above;
    h = lo - 1;
  }
  // keep the keys >= pre (pre's bits below the last digit are zero), in order:
  // a read round has landed completely before its kept keys are written, and
  // they go to slots at or before their old ones, never into a later round's
  uint32_t w = 0;
  lor = 0ull;
  land = ~0ull;
  for (uint32_t c0 = 0; c0 < cnt_in; c0 += 64 * kListChunk) {
    uint64_t k[kListChunk];
#pragma unroll
    for (int j = 0; j < kListChunk; ++j) {
      const uint32_t i = c0 + j * 64 + lane;
      k[j] = i < cnt_in ? list_load(buf + i) : 0ull;
    }
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int j = 0; j < kListChunk; ++j) {
      const bool keep = c0 + j * 64 + lane < cnt_in && k[j] >= pre;
      const uint64_t m = __ballot(keep);
      if (keep) {
        buf[w + lane_rank(m)] = k[j];
        lor |= k[j];
        land &= k[j];
      }
      w += uint32_t(__builtin_popcountll(m));
    }
  }
  n = w;
  return pre;
}

}  // namespace dsa
