// index_scores: indexer scores with candidate validity (page "Module
// glm5next_dsa", "Shape of the pipeline" and "Traps carried from Slice 8":
// k_norm is a LayerNorm with bias; page "Module tp", "Why the indexer is
// REPLICATED, not sharded": score = sum over heads of w[h]*relu(scale*dot)).
//
// MFMA path (bf16, D = 128, H in {16, 32}).  The LayerNorm is folded into the
// contraction.  With x a pooled key, mu / r its mean / inverse std,
// g[h,c] = q[h,c]*gamma[c] and g'[h,c] = g[h,c] - mean_c g[h,c],
//     <q_h, LN(x)> = r * sum_c g'[h,c] x_c + sum_c q[h,c] beta[c]
// (the centring of g' removes the mean of x exactly).  sum_c g'[h,c] x_c runs
// on the matrix cores, heads as M and pools as N: x is exact bf16 and g' is an
// unevaluated pair g'_hi + g'_lo of bf16 values (|g' - g'_hi - g'_lo| ~ 2^-17
// |g'|), both accumulated into one fp32 accumulator.  The LayerNorm statistics
// come from the matrix cores too: a ones operand gives sum_c x_c, and the
// 16x16 Gram block of a tile with itself has sum_c x_c^2 on its diagonal, so
// the vector ALUs only finish r, apply relu/w and reduce the heads.  The normed
// key is never rounded.
//
// Lane l of a wave holds pool (l & 15) of a 16-pool tile and channels
// 8*(kg + 4i) .. +8, kg = l >> 4, for k-step i (one 16-byte load each; in the
// tile-interleaved pool cache the 64 lanes' loads of one k-step are 1 KiB of
// contiguous memory); the MFMA output puts heads 4*kg + j (j < 4) of that pool
// in the lane.
//
// Decode kernel: one row per grid row, pools split over grid.x, each wave
// streaming its tiles through a register ring.  Prefill kernel: a workgroup
// holds 8 rows' operands in registers and streams a range of tiles through
// LDS.  Both use the same operand layout, statistics, accumulation order and
// epilogue, so a row's scores are bit-identical whichever kernel computes
// them.
//
// Per pool the decode kernel reads 256 B of key + 1 B valid and writes 4 B of
// score (the pool's start follows from the sequence's first start): it is
// HBM-bound.
#include <climits>

#include "dsa_common.hpp"
#include "dsa_host.hpp"
#include "dsa_select.hpp"

namespace dsa {

constexpr int kIsThreads = 256;
constexpr int kIsWaves = kIsThreads / kWave;
constexpr int kIsD = 128;
constexpr int kIsLd = kIsD + 8;  // padded LDS row: 16 lanes reading 16 rows hit distinct banks

// Stage one row's g' = q*gamma - mean(q*gamma) as (hi, lo) bf16 pairs, the
// bias term QB = sum_c q*beta and the head weights.  8 threads per head, 16
// channels each: u in [0, 8H) gives head u / 8, channels 16*(u % 8) .. +16.
// Callers pass u for whole waves (the shuffles stay inside 8-lane groups).
// Split in a load half and a compute half so that callers can issue other
// loads in between.
struct RowIn {
  u32x4 q[2];
  f32x4 g[4], b[4];
  float w;
};

__device__ __forceinline__ RowIn stage_row_load(const uint16_t* __restrict__ q_row,
                                                const float* __restrict__ w_row,
                                                const float* __restrict__ gamma,
                                                const float* __restrict__ beta, int u) {
  const int h = u >> 3, c0 = (u & 7) * 16;
  RowIn in;
  in.w = w_row[h];
#pragma unroll
  for (int z = 0; z < 2; ++z) in.q[z] = *reinterpret_cast<const u32x4*>(q_row + h * kIsD + c0 + 8 * z);
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    in.g[z] = *reinterpret_cast<const f32x4*>(gamma + c0 + 4 * z);
    in.b[z] = *reinterpret_cast<const f32x4*>(beta + c0 + 4 * z);
  }
  return in;
}

__device__ __forceinline__ void stage_row_store(const RowIn& in, uint16_t (*ghi)[kIsLd], uint16_t (*glo)[kIsLd],
                                                float* QB, float* Wsh, int u) {
  const int h = u >> 3, part = u & 7, c0 = part * 16;
  float g[16];
  float qbs = 0.f, gs = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t word = in.q[e >> 3][(e & 7) >> 1];
    const float qv = (e & 1) ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
    g[e] = qv * in.g[e >> 2][e & 3];
    gs += g[e];
    qbs = fmaf(qv, in.b[e >> 2][e & 3], qbs);
  }
  gs += __shfl_xor(gs, 1, kWave);
  gs += __shfl_xor(gs, 2, kWave);
  gs += __shfl_xor(gs, 4, kWave);
  qbs += __shfl_xor(qbs, 1, kWave);
  qbs += __shfl_xor(qbs, 2, kWave);
  qbs += __shfl_xor(qbs, 4, kWave);
  const float mean = gs * (1.0f / kIsD);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float gc = g[half * 8 + 2 * e + z] - mean;
        const uint16_t hi = f2bf(gc);
        hw[z] = hi;
        lw[z] = f2bf(gc - bf2f(hi));
      }
      ph[e] = hw[0] | (hw[1] << 16);
      pl[e] = lw[0] | (lw[1] << 16);
    }
    *reinterpret_cast<u32x4*>(&ghi[h][c0 + half * 8]) = ph;
    *reinterpret_cast<u32x4*>(&glo[h][c0 + half * 8]) = pl;
  }
  if (part == 0) {
    QB[h] = qbs;
    Wsh[h] = in.w;
  }
}

// Sum of v over the four lanes (kg, ln), kg = 0..3, in every lane: the lane
// swaps of 16- and 32-lane rows (same register as both operands: the two
// results hold the value of the partner rows), no LDS.
__device__ __forceinline__ float sum_lane_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A tile's contribution is split in a matrix-core half (tile_mfma: LayerNorm
// statistics and the folded head dots) and a vector half (tile_epilogue: relu,
// head weights and the sum over the lane's heads and the wave's four lane
// groups), so that the decode loop can issue the next tile's MFMAs before the
// current tile's epilogue.
//
// The matrix-core half: folded head dots, sum_c x_c (ones operand) and the
// Gram block <x_m, x_n>.
template <int NH>
struct TileAcc {
  f32x4 acc[NH], sacc, gacc;
};

template <int NH>
__device__ __forceinline__ TileAcc<NH> tile_mfma(const u32x4 (&x)[4], const bf16x8 (&ahi)[NH][4],
                                                 const bf16x8 (&alo)[NH][4]) {
  const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  TileAcc<NH> t;
#pragma unroll
  for (int mb = 0; mb < NH; ++mb) t.acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  t.sacc = f32x4{0.f, 0.f, 0.f, 0.f};
  t.gacc = f32x4{0.f, 0.f, 0.f, 0.f};
  // in each k-step the two products that accumulate into one head block are
  // separated by other MFMAs (measured faster than issuing them back to back)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8 bx = as_bf16x8(x[i]);
#pragma unroll
    for (int mb = 0; mb < NH; ++mb) t.acc[mb] = mfma16x16x32(ahi[mb][i], bx, t.acc[mb]);
    t.sacc = mfma16x16x32(ones, bx, t.sacc);  // every row: sum_c x_c of pool (lane & 15)
#pragma unroll
    for (int mb = 0; mb < NH; ++mb) t.acc[mb] = mfma16x16x32(alo[mb][i], bx, t.acc[mb]);
    t.gacc = mfma16x16x32(bx, bx, t.gacc);    // Gram block: <x_m, x_n>
  }
  return t;
}

// The folded head dots of a tile with the head blocks' products interleaved
// (per accumulator the order is that of tile_mfma: hi, then lo, per k-step).
template <int NH>
__device__ __forceinline__ void head_mfma_i(const u32x4 (&x)[4], const bf16x8 (&ahi)[NH][4],
                                            const bf16x8 (&alo)[NH][4], f32x4 (&acc)[NH]) {
#pragma unroll
  for (int mb = 0; mb < NH; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x8 bx = as_bf16x8(x[i]);
#pragma unroll
    for (int mb = 0; mb < NH; ++mb) acc[mb] = mfma16x16x32(ahi[mb][i], bx, acc[mb]);
#pragma unroll
    for (int mb = 0; mb < NH; ++mb) acc[mb] = mfma16x16x32(alo[mb][i], bx, acc[mb]);
  }
}

// The vector half: LayerNorm statistics, relu, head weights and the sum over
// the lane's heads and the wave's four lane groups.  Returns the score of pool
// (lane & 15) in all lanes.  cQs = scale * QB, so scale * (r * dot + QB) =
// (scale * r) * dot + cQs (relu is applied to the product, so the sign of
// scale does not matter).  diag_addr is the ds_bpermute byte address of the
// lane holding the Gram diagonal of pool (lane & 15):
// 4 * (16 * ((lane & 15) >> 2) + (lane & 15)).
template <int NH>
__device__ __forceinline__ float tile_epilogue(const TileAcc<NH>& t, const float (&cQs)[NH][4],
                                               const float (&cW)[NH][4], float scale, float eps, int ln,
                                               int diag_addr) {
  const f32x4 (&acc)[NH] = t.acc;
  const f32x4 sacc = t.sacc, gacc = t.gacc;
  // diagonal <x_n, x_n> sits in lane 16*(n >> 2) + n, register n & 3 (a
  // branch-free pick of register ln & 3, then one lane permute)
  const int jd = ln & 3;
  float dg = gacc[0];
  dg = jd == 1 ? gacc[1] : dg;
  dg = jd == 2 ? gacc[2] : dg;
  dg = jd == 3 ? gacc[3] : dg;
  const float sumsq = __int_as_float(__builtin_amdgcn_ds_bpermute(diag_addr, __float_as_int(dg)));
  const float mu = sacc[0] * (1.0f / kIsD);
  const float var = fmaxf(sumsq * (1.0f / kIsD) - mu * mu, 0.f);
  const float rs = scale * __builtin_amdgcn_rsqf(var + eps);  // v_rsq_f32: 1 ulp
  float part = 0.f;
#pragma unroll
  for (int mb = 0; mb < NH; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) part = fmaf(cW[mb][j], fmaxf(0.f, fmaf(rs, acc[mb][j], cQs[mb][j])), part);
  return sum_lane_groups(part);
}

// A lane's operands for the head MFMAs and the epilogue: g' hi/lo of its 16-head blocks, scale * QB
// and w of the heads whose results it receives.
template <int NH>
__device__ __forceinline__ void load_operands(const uint16_t (*ghi)[kIsLd], const uint16_t (*glo)[kIsLd],
                                              const float* QB, const float* Wsh, int kg, int ln, float scale,
                                              bf16x8 (&ahi)[NH][4], bf16x8 (&alo)[NH][4],
                                              float (&cQs)[NH][4], float (&cW)[NH][4]) {
#pragma unroll
  for (int mb = 0; mb < NH; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ahi[mb][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&ghi[mb * 16 + ln][(kg + 4 * i) * 8]));
      alo[mb][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&glo[mb * 16 + ln][(kg + 4 * i) * 8]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cQs[mb][j] = scale * QB[mb * 16 + 4 * kg + j];
      cW[mb][j] = Wsh[mb * 16 + 4 * kg + j];
    }
  }
}

// Decode kernel.  A workgroup owns 4*NT 16-pool tiles of one row, taken in
// blocks of PW = min(NT, 2) consecutive tiles per wave: in block b the row's
// workgroups cover one contiguous stretch of the pool cache together (wave w
// of workgroup g reads tiles b*G*4*PW + g*4*PW + PW*w ..), so the requests in
// flight at any time fall in a window that moves through the cache rather
// than in 4*G separate stretches (measured faster, as the plain read stream
// is faster with short per-wave stretches).  Each wave runs through its tiles
// with a kStreamRing-deep register ring: a ring slot is refilled right after
// the MFMAs that read it are issued, and scheduling barriers keep the
// compiler from sinking those loads below the epilogue (it otherwise issues
// several tiles' MFMAs first and the last loads only after all earlier ones
// have landed).  In the tile-interleaved pool cache each of a tile's 4 key
// loads per lane covers 1 KiB of contiguous memory and lands directly in the
// matrix-core operand layout; keys are read non-temporally (each byte is
// used once).  The row's folded LayerNorm operands are staged once in LDS (8
// threads per head) while the first ring of keys is in flight.  The scores
// are gathered in LDS and written at the end with coalesced stores (stores
// interleaved with the key stream measured slower); the candidate test is
// applied there, from pool_valid loaded at the start.
constexpr int kStreamRing = 2;           // tiles in flight per wave
constexpr int kTileElems = 16 * kIsD;    // 4 KiB of bf16 keys

__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int NH, int NT>
__global__ __launch_bounds__(kIsThreads) __attribute__((amdgpu_waves_per_eu(2))) void index_scores_stream(
    const uint16_t* __restrict__ q, const float* __restrict__ w, float scale,
    const uint16_t* __restrict__ k_pool, const int32_t* __restrict__ pool_start,
    const uint8_t* __restrict__ pool_valid, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int B, int P_max, int kp, float* __restrict__ scores) {
  constexpr int H = NH * 16;
  constexpr int kPools = kIsWaves * NT * 16;  // pools per workgroup
  constexpr int R = NT < kStreamRing ? NT : kStreamRing;
  constexpr int PW = NT < 2 ? NT : 2;         // consecutive tiles per wave and block
  constexpr int MP = (kPools + kIsThreads - 1) / kIsThreads;  // metadata entries per thread
  static_assert(NT % R == 0 && NT % PW == 0, "the ring and the blocks divide the wave's tiles");
  __shared__ uint16_t ghi[H][kIsLd];
  __shared__ uint16_t glo[H][kIsLd];
  __shared__ float sQB[H], sW[H];
  __shared__ float sOut[kPools];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, ln = lane & 15;
  const int diag_addr = 4 * (16 * (ln >> 2) + ln);
  const int r = blockIdx.y;
  const int b = row_seq[r];
  const int pos = row_pos[r];
  const bool ok = b >= 0 && b < B;
  const int P_tiles = pool_tiles(P_max);
  const int G = gridDim.x;  // workgroups per row
  // tile of the wave's j-th tile (see above)
  auto tile_of = [&](int wv, int j) {
    return (j / PW) * (G * kIsWaves * PW) + int(blockIdx.x) * (kIsWaves * PW) + PW * wv + (j % PW);
  };
  // store slot e (< kPools) of the workgroup: in block e / (64 PW), the
  // (e % (64 PW))-th of its 64 PW contiguous pools; -> (LDS index, pool)
  auto slot = [&](int e, int& lp) {
    const int bl = e / (64 * PW), k = (e % (64 * PW)) >> 4;
    const int wv = k / PW, j = bl * PW + k % PW;
    lp = (wv * NT + j) * 16 + (e & 15);
    return tile_of(wv, j) * 16 + (e & 15);
  };
  const size_t seq0 = size_t(ok ? b : 0) * P_max;
  const uint16_t* kseq = k_pool + size_t(ok ? b : 0) * P_tiles * kTileElems;

  // operand loads first, then the validity of the pools this thread stores
  // (used only at the end), then the first ring of key tiles.  A pool's start
  // is the sequence's first start plus p * kpool (pool p begins kpool * p
  // tokens after the anchor), so one start per sequence is read instead of
  // one per pool.
  RowIn rin;
  if (tid < H * 8) rin = stage_row_load(q + size_t(r) * H * kIsD, w + size_t(r) * H, gamma, beta, tid);
  const int start0 = pool_start[seq0];
  uint8_t vl[MP];
#pragma unroll
  for (int u = 0; u < MP; ++u) {
    const int e = u * kIsThreads + tid;
    int lp;
    const int p = slot(e, lp);
    const size_t pi = (ok && e < kPools && p < P_max) ? seq0 + p : 0;
    vl[u] = pool_valid[pi];
  }
  u32x4 xb[R][4];
  auto issue = [&](int rs, int j) {
    const int t = tile_of(wave, j);
    const bool in = j < NT && t < P_tiles;
    const uint16_t* src = kseq + size_t(in ? t : 0) * kTileElems + 8 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[rs][i] = ld_stream(src + 512 * i);
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < R; ++s) issue(s, s);
  // keep the key stream's first loads ahead of the operand arithmetic (the
  // scheduler would otherwise sink them below it to save registers, and the
  // whole grid would wait for its operands before any key is requested)
  __builtin_amdgcn_sched_barrier(0);
  if (tid < H * 8) stage_row_store(rin, ghi, glo, sQB, sW, tid);
  __syncthreads();
  bf16x8 ahi[NH][4], alo[NH][4];
  float cQ[NH][4], cW[NH][4];
  load_operands<NH>(ghi, glo, sQB, sW, kg, ln, scale, ahi, alo, cQ, cW);
  // software pipeline: tile j+1's matrix-core work is issued before tile j's
  // vector epilogue, which then runs while the matrix cores are busy; a ring
  // slot is refilled as soon as its tile's MFMAs are issued, and the
  // scheduling barriers keep each phase in that order
  TileAcc<NH> cur = tile_mfma<NH>(xb[0], ahi, alo);
  if (R < NT) issue(0, R);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j0 = 0; j0 < NT; j0 += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int j = j0 + s;
      TileAcc<NH> nxt;
      if (j + 1 < NT) {
        const int s1 = (s + 1) % R;
        nxt = tile_mfma<NH>(xb[s1], ahi, alo);
        if (j + 1 + R < NT) issue(s1, j + 1 + R);  // resolved at compile time (unrolled)
      }
      __builtin_amdgcn_sched_barrier(0);
      const float sc = tile_epilogue<NH>(cur, cQ, cW, scale, eps, ln, diag_addr);
      // the four lane groups hold the same sum: all write it (no branch)
      sOut[(wave * NT + j) * 16 + ln] = sc;
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < NT) cur = nxt;
    }
  }
  __syncthreads();
  // candidate test (valid pool whose last token is at or before the row's
  // position: start0 + p * kpool + kpool - 1 <= pos, in 64-bit so that no
  // position overflows) and coalesced stores
  const long last_ok = long(pos) - (kp - 1) - start0;
  float* srow = scores + size_t(r) * P_max;
#pragma unroll
  for (int u = 0; u < MP; ++u) {
    const int e = u * kIsThreads + tid;
    int lp;
    const int p = slot(e, lp);
    if (e < kPools && p < P_max)
      srow[p] = (ok && vl[u] != 0 && long(p) * kp <= last_ok) ? sOut[lp] : -INFINITY;
  }
}

// Many rows, GEMM-shaped (prefill chunks).  A workgroup of 8 waves takes 8
// rows (one per wave) and a range of pool tiles.  The rows' folded operands
// are staged once (the decode kernel's staging arithmetic, through LDS) and
// then held in each wave's registers for the whole range; the workgroup
// streams the range's key tiles through two LDS buffers, 16 tiles per stage
// (two loaded by each wave, which also forms those tiles' LayerNorm
// statistics, so every tile's statistics are formed once per workgroup),
// one barrier per stage: while a stage is computed, the next stage's tiles
// are in flight.  Each (row, tile) costs 16 MFMAs (hi/lo x head blocks x 4
// k-steps) and a short epilogue, the MFMAs of tile j+1 issued before the
// epilogue of tile j; lane (kg, ln) keeps tiles kg + 4u of a stage, so a
// stage's 256 scores of a row go out in four 256-byte stores.  Rows of
// several sequences in one workgroup take one pass per sequence.  (Measured
// on the 4096-row chunk: 1.61 ms; four waves with two rows each, and the
// 32x32x16 MFMA shape over pairs of tiles, were both slower.)
//
// With FILTER the scores are not stored: each wave keeps its row's candidate
// keys (the top-k order keys of score and pool index) over its workgroup's
// pool range in a list of fo.cap keys, leaving out the pools that score below
// its threshold (dsa_select.hpp: such a key has K larger keys in the row).
// The wave visits the stages of its range in a scrambled order (below), so
// that scores trending along the pool index fill the lists no faster than
// random ones.  A list that could not take the next stage is shrunk by a
// radix select that raises the threshold.  A wave whose list is full after a stage stamps that
// stage in LDS, and at the next stage every wave whose list holds more than
// the target shrinks it too, so that the shrinks overlap rather than each
// holding the workgroup at the stage barrier (measured on the prefill
// chunk's scores + top-k, same run: 1.89 -> 1.80 ms; a full list is shrunk
// on its own length, so the stamp decides only when the others shrink, never
// whether a full list does).  The list of row r and
// pool range x is fo.keys[(r * gridDim.x + x) * fo.cap ..], its length
// fo.counts[r * gridDim.x + x]; a top-k over the lists gives the row's K
// largest keys.  The scores themselves are those of the storing kernel, bit
// for bit.
constexpr int kGemmWaves = 8;
constexpr int kGemmStage = 16;  // tiles per stage (two per wave)

struct FilterOut {
  uint64_t* keys;    // [Q, ranges, cap] candidate keys
  uint32_t* counts;  // [Q, ranges] list lengths
  int cap;           // keys per list: >= K + 512 (room for one stage after a shrink)
  int K;             // keys the row's selection keeps
  int target;        // a shrink keeps at most this many keys (exactly K at the last bit)
};

template <int NH, bool FILTER>
__global__ __launch_bounds__(kGemmWaves * 64) void index_scores_gemm(
    const uint16_t* __restrict__ q, const float* __restrict__ w, float scale,
    const uint16_t* __restrict__ k_pool, const int32_t* __restrict__ pool_start,
    const uint8_t* __restrict__ pool_valid, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int Q, int B, int P_max, int kp, int tiles_per_wg,
    float* __restrict__ scores, FilterOut fo) {
  constexpr int H = NH * 16;
  constexpr size_t kStageBytes = 8 * H * kIsLd * 2 * 2 + 8 * H * 4 * 2;  // ghi + glo + QB + W of 8 rows
  constexpr size_t kKeyBytes = 2 * kGemmStage * kTileElems * 2;          // two stages of key tiles
  constexpr size_t kLds = kStageBytes > kKeyBytes ? kStageBytes : kKeyBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  __shared__ float srs[2][kGemmStage * 16];  // scale / sigma per pool of a stage
  __shared__ int sseq[kGemmWaves];
  __shared__ __attribute__((aligned(16))) uint32_t shist[FILTER ? kGemmWaves : 1][256];  // list shrinks
  __shared__ uint32_t sfull[2];  // FILTER: stamp (pass, stage) + 1 of the last stage that left a list full (by parity)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, ln = lane & 15;
  const int diag_addr = 4 * (16 * (ln >> 2) + ln);
  const int r0 = blockIdx.y * kGemmWaves;
  const int r = r0 + wave;
  const bool rok = r < Q;
  const int b_row = rok ? row_seq[r] : -1;
  const bool ok = rok && b_row >= 0 && b_row < B;
  const int pos = rok ? row_pos[r] : 0;
  const int P_tiles = pool_tiles(P_max);
  const int tb = blockIdx.x * tiles_per_wg;
  const int te = min(P_tiles, tb + tiles_per_wg);
  const int nstage = te > tb ? (te - tb + kGemmStage - 1) / kGemmStage : 0;

  // 1. the 8 rows' folded operands: staged in LDS with the decode kernel's
  // arithmetic, then each wave takes its row's fragments into registers
  {
    uint16_t (*ghi)[H][kIsLd] = reinterpret_cast<uint16_t (*)[H][kIsLd]>(lds);
    uint16_t (*glo)[H][kIsLd] = reinterpret_cast<uint16_t (*)[H][kIsLd]>(lds + 8 * H * kIsLd * 2);
    float (*sQB)[H] = reinterpret_cast<float (*)[H]>(lds + 8 * H * kIsLd * 4);
    float (*sW)[H] = reinterpret_cast<float (*)[H]>(lds + 8 * H * kIsLd * 4 + 8 * H * 4);
    const int nr = min(kGemmWaves, Q - r0);
    for (int u = tid; u < nr * H * 8; u += kGemmWaves * 64) {
      const int rr = u / (H * 8);
      const RowIn rin = stage_row_load(q + size_t(r0 + rr) * H * kIsD, w + size_t(r0 + rr) * H, gamma, beta,
                                       u - rr * H * 8);
      stage_row_store(rin, ghi[rr], glo[rr], sQB[rr], sW[rr], u - rr * H * 8);
    }
    if (lane == 0) sseq[wave] = ok ? b_row : -1;
    if (FILTER && tid == 0) sfull[0] = sfull[1] = 0u;
    __syncthreads();
  }
  bf16x8 ahi[NH][4], alo[NH][4];
  float cQ[NH][4], cW[NH][4];
  if (rok) {
    uint16_t (*ghi)[H][kIsLd] = reinterpret_cast<uint16_t (*)[H][kIsLd]>(lds);
    uint16_t (*glo)[H][kIsLd] = reinterpret_cast<uint16_t (*)[H][kIsLd]>(lds + 8 * H * kIsLd * 2);
    float (*sQB)[H] = reinterpret_cast<float (*)[H]>(lds + 8 * H * kIsLd * 4);
    float (*sW)[H] = reinterpret_cast<float (*)[H]>(lds + 8 * H * kIsLd * 4 + 8 * H * 4);
    load_operands<NH>(ghi[wave], glo[wave], sQB[wave], sW[wave], kg, ln, scale, ahi, alo, cQ, cW);
  }
  __syncthreads();  // the staging area is reused for the key tiles
  uint16_t (*skeys)[kGemmStage][kTileElems] = reinterpret_cast<uint16_t (*)[kGemmStage][kTileElems]>(lds);
  const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  // FILTER: this wave's candidate list (length, threshold)
  uint64_t* fbuf = FILTER && rok ? fo.keys + (size_t(r) * gridDim.x + blockIdx.x) * size_t(fo.cap) : nullptr;
  uint32_t fn = 0;
  uint64_t fthr = 0;
  float fthr_s = -INFINITY;       // the score of fthr's hi: hi >= fthr's hi exactly when the score is >= this
  uint32_t fthr_p = 0xffffffffu;  // at a score equal to fthr_s, the largest pool index whose key is >= fthr
  uint64_t flor = 0ull, fland = ~0ull;  // this lane's OR / AND of the keys it listed  // the score of fthr's hi: hi >= fthr's hi exactly when the score is >= this

  for (int i8 = 0; i8 < kGemmWaves; ++i8) {
    const int b = sseq[i8];
    bool first = b >= 0;
    for (int j = 0; j < i8; ++j) first = first && sseq[j] != b;
    if (!first) continue;  // uniform: every wave reads the same LDS words
    const bool mine = ok && b_row == b;
    const uint16_t* kseq = k_pool + size_t(b) * P_tiles * kTileElems;
    const int start0 = pool_start[size_t(b) * P_max];
    const long last_ok = long(pos) - (kp - 1) - start0;
    float* srow = FILTER ? nullptr : scores + size_t(r) * P_max;
    // this wave's tile of stage s: keys into registers (and the validity of
    // the pools this lane stores in stage s)
    constexpr int TW = kGemmStage / kGemmWaves;  // tiles per wave and stage
    constexpr int NU = kGemmStage / 4;           // scores per lane and stage
    u32x4 xk[TW][4];
    uint8_t vl[NU];
    // FILTER: the wave visits its range's stages in a scrambled order, stage
    // s -> block s * pstep mod nstage (pstep a prime that does not divide
    // nstage), so that scores trending along the pool index fill the lists no
    // faster than scores in random order; a block is still 16 contiguous
    // tiles, and every workgroup takes the same order.  The block of the next
    // stage is formed by one addition.
    int pstep = 1;
    if (FILTER) {
      pstep = 37;
      if (nstage % pstep == 0) pstep = 41;
      if (nstage % pstep == 0) pstep = 43;
      pstep %= nstage > 0 ? nstage : 1;
    }
    auto next_blk = [&](int b) { b += pstep; return b >= nstage ? b - nstage : b; };
    auto fetch = [&](int s) {
#pragma unroll
      for (int e = 0; e < TW; ++e) {
        const int t = tb + kGemmStage * s + TW * wave + e;
        const uint16_t* src = kseq + size_t(t < te ? t : tb) * kTileElems + 8 * lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) xk[e][i] = *reinterpret_cast<const u32x4*>(src + 512 * i);
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int p = (tb + kGemmStage * s + kg + 4 * u) * 16 + ln;
        vl[u] = pool_valid[size_t(b) * P_max + (p < P_max ? p : 0)];
      }
    };
    // publish this wave's tile of stage s: keys to LDS, scale/sigma of its pools
    auto publish = [&](int s) {
      const int buf = s & 1;
#pragma unroll
      for (int e = 0; e < TW; ++e) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(&skeys[buf][TW * wave + e][8 * lane + 512 * i]) = xk[e][i];
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, gacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 bx = as_bf16x8(xk[e][i]);
          sacc = mfma16x16x32(ones, bx, sacc);
          gacc = mfma16x16x32(bx, bx, gacc);
        }
        const int jd = ln & 3;
        float dg = gacc[0];
        dg = jd == 1 ? gacc[1] : dg;
        dg = jd == 2 ? gacc[2] : dg;
        dg = jd == 3 ? gacc[3] : dg;
        const float sumsq = __int_as_float(__builtin_amdgcn_ds_bpermute(diag_addr, __float_as_int(dg)));
        const float mu = sacc[0] * (1.0f / kIsD);
        const float var = fmaxf(sumsq * (1.0f / kIsD) - mu * mu, 0.f);
        if (kg == 0) srs[buf][(TW * wave + e) * 16 + ln] = scale * __builtin_amdgcn_rsqf(var + eps);
      }
    };
    uint8_t vcur[NU];
    fetch(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) vcur[u] = vl[u];
    publish(0);
    __syncthreads();
    int bc = 0;  // the block of stage s
    for (int s = 0; s < nstage; ++s) {
      const int buf = s & 1;
      const int bn = next_blk(bc);  // the block of stage s + 1
      if constexpr (FILTER) {
        // a list that could not take this stage's candidates is shrunk first
        // (before the next stage's keys are requested: their registers are
        // free here)
        // a full list is shrunk now; so is every list above the target when
        // some wave's list was full after the last stage (its stamp: the
        // shrinks of a workgroup's waves overlap instead of each holding the
        // others at the barrier)
        const uint32_t room = uint32_t(fo.cap - kGemmStage * 16);
        const bool any_full = s > 0 && sfull[(s + 1) & 1] == ((uint32_t(i8) << 16) | uint32_t(s));
        if (mine && (fn > room || (any_full && fn > uint32_t(fo.target)))) {
          const uint64_t t = list_compact(fbuf, fn, uint32_t(fo.K), uint32_t(fo.target), shist[wave], flor, fland);
          fthr = t > fthr ? t : fthr;
          // (a threshold below the key of -FLT_MAX stands for no score: keep all)
          const bool none = uint32_t(fthr >> 32) < 0x00800000u;
          fthr_s = none ? -INFINITY : key_float(uint32_t(fthr >> 32));
          fthr_p = none ? 0xffffffffu : 0xffffffffu - uint32_t(fthr);
        }
      }
      if (s + 1 < nstage) fetch(bn);  // in flight while stage s is computed
      if (mine) {
        float mine_sc[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) mine_sc[u] = 0.f;
        // software pipeline: tile j+1's MFMAs are issued before tile j's
        // epilogue; the fragments of tile j+2 are read meanwhile
        u32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const u32x4*>(&skeys[buf][0][8 * lane + 512 * i]);
        f32x4 cur[NH];
        head_mfma_i<NH>(x, ahi, alo, cur);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const u32x4*>(&skeys[buf][1][8 * lane + 512 * i]);
#pragma unroll
        for (int j = 0; j < kGemmStage; ++j) {
          // the two waves of a SIMD share its matrix core; the older one wins
          // the arbitration, runs ahead and then waits at the stage barrier
          // while the other runs alone.  A wave's priority falls as it works
          // through the stage, so the wave that is behind wins instead (the
          // schedule measured best of several: 1.69 -> 1.61 ms per chunk)
          if (j < 6) __builtin_amdgcn_s_setprio(3);
          else if (j < 10) __builtin_amdgcn_s_setprio(2);
          else if (j < 13) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
          f32x4 nxt[NH];
          if (j + 1 < kGemmStage) {
            head_mfma_i<NH>(x, ahi, alo, nxt);
            if (j + 2 < kGemmStage) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                x[i] = *reinterpret_cast<const u32x4*>(&skeys[buf][j + 2][8 * lane + 512 * i]);
            }
          }
          const float rs = srs[buf][j * 16 + ln];
          float part = 0.f;
#pragma unroll
          for (int mb = 0; mb < NH; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) part = fmaf(cW[mb][jj], fmaxf(0.f, fmaf(rs, cur[mb][jj], cQ[mb][jj])), part);
          const float sc = sum_lane_groups(part);
          mine_sc[j >> 2] = kg == (j & 3) ? sc : mine_sc[j >> 2];
          if (j + 1 < kGemmStage) {
#pragma unroll
            for (int mb = 0; mb < NH; ++mb) cur[mb] = nxt[mb];
          }
        }
        if constexpr (FILTER) {
          // append the candidates whose key is >= the threshold, decided on
          // the score (the score map is monotone) and, at a score equal to
          // the threshold's, on the pool index (without that, a row whose
          // scores tie widely refills its list every few stages: 2.26 ms
          // against 1.64 ms for the prefill chunk with every pooled key
          // equal); at most 256, and the list has room for them.  The keys
          // are formed only when some lane keeps one (one ballot per stage:
          // after the first shrinks most stages keep nothing).
          uint32_t add = 0;
          bool keep[NU];
          bool any = false;
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int p = (tb + kGemmStage * bc + kg + 4 * u) * 16 + ln;
            keep[u] = p < P_max && vcur[u] != 0 && long(p) * kp <= last_ok && mine_sc[u] > -INFINITY &&
                      (mine_sc[u] > fthr_s || (mine_sc[u] == fthr_s && uint32_t(p) <= fthr_p));
            any = any || keep[u];
          }
          if (__ballot(any)) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
              const int p = (tb + kGemmStage * bc + kg + 4 * u) * 16 + ln;
              const uint64_t m = __ballot(keep[u]);
              const uint32_t at = fn + add + lane_rank(m);
              if (keep[u] && at < uint32_t(fo.cap)) {  // always in range: a shrink leaves <= cap - 256
                const uint64_t key = (uint64_t(score_key(mine_sc[u])) << 32) | (0xffffffffu - uint32_t(p));
                fbuf[at] = key;
                flor |= key;
                fland &= key;
              }
              add += uint32_t(__builtin_popcountll(m));
            }
          }
          fn += add;
          if (lane == 0 && fn > uint32_t(fo.cap - kGemmStage * 16)) sfull[s & 1] = ((uint32_t(i8) << 16) | uint32_t(s)) + 1u;
        } else {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int p = (tb + kGemmStage * bc + kg + 4 * u) * 16 + ln;
            if (p < P_max) srow[p] = (vcur[u] != 0 && long(p) * kp <= last_ok) ? mine_sc[u] : -INFINITY;
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      bc = bn;
      if (s + 1 < nstage) {
        publish(s + 1);
#pragma unroll
        for (int u = 0; u < NU; ++u) vcur[u] = vl[u];
      }
      __syncthreads();
    }
  }
  if constexpr (FILTER) {
    if (rok && lane == 0) fo.counts[size_t(r) * gridDim.x + blockIdx.x] = fn;  // 0 for rows naming no sequence
  } else {
    // rows naming no sequence: -inf throughout
    if (rok && !ok) {
      for (int t = tb; t < te; ++t)
        if (t * 16 + ln < P_max && kg == 0) scores[size_t(r) * P_max + t * 16 + ln] = -INFINITY;
    }
  }
}

// channels c .. c+7 of pool p from the pool cache (one 16-byte piece for
// bf16, two for fp32)
__device__ __forceinline__ void load_kp8(const uint16_t* k_pool, int b, int p, int c, int P_tiles, int D,
                                         float (&v)[8]) {
  load8(k_pool + KpLayout<uint16_t>::index(b, p, c, P_tiles, D), v);
}
__device__ __forceinline__ void load_kp8(const float* k_pool, int b, int p, int c, int P_tiles, int D,
                                         float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(k_pool + KpLayout<float>::index(b, p, c, P_tiles, D));
  const f32x4 z = *reinterpret_cast<const f32x4*>(k_pool + KpLayout<float>::index(b, p, c + 4, P_tiles, D));
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = z[i]; }
}

// Generic path: any H <= 64, D in {32, 64, 128}, fp32 or bf16 activations.
// One thread per pool; the normed key is formed explicitly in fp32 registers.
template <typename T, int D>
__global__ __launch_bounds__(256) void index_scores_generic(
    const T* __restrict__ q, const float* __restrict__ w, float scale, const T* __restrict__ k_pool,
    const int32_t* __restrict__ pool_start, const uint8_t* __restrict__ pool_valid,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int H, int B,
    int P_max, int kp, float* __restrict__ scores) {
  __shared__ float sq[64 * D];
  __shared__ float sw[64];
  const int r = blockIdx.y;
  const int b = row_seq[r];
  const int pos = row_pos[r];
  for (int u = threadIdx.x; u < H * D; u += blockDim.x) sq[u] = Act<T>::ld(q + size_t(r) * H * D + u);
  for (int u = threadIdx.x; u < H; u += blockDim.x) sw[u] = w[size_t(r) * H + u];
  __syncthreads();
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P_max) return;
  float* out = scores + size_t(r) * P_max + p;
  if (b < 0 || b >= B) { *out = -INFINITY; return; }
  const size_t pi = size_t(b) * P_max + p;
  if (!(pool_valid[pi] != 0 && pool_start[pi] + kp - 1 <= pos)) { *out = -INFINITY; return; }
  const int P_tiles = pool_tiles(P_max);
  float x[D];
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    float v[8];
    load_kp8(k_pool, b, p, c, P_tiles, D, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c + e] = v[e];
  }
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) m += x[c];
  m *= 1.0f / D;
  float v2 = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) v2 = fmaf(x[c] - m, x[c] - m, v2);
  const float rstd = 1.0f / sqrtf(v2 * (1.0f / D) + eps);
#pragma unroll
  for (int c = 0; c < D; ++c) x[c] = (x[c] - m) * rstd * gamma[c] + beta[c];
  float s = 0.f;
  for (int h = 0; h < H; ++h) {
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) d = fmaf(sq[h * D + c], x[c], d);
    s = fmaf(sw[h], fmaxf(0.f, scale * d), s);
  }
  *out = s;
}

// Decode launch shape: tiles per wave (tuned on MI355X at 4 x 65536 pools: 8
// tiles per wave, 512 pools per workgroup and two workgroups per CU, while
// that still gives >= 256 workgroups, then 4, then 1; 8 tiles per wave beat
// 4 (1024 workgroups), and a 2-deep ring with interleaved tile pairs beat a
// 4-deep ring).
static int stream_tiles(int Q, int P_max) {
  const long ntile = (P_max + 15) / 16;
  if (long(Q) * ((ntile + 31) / 32) >= 256) return 8;
  if (long(Q) * ((ntile + 15) / 16) >= 128) return 4;
  return 1;
}

// Prefill launch shape: 8 rows per workgroup; pool ranges of whole stages so
// that the grid has about 512 workgroups (two rounds over the CUs at one
// workgroup per CU), at most max_nx ranges per row.
static void gemm_grid(int Q, int P_max, int max_nx, int& nx, int& tiles_per_wg) {
  const int batches = ceil_div(Q, kGemmWaves);
  const int ptiles = pool_tiles(P_max);
  int lim = ceil_div(ptiles, kGemmStage);
  if (lim > max_nx) lim = max_nx;
  nx = ceil_div(512, batches);
  if (nx > lim) nx = lim;
  if (nx < 1) nx = 1;
  tiles_per_wg = ceil_div(ceil_div(ptiles, nx), kGemmStage) * kGemmStage;
  nx = ceil_div(ptiles, tiles_per_wg);
}

int filter_supported(int Q, int H, int D, int dtype) {
  return dtype == DSA_BF16 && D == 128 && (H == 16 || H == 32) && Q > 64 && ceil_div(Q, kGemmWaves) <= 65535;
}

int filter_ranges(int Q, int P_max, int max_ranges) {
  int nx, tpw;
  gemm_grid(Q, P_max, max_ranges, nx, tpw);
  return nx;
}

int index_scores_filter(const void* q, const float* w, float scale, const void* k_pool, const int32_t* pool_start,
                        const uint8_t* pool_valid, const float* ln_gamma, const float* ln_beta, float ln_eps,
                        const int32_t* row_seq, const int32_t* row_pos, int Q, int H, int B, int P_max, int kpool,
                        int K, int cap, int max_ranges, uint64_t* keys, uint32_t* counts, hipStream_t s) {
  int nx, tiles_per_wg;
  gemm_grid(Q, P_max, max_ranges, nx, tiles_per_wg);
  dim3 g(nx, ceil_div(Q, kGemmWaves));
  const FilterOut fo{keys, counts, cap, K, K + (cap - kGemmStage * 16 - K) / 2};
#define DSA_IS_FILTER(NH)                                                                                   \
  hipLaunchKernelGGL((index_scores_gemm<NH, true>), g, dim3(kGemmWaves * 64), 0, s, (const uint16_t*)q, w, scale, \
                     (const uint16_t*)k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq, row_pos, \
                     Q, B, P_max, kpool, tiles_per_wg, nullptr, fo)
  if (H == 32) DSA_IS_FILTER(2);
  else DSA_IS_FILTER(1);
#undef DSA_IS_FILTER
  return launch_status();
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_index_scores(const void* q, const float* w, float scale, const void* k_pool,
                                const int32_t* pool_start, const uint8_t* pool_valid,
                                const float* ln_gamma, const float* ln_beta, float ln_eps,
                                const int32_t* row_seq, const int32_t* row_pos, int Q, int H, int D,
                                int B, int P_max, int kpool, int dtype, float* scores,
                                void* stream) {
  if (!q || !w || !k_pool || !pool_start || !pool_valid || !ln_gamma || !ln_beta || !row_seq ||
      !row_pos || !scores)
    return DSA_ERR_NULL;
  if (Q <= 0 || H <= 0 || D <= 0 || B <= 0 || P_max <= 0 || kpool <= 0) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL) return DSA_ERR_UNSUPPORTED;
  if (H > 64 || (D != 32 && D != 64 && D != 128)) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (dtype == DSA_BF16 && D == 128 && (H == 16 || H == 32)) {
    if (Q <= 64) {
      // decode kernel: one row per grid row
      const int tw = stream_tiles(Q, P_max);
      dim3 grid(ceil_div(P_max, kIsWaves * tw * 16), Q);
#define DSA_IS_STREAM(NH, NT)                                                                       \
  hipLaunchKernelGGL((index_scores_stream<NH, NT>), grid, dim3(kIsThreads), 0, s, (const uint16_t*)q, w, \
                     scale, (const uint16_t*)k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps,   \
                     row_seq, row_pos, B, P_max, kpool, scores)
      if (H == 32) {
        if (tw == 8) DSA_IS_STREAM(2, 8);
        else if (tw == 4) DSA_IS_STREAM(2, 4);
        else DSA_IS_STREAM(2, 1);
      } else {
        if (tw == 8) DSA_IS_STREAM(1, 8);
        else if (tw == 4) DSA_IS_STREAM(1, 4);
        else DSA_IS_STREAM(1, 1);
      }
#undef DSA_IS_STREAM
      return launch_status();
    }
    // prefill kernel (launch shape: gemm_grid)
    const int batches = ceil_div(Q, kGemmWaves);
    if (batches > 65535) return DSA_ERR_UNSUPPORTED;
    int nx, tiles_per_wg;
    gemm_grid(Q, P_max, INT_MAX, nx, tiles_per_wg);
    dim3 g(nx, batches);
#define DSA_IS_GEMM(NH)                                                                                    \
  hipLaunchKernelGGL((index_scores_gemm<NH, false>), g, dim3(kGemmWaves * 64), 0, s, (const uint16_t*)q, w, scale, \
                     (const uint16_t*)k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq,         \
                     row_pos, Q, B, P_max, kpool, tiles_per_wg, scores, FilterOut{})
    if (H == 32) DSA_IS_GEMM(2);
    else DSA_IS_GEMM(1);
#undef DSA_IS_GEMM
    return launch_status();
  }
  if (Q > 65535) return DSA_ERR_UNSUPPORTED;
  dim3 grid(ceil_div(P_max, 256), Q);
#define DSA_IS_GENERIC(T, DD)                                                                      \
  hipLaunchKernelGGL((index_scores_generic<T, DD>), grid, dim3(256), 0, s, (const T*)q, w, scale, \
                     (const T*)k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps, row_seq, \
                     row_pos, H, B, P_max, kpool, scores)
  if (dtype == DSA_BF16) {
    if (D == 32) DSA_IS_GENERIC(uint16_t, 32);
    else if (D == 64) DSA_IS_GENERIC(uint16_t, 64);
    else DSA_IS_GENERIC(uint16_t, 128);
  } else {
    if (D == 32) DSA_IS_GENERIC(float, 32);
    else if (D == 64) DSA_IS_GENERIC(float, 64);
    else DSA_IS_GENERIC(float, 128);
  }
#undef DSA_IS_GENERIC
  return launch_status();
}
