// index_scores: indexer scores with candidate validity (page "Module
// glm5next_dsa", "Shape of the pipeline" and "Traps carried from Slice 8":
// k_norm is a LayerNorm with bias; page "Module tp", "Why the indexer is
// REPLICATED, not sharded": score = sum over heads of w[h]*relu(scale*dot)).
//
// MFMA path (bf16, D = 128, H in {16, 32}).  The LayerNorm is folded into the
// contraction: with x the pooled key, mu / r its mean / inverse std and
// g[h,c] = q[h,c]*gamma[c],
//     <q_h, LN(x)> = r * (sum_c g[h,c] x_c - mu * sum_c g[h,c]) + sum_c q[h,c] beta[c].
// sum_c g[h,c] x_c runs on the matrix cores with heads as M and pools as N:
// x is exact bf16, and g is carried as an unevaluated pair g_hi + g_lo of
// bf16 values (g - g_hi - g_lo is ~2^-17 |g|), both accumulated into the same
// fp32 accumulator.  The normed key is never rounded.
//
// A workgroup is 4 waves; each wave owns kTiles tiles of 16 pools and keeps
// their keys in registers (one 16-byte load per lane per 32 channels, the
// lane's pool is lane & 15).  Key loads are issued before the per-row set-up,
// so they are in flight while the workgroup prepares g.  The same kernel runs
// decode (one row per workgroup, grid.y = rows) and prefill (a group of rows
// of one sequence per workgroup; the keys are reused across the rows).
//
// Per pool the decode kernel moves 256 B of key + 1 B valid + 4 B start and
// writes 4 B of score: HBM-bound (the fold keeps the fp32 vector work to the
// LayerNorm statistics and the head reduction).
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kIsThreads = 256;
constexpr int kIsWaves = kIsThreads / kWave;
constexpr int kIsD = 128;
constexpr int kIsLd = kIsD + 8;  // padded LDS row: 16 lanes reading 16 rows hit distinct banks

template <int NH, int RPB>  // H = 16 * NH index heads; RPB rows staged in LDS at once
struct IsShared {
  uint16_t ghi[RPB][NH * 16][kIsLd];
  uint16_t glo[RPB][NH * 16][kIsLd];
  float G[RPB][NH * 16];   // sum_c (g_hi + g_lo)
  float QB[RPB][NH * 16];  // sum_c q * beta
  float W[RPB][NH * 16];
  int pos[RPB];
  int seq[RPB];
};

template <int NH, int kTiles, int RPB>
__global__ __launch_bounds__(kIsThreads) void index_scores_mfma(
    const uint16_t* __restrict__ q, const float* __restrict__ w, float scale,
    const uint16_t* __restrict__ k_pool, const int32_t* __restrict__ pool_start,
    const uint8_t* __restrict__ pool_valid, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int Q, int B, int P_max, int kp, int rows_per_group,
    float* __restrict__ scores) {
  constexpr int H = NH * 16;
  __shared__ IsShared<NH, RPB> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, ln = lane & 15;
  const int r_begin = blockIdx.y * rows_per_group;
  const int r_end = min(Q, r_begin + rows_per_group);
  const int p_wave = blockIdx.x * (kIsWaves * kTiles * 16) + wave * (kTiles * 16);

  // sequence of the first row decides which keys are loaded; rows of another
  // sequence in the same group reload (correct, slower; groups are normally
  // rows of one sequence)
  int b_loaded = row_seq[r_begin];

  // ---- issue the key loads of this wave's tiles ----
  u32x4 xk[kTiles][4];
  auto load_keys = [&](int b) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int p = p_wave + t * 16 + ln;
      const bool in = (p < P_max) && b >= 0 && b < B;
      const uint16_t* src = k_pool + (size_t(in ? b : 0) * P_max + (in ? p : 0)) * kIsD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // channel group kg + 4i of this pool: 8 channels, 16 bytes
        xk[t][i] = in ? *reinterpret_cast<const u32x4*>(src + (kg + 4 * i) * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  load_keys(b_loaded);

  float mu[kTiles], rs[kTiles];
  auto ln_stats = [&]() {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      float s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s1 += __uint_as_float(xk[t][i][e] << 16);
          s1 += __uint_as_float(xk[t][i][e] & 0xffff0000u);
        }
      s1 += __shfl_xor(s1, 16, kWave);
      s1 += __shfl_xor(s1, 32, kWave);
      const float m = s1 * (1.0f / kIsD);
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = __uint_as_float(xk[t][i][e] << 16) - m;
          const float c = __uint_as_float(xk[t][i][e] & 0xffff0000u) - m;
          s2 = fmaf(a, a, s2);
          s2 = fmaf(c, c, s2);
        }
      s2 += __shfl_xor(s2, 16, kWave);
      s2 += __shfl_xor(s2, 32, kWave);
      mu[t] = m;
      rs[t] = 1.0f / sqrtf(s2 * (1.0f / kIsD) + eps);
    }
  };
  bool stats_done = false;

  for (int rb = r_begin; rb < r_end; rb += RPB) {
    const int nr = min(RPB, r_end - rb);
    __syncthreads();  // previous batch's LDS reads are finished
    // ---- stage g = q * gamma as (hi, lo) bf16 pairs, G, QB, w ----
    for (int u = tid; u < nr * H * 8; u += kIsThreads) {
      const int rr = u / (H * 8), h = (u / 8) % H, part = u % 8;
      const int r = rb + rr;
      const uint16_t* qs = q + (size_t(r) * H + h) * kIsD + part * 16;
      float gs = 0.f, qbs = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float qv[8], gm[8], bt[8];
        load8(qs + half * 8, qv);
        load8(gamma + part * 16 + half * 8, gm);
        load8(beta + part * 16 + half * 8, bt);
        uint16_t hi8[8], lo8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = qv[e] * gm[e];
          const uint16_t hi = f2bf(g);
          const uint16_t lo = f2bf(g - bf2f(hi));
          hi8[e] = hi;
          lo8[e] = lo;
          gs += bf2f(hi) + bf2f(lo);
          qbs = fmaf(qv[e], bt[e], qbs);
        }
        u32x4 ph, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[e] = uint32_t(hi8[2 * e]) | (uint32_t(hi8[2 * e + 1]) << 16);
          pl[e] = uint32_t(lo8[2 * e]) | (uint32_t(lo8[2 * e + 1]) << 16);
        }
        *reinterpret_cast<u32x4*>(&sh.ghi[rr][h][part * 16 + half * 8]) = ph;
        *reinterpret_cast<u32x4*>(&sh.glo[rr][h][part * 16 + half * 8]) = pl;
      }
      // reduce over the 8 consecutive threads of one (row, head)
      gs += __shfl_xor(gs, 1, kWave);
      gs += __shfl_xor(gs, 2, kWave);
      gs += __shfl_xor(gs, 4, kWave);
      qbs += __shfl_xor(qbs, 1, kWave);
      qbs += __shfl_xor(qbs, 2, kWave);
      qbs += __shfl_xor(qbs, 4, kWave);
      if (part == 0) {
        sh.G[rr][h] = gs;
        sh.QB[rr][h] = qbs;
        sh.W[rr][h] = w[size_t(r) * H + h];
      }
    }
    if (tid < nr) {
      sh.pos[tid] = row_pos[rb + tid];
      sh.seq[tid] = row_seq[rb + tid];
    }
    __syncthreads();

    for (int rr = 0; rr < nr; ++rr) {
      const int r = rb + rr;
      const int b = sh.seq[rr];
      const int pos = sh.pos[rr];
      float* srow = scores + size_t(r) * P_max;
      const bool ok = b >= 0 && b < B;
      if (ok && b != b_loaded) {  // row of another sequence: reload its keys
        b_loaded = b;
        load_keys(b);
        stats_done = false;
      }
      if (!ok) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int p = p_wave + t * 16 + ln;
          if (kg == 0 && p < P_max) srow[p] = -INFINITY;
        }
        continue;
      }
      if (!stats_done) {
        ln_stats();
        stats_done = true;
      }
      // A operands (g for this row): M-block mb, k-step i
      bf16x8 ahi[NH][4], alo[NH][4];
      float cG[NH][4], cQ[NH][4], cW[NH][4];
#pragma unroll
      for (int mb = 0; mb < NH; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ahi[mb][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.ghi[rr][mb * 16 + ln][(kg + 4 * i) * 8]));
          alo[mb][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.glo[rr][mb * 16 + ln][(kg + 4 * i) * 8]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = mb * 16 + 4 * kg + j;
          cG[mb][j] = sh.G[rr][h];
          cQ[mb][j] = sh.QB[rr][h];
          cW[mb][j] = sh.W[rr][h];
        }
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const int p = p_wave + t * 16 + ln;
        int ps = -1, pv = 0;
        if (kg == 0 && p < P_max) {
          ps = pool_start[size_t(b) * P_max + p];
          pv = pool_valid[size_t(b) * P_max + p];
        }
        f32x4 acc[NH];
#pragma unroll
        for (int mb = 0; mb < NH; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 bx = as_bf16x8(xk[t][i]);
#pragma unroll
          for (int mb = 0; mb < NH; ++mb) {
            acc[mb] = mfma16x16x32(ahi[mb][i], bx, acc[mb]);
            acc[mb] = mfma16x16x32(alo[mb][i], bx, acc[mb]);
          }
        }
        float part = 0.f;
#pragma unroll
        for (int mb = 0; mb < NH; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float dot = rs[t] * (acc[mb][j] - mu[t] * cG[mb][j]) + cQ[mb][j];
            part = fmaf(cW[mb][j], fmaxf(0.f, scale * dot), part);
          }
        part += __shfl_xor(part, 16, kWave);
        part += __shfl_xor(part, 32, kWave);
        if (kg == 0 && p < P_max) {
          const bool cand = pv != 0 && ps + kp - 1 <= pos;
          srow[p] = cand ? part : -INFINITY;
        }
      }
    }
  }
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
  float x[D];
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    float v[8];
    load8(k_pool + pi * D + c, v);
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

// Pools per workgroup and rows per workgroup for the MFMA path.
struct IsPlan {
  int tiles;           // 16-pool tiles per wave (fixed at 4)
  int rows_per_group;  // rows per workgroup (1: decode)
};

static IsPlan is_plan(int Q, int P_max) {
  // Decode (few rows): one row per workgroup, 4 tiles per wave (256 pools per
  // workgroup): ~1000 workgroups at 4 x 65536 pools, all key loads in flight
  // from the start.  Many rows: groups of rows share the keys held in registers.
  IsPlan pl{4, 1};
  if (Q > 64) {
    const long chunks = (P_max + 255) / 256;
    int groups = int((2048 + chunks - 1) / chunks);
    if (groups < 1) groups = 1;
    const int per = (Q + groups - 1) / groups;
    pl.rows_per_group = per > 16 ? per : 16;
  }
  return pl;
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
  if (Q > 65535 * 64) return DSA_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (dtype == DSA_BF16 && D == 128 && (H == 16 || H == 32)) {
    const IsPlan pl = is_plan(Q, P_max);
    const int pools_per_wg = kIsWaves * pl.tiles * 16;
    dim3 grid(ceil_div(P_max, pools_per_wg), ceil_div(Q, pl.rows_per_group));
    if (grid.y > 65535) return DSA_ERR_UNSUPPORTED;
    auto args = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(kIsThreads), 0, s, (const uint16_t*)q, w, scale,
                         (const uint16_t*)k_pool, pool_start, pool_valid, ln_gamma, ln_beta, ln_eps,
                         row_seq, row_pos, Q, B, P_max, kpool, pl.rows_per_group, scores);
    };
    if (pl.rows_per_group == 1) {
      if (H == 32) args(index_scores_mfma<2, 4, 1>);
      else args(index_scores_mfma<1, 4, 1>);
    } else {
      if (H == 32) args(index_scores_mfma<2, 4, 4>);
      else args(index_scores_mfma<1, 4, 4>);
    }
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
