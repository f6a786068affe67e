// sparse_mla_decode: absorbed NoPE MLA decode restricted to the selected
// tokens (page "Module glm5next_dsa", "Shape of the pipeline" and "Traps
// carried from Slice 8": NoPE, the rotary slice is zero-width; page "Module
// tp", "Traps this module encodes": one shared latent per token, no head axis).
//
// Absorbed MLA attends with the latent as both key and value: for each head,
// logits sm_scale * <q_lat_h, kv_j> over the listed tokens j, softmax, and the
// softmax-weighted sum of the same kv_j rows.
//
// MFMA path (bf16, Dl = 512, Hm a multiple of 16).  A workgroup handles one
// row, one group of 16 heads and a contiguous slice ("split") of 64 ids of the
// row's list.  Its 4 waves each own a quarter of the latent width (128 of the
// 512 channels):
//   - the split's 64 latent rows are gathered into LDS (16-byte loads);
//   - each wave forms partial logits S^T[token, head] = kv . q^T over its
//     quarter on the matrix cores; the four partials are summed through LDS;
//   - every wave takes the (same) softmax over the 64 ids and accumulates its
//     quarter of O^T[dl, head] = kv^T . P^T on the matrix cores.
// The row-major LDS copy serves both contractions: 16-byte reads for the
// logits and eight 16-bit reads per lane for kv^T; the row swizzle makes both
// bank-conflict free.  80 KiB of LDS and <= 256 registers per lane keep two
// workgroups per CU.  The head groups of one (row, split) read the same latent
// rows; their workgroup ids are spaced by a multiple of 8 so that they share an
// XCD and its L2.  Splits write normalised partial outputs, rounded to bf16 (in
// the lanes' order: 512 B per store instruction), and their fp32 log-sum-exp;
// a combine launch merges them in fp32.  The gather is the HBM traffic (1 KiB per selected token).
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kMlaDl = 512;
constexpr int kMlaSplit = 64;   // ids per workgroup
constexpr int kMlaThreads = 256;

struct MlaShared {
  uint16_t rows[kMlaSplit][kMlaDl];  // 16-byte pieces swizzled per row (64 KiB)
  union {
    int ids[kMlaSplit];              // during the gather
    f32x4 lg[4][4][64];              // partial logits [wave][block][lane] (16 KiB)
  } u;
};

// piece c of token row t sits at piece (c ^ row_swz(t)).  The 16 rows of one
// logits read (t = 8a + 4b + j, a, j < 4) and the 4 row groups of one kv^T
// read (t = 8kg + e) both land on distinct banks.
__device__ __forceinline__ int row_swz(int t) { return (t & 3) | ((t >> 1) & 12); }

// token held by row m of logits block mb: lane group kg of block pair
// (2ks, 2ks+1) receives tokens 32ks + 8kg .. 32ks + 8kg + 7
__device__ __forceinline__ int blk_token(int mb, int m) {
  return 32 * (mb >> 1) + 8 * (m >> 2) + 4 * (mb & 1) + (m & 3);
}

// offset (in elements) of partial-output element (head group hg, lane, dl) of a
// (row, split): [hg][dq][blk][lane][j], dl = 128 dq + 16 blk + 4 kg + j
__device__ __forceinline__ size_t part_off(size_t rs, int HG, int hg, int dq, int blk, int lane) {
  return ((((rs * HG + hg) * 4 + dq) * 8 + blk) * 64 + lane) * 4;
}

__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_decode_mfma(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int Hm, int B,
    int T_max, int W, int nsplit, int ns8, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ MlaShared sh;
  const int tid = threadIdx.x, lane = tid & 63, dq = tid >> 6;  // wave = latent quarter
  const int kg = lane >> 4, ln = lane & 15;
  const int HG = Hm >> 4;
  const int hg = blockIdx.x / ns8, sp = blockIdx.x % ns8;
  if (sp >= nsplit) return;  // padding workgroups (uniform exit)
  const int r = blockIdx.y;
  const int h = hg * 16 + ln;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const size_t seq_base = size_t(bok ? b : 0) * T_max;
  const int c_begin = sp * kMlaSplit;

  if (tid < kMlaSplit) {
    const int c = c_begin + tid;
    int id = -1;
    if (c < W) {
      id = token_ids[size_t(r) * W + c];
      if (!bok || id < 0 || id >= T_max) id = -1;
    }
    sh.u.ids[tid] = id;
  }
  // q_lat of head h, latent quarter dq, as the B operand of the logits
  bf16x8 qop[4];
  {
    const uint16_t* qs = q_lat + (size_t(r) * Hm + h) * kMlaDl + dq * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) qop[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + (kg + 4 * i) * 8));
  }
  __syncthreads();
  // validity of this lane's 16 logits (tokens 32ks + 8kg + e), read before the
  // id array is reused for the logits exchange
  uint32_t vmask = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) vmask |= (sh.u.ids[32 * (e >> 3) + 8 * kg + (e & 7)] >= 0 ? 1u : 0u) << e;
  {
    // gather: piece k of this thread is row (tid >> 6) + 4k, 16-byte piece tid & 63
    u32x4 gv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int id = sh.u.ids[(tid >> 6) + 4 * k];
      gv[k] = *reinterpret_cast<const u32x4*>(kv + (seq_base + (id >= 0 ? id : 0)) * kMlaDl + (tid & 63) * 8);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = (tid >> 6) + 4 * k, c = tid & 63;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sh.rows[t][(c ^ row_swz(t)) * 8]) = sh.u.ids[t] >= 0 ? gv[k] : z;
    }
  }
  __syncthreads();

  // partial logits over this wave's latent quarter
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int t = blk_token(mb, ln);
    const int sw = row_swz(t);
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.rows[t][((dq * 16 + kg + 4 * i) ^ sw) * 8]));
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = mfma16x16x32(a[i], qop[i], acc);
    sh.u.lg[dq][mb][lane] = acc;
  }
  __syncthreads();
  // lane (kg, ln): head h, logits of tokens 32ks + 8kg + e at x[8ks + e]
  float x[16];
  float m = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const f32x4 s0 = sh.u.lg[0][mb][lane], s1 = sh.u.lg[1][mb][lane];
    const f32x4 s2 = sh.u.lg[2][mb][lane], s3 = sh.u.lg[3][mb][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 8 * (mb >> 1) + 4 * (mb & 1) + j;
      const float v = ((s0[j] + s1[j]) + (s2[j] + s3[j])) * scale_log2;
      x[e] = (vmask >> e) & 1u ? v : -INFINITY;
      m = fmaxf(m, x[e]);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  const float m_use = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  uint32_t pk[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[8 * ks + e] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(x[8 * ks + e + 1] - m_use);
      l += p0 + p1;
      pk[ks][e >> 1] = pack2bf(p0, p1);
    }
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  const bf16x8 pb0 = as_bf16x8(u32x4{pk[0][0], pk[0][1], pk[0][2], pk[0][3]});
  const bf16x8 pb1 = as_bf16x8(u32x4{pk[1][0], pk[1][1], pk[1][2], pk[1][3]});

  // O^T[dl, head] = kv^T[dl, tokens] . P^T[tokens, head] over this quarter
  f32x4 o[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int d = dq * 128 + blk * 16 + ln;
    const int c = d >> 3, off = d & 7;
    uint32_t wv[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int t0 = 32 * ks + 8 * kg + e, t1 = t0 + 1;
        const uint32_t lo = sh.rows[t0][((c ^ row_swz(t0)) << 3) + off];
        const uint32_t hi = sh.rows[t1][((c ^ row_swz(t1)) << 3) + off];
        wv[ks][e >> 1] = lo | (hi << 16);
      }
    o[blk] = mfma16x16x32(as_bf16x8(u32x4{wv[0][0], wv[0][1], wv[0][2], wv[0][3]}), pb0, f32x4{0.f, 0.f, 0.f, 0.f});
    o[blk] = mfma16x16x32(as_bf16x8(u32x4{wv[1][0], wv[1][1], wv[1][2], wv[1][3]}), pb1, o[blk]);
  }

  // o[blk][j] = sum_t p_t kv[t][dl = 128 dq + 16 blk + 4 kg + j] for head h
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const float lse_v = l > 0.f ? (m_use + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
  if (nsplit == 1) {
    uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + dq * 128 + 4 * kg;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      u32x2 pkd;
      pkd[0] = pack2bf(o[blk][0] * inv, o[blk][1] * inv);
      pkd[1] = pack2bf(o[blk][2] * inv, o[blk][3] * inv);
      *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
    }
    if (dq == 0 && kg == 0 && lse) lse[size_t(r) * Hm + h] = lse_v;
  } else {
    const size_t rs = size_t(r) * nsplit + sp;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      u32x2 pkd;
      pkd[0] = pack2bf(o[blk][0] * inv, o[blk][1] * inv);
      pkd[1] = pack2bf(o[blk][2] * inv, o[blk][3] * inv);
      *reinterpret_cast<u32x2*>(part_o + part_off(rs, HG, hg, dq, blk, lane)) = pkd;
    }
    if (dq == 0 && kg == 0) part_lse[rs * Hm + h] = lse_v;
  }
}

// Merge split partials: out = sum_s e^{lse_s} O_s / sum_s e^{lse_s}.  One
// workgroup per (row, head group, latent quarter); thread = (blk, lane) of
// the partial layout, so every split's read is one contiguous 8 KiB block.
constexpr int kMaxSplit = 256;
__global__ __launch_bounds__(512) void mla_combine(const uint16_t* __restrict__ part_o,
                                                   const float* __restrict__ part_lse, int nsplit,
                                                   int Hm, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse) {
  __shared__ float wgt[kMaxSplit][16];
  __shared__ float sM[16], sWs[16];
  const int HG = Hm >> 4;
  const int hg = blockIdx.x >> 2, dq = blockIdx.x & 3, r = blockIdx.y;
  const int tid = threadIdx.x, blk = tid >> 6, lane = tid & 63, kg = lane >> 4, ln = lane & 15;
  // split weights per head of the group: thread (s, head) loads one lse; the
  // max and the sum over splits run as LDS reductions per head
  for (int u = tid; u < nsplit * 16; u += 512)
    wgt[u >> 4][u & 15] = part_lse[(size_t(r) * nsplit + (u >> 4)) * Hm + hg * 16 + (u & 15)];
  __syncthreads();
  if (tid < 16) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, wgt[s][tid]);
    sM[tid] = M;
  }
  __syncthreads();
  for (int u = tid; u < nsplit * 16; u += 512) {
    const float M = sM[u & 15], l = wgt[u >> 4][u & 15];
    wgt[u >> 4][u & 15] = (M == -INFINITY || l == -INFINITY) ? 0.f : __expf(l - M);
  }
  __syncthreads();
  if (tid < 16) {
    float ws = 0.f;
    for (int s = 0; s < nsplit; ++s) ws += wgt[s][tid];
    sWs[tid] = ws;
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const u32x2 pv = *reinterpret_cast<const u32x2*>(part_o + part_off(size_t(r) * nsplit + s, HG, hg, dq, blk, lane));
    const f32x4 v = {__uint_as_float(pv[0] << 16), __uint_as_float(pv[0] & 0xffff0000u),
                     __uint_as_float(pv[1] << 16), __uint_as_float(pv[1] & 0xffff0000u)};
    acc += wgt[s][ln] * v;
  }
  const float ws = sWs[ln];
  const float inv = ws > 0.f ? 1.0f / ws : 0.f;
  const int h = hg * 16 + ln;
  u32x2 pk;
  pk[0] = pack2bf(acc[0] * inv, acc[1] * inv);
  pk[1] = pack2bf(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(out + (size_t(r) * Hm + h) * kMlaDl + dq * 128 + blk * 16 + 4 * kg) = pk;
  if (dq == 0 && blk == 0 && kg == 0 && lse) lse[size_t(r) * Hm + h] = ws > 0.f ? sM[ln] + logf(ws) : -INFINITY;
}

// Generic path (fp32 or bf16, any Dl <= 512, any Hm): one workgroup per
// (head, row), 256 ids per step, online softmax, fp32 throughout.
template <typename T>
__global__ __launch_bounds__(256) void mla_decode_generic(
    const T* __restrict__ q_lat, const T* __restrict__ kv, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ token_ids, int Hm, int Dl, int B, int T_max, int W, float sm_scale,
    T* __restrict__ out, float* __restrict__ lse) {
  __shared__ float sq[kMlaDl];
  __shared__ float sp[256];
  __shared__ int sid[256];
  __shared__ float red[4];
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  for (int d = tid; d < Dl; d += 256) sq[d] = Act<T>::ld(q_lat + (size_t(r) * Hm + h) * Dl + d);
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int cb = 0; cb < W; cb += 256) {
    const int c = cb + tid;
    int id = -1;
    if (c < W) {
      id = token_ids[size_t(r) * W + c];
      if (!bok || id < 0 || id >= T_max) id = -1;
    }
    float logit = -INFINITY;
    if (id >= 0) {
      const T* row = kv + (size_t(b) * T_max + id) * Dl;
      float dot = 0.f;
      for (int d = 0; d < Dl; ++d) dot = fmaf(sq[d], Act<T>::ld(row + d), dot);
      logit = dot * sm_scale;
    }
    sid[tid] = id;
    float cm = wave_max(logit);
    if (lane == 0) red[wave] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, cm);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float p = expf(logit - m_use);
    sp[tid] = p;
    float ps = wave_sum(p);
    if (lane == 0) red[wave] = ps;
    __syncthreads();
    ps = red[0] + red[1] + red[2] + red[3];
    const float alpha = expf(m_run - m_use);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    acc0 *= alpha;
    acc1 *= alpha;
    const int n = min(256, W - cb);
    for (int t = 0; t < n; ++t) {
      const int idt = sid[t];
      if (idt < 0) continue;
      const T* row = kv + (size_t(b) * T_max + idt) * Dl;
      const float pt = sp[t];
      if (tid < Dl) acc0 = fmaf(pt, Act<T>::ld(row + tid), acc0);
      if (tid + 256 < Dl) acc1 = fmaf(pt, Act<T>::ld(row + tid + 256), acc1);
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  T* dst = out + (size_t(r) * Hm + h) * Dl;
  if (tid < Dl) Act<T>::st(dst + tid, acc0 * inv);
  if (tid + 256 < Dl) Act<T>::st(dst + tid + 256, acc1 * inv);
  if (tid == 0 && lse) lse[size_t(r) * Hm + h] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

struct MlaPlan {
  bool mfma;
  int nsplit;  // id slices of kMlaSplit per row
  int ns8;     // nsplit rounded up to a multiple of 8 (XCD spacing)
};

static MlaPlan mla_plan(int Q, int Hm, int Dl, int W, int dtype) {
  MlaPlan pl{false, 1, 1};
  if (!(dtype == DSA_BF16 && Dl == kMlaDl && Hm % 16 == 0 && Hm <= 128)) return pl;
  pl.mfma = true;
  pl.nsplit = (W + kMlaSplit - 1) / kMlaSplit;
  pl.ns8 = (pl.nsplit + 7) / 8 * 8;
  return pl;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_sparse_mla_workspace_bytes(int Q, int Hm, int Dl, int W, int dtype) {
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || W <= 0) return 0;
  const MlaPlan pl = mla_plan(Q, Hm, Dl, W, dtype);
  if (!pl.mfma || pl.nsplit == 1) return 0;
  return align256(size_t(Q) * pl.nsplit * Hm * Dl * sizeof(uint16_t)) +
         align256(size_t(Q) * pl.nsplit * Hm * sizeof(float));
}

extern "C" int dsa_sparse_mla_decode(const void* q_lat, const void* kv, const int32_t* row_seq,
                                     const int32_t* token_ids, int Q, int Hm, int Dl, int B,
                                     int T_max, int W, float sm_scale, int dtype, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!q_lat || !kv || !row_seq || !token_ids || !out) return DSA_ERR_NULL;
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || B <= 0 || T_max <= 0 || W <= 0) return DSA_ERR_SHAPE;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  if (Dl != 64 && Dl != 128 && Dl != 256 && Dl != 512) return DSA_ERR_UNSUPPORTED;
  if (Hm > 128 || Q > 65535) return DSA_ERR_UNSUPPORTED;
  if (long(W) > long(kMlaSplit) * kMaxSplit) return DSA_ERR_UNSUPPORTED;
  const MlaPlan pl = mla_plan(Q, Hm, Dl, W, dtype);
  const size_t need = dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  if (!pl.mfma) {
    dim3 grid(Hm, Q);
    if (dtype == DSA_BF16)
      hipLaunchKernelGGL(mla_decode_generic<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)q_lat,
                         (const uint16_t*)kv, row_seq, token_ids, Hm, Dl, B, T_max, W, sm_scale,
                         (uint16_t*)out, lse);
    else
      hipLaunchKernelGGL(mla_decode_generic<float>, grid, dim3(256), 0, s, (const float*)q_lat,
                         (const float*)kv, row_seq, token_ids, Hm, Dl, B, T_max, W, sm_scale,
                         (float*)out, lse);
    return launch_status();
  }
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (pl.nsplit > 1) {
    part_o = static_cast<uint16_t*>(workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(size_t(Q) * pl.nsplit * Hm * Dl * sizeof(uint16_t)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid((Hm / 16) * pl.ns8, Q);
  hipLaunchKernelGGL(mla_decode_mfma, grid, dim3(kMlaThreads), 0, s, (const uint16_t*)q_lat,
                     (const uint16_t*)kv, row_seq, token_ids, Hm, B, T_max, W, pl.nsplit, pl.ns8,
                     scale_log2, (uint16_t*)out, lse, part_o, part_lse);
  int st = launch_status();
  if (st || pl.nsplit == 1) return st;
  hipLaunchKernelGGL(mla_combine, dim3((Hm / 16) * 4, Q), dim3(512), 0, s, part_o, part_lse, pl.nsplit,
                     Hm, (uint16_t*)out, lse);
  return launch_status();
}
