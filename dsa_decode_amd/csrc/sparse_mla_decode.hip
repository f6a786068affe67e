// sparse_mla_decode: absorbed NoPE MLA decode restricted to the selected
// tokens (page "Module glm5next_dsa", "Shape of the pipeline" and "Traps
// carried from Slice 8": NoPE, the rotary slice is zero-width; page "Module
// tp", "Traps this module encodes": one shared latent per token, no head axis).
//
// Absorbed MLA attends with the latent as both key and value: for each head,
// logits sm_scale * <q_lat_h, kv_j> over the listed tokens j, softmax, and the
// softmax-weighted sum of the same kv_j rows.
//
// MFMA path (bf16, Dl = 512, Hm = 16 * waves).  A workgroup handles one row and
// a contiguous slice ("split") of at most 64 ids of its list; each wave owns
// 16 heads.  The workgroup gathers the split's latent rows (1 KiB each, 16-byte
// loads) into LDS once, computes all logits S^T[token, head] = kv . q^T on the
// matrix cores, takes the softmax of the split in one pass (no running
// rescale), and accumulates O^T[dl, head] = kv^T . P^T.  The kv^T operand is
// read from the same row-major LDS copy as eight 16-bit reads per lane; the
// row swizzle makes both access patterns bank-conflict free.  Splits write
// normalised fp32 partial outputs and their log-sum-exp; a combine launch
// merges them.  The gather is the HBM traffic (1 KiB per selected token); the
// two contractions are ~256 flop per gathered byte.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kMlaDl = 512;
constexpr int kMlaSplit = 64;  // ids per workgroup

struct MlaShared {
  uint16_t rows[kMlaSplit][kMlaDl];  // 16-byte pieces swizzled per row
  int ids[kMlaSplit];
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

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void mla_decode_mfma(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int Hm, int B,
    int T_max, int W, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ MlaShared sh;
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, ln = lane & 15;
  const int r = blockIdx.y, sp = blockIdx.x, nsplit = gridDim.x;
  const int h = wave * 16 + ln;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const int c_begin = sp * kMlaSplit;

  if (tid < kMlaSplit) {
    const int c = c_begin + tid;
    int id = -1;
    if (c < W) {
      id = token_ids[size_t(r) * W + c];
      if (!bok || id < 0 || id >= T_max) id = -1;
    }
    sh.ids[tid] = id;
  }
  // q_lat of head h as the B operand of the logits: Dl piece kg + 4i at k-step i
  bf16x8 qop[16];
  {
    const uint16_t* qs = q_lat + (size_t(r) * Hm + h) * kMlaDl;
#pragma unroll
    for (int i = 0; i < 16; ++i) qop[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + (kg + 4 * i) * 8));
  }
  __syncthreads();
  // gather: every load of this thread is issued before any LDS store (masked
  // ids read a valid row and store zeros)
  constexpr int kPieces = kMlaSplit * (kMlaDl / 8);
  constexpr int kPer = (kPieces + NT - 1) / NT;
  {
    u32x4 v[kPer];
    const size_t seq_base = size_t(bok ? b : 0) * T_max;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = min(tid + k * NT, kPieces - 1), t = u >> 6, c = u & 63;
      const int id = sh.ids[t];
      v[k] = *reinterpret_cast<const u32x4*>(kv + (seq_base + (id >= 0 ? id : 0)) * kMlaDl + c * 8);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = tid + k * NT, t = u >> 6, c = u & 63;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (u < kPieces) *reinterpret_cast<u32x4*>(&sh.rows[t][(c ^ row_swz(t)) * 8]) = sh.ids[t] >= 0 ? v[k] : z;
    }
  }
  __syncthreads();

  // logits, 4 blocks of 16 tokens
  f32x4 sacc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int t = blk_token(mb, ln);
    const int sw = row_swz(t);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.rows[t][((kg + 4 * i) ^ sw) * 8]));
      sacc[mb] = mfma16x16x32(a, qop[i], sacc[mb]);
    }
  }
  // lane (kg, ln): head h, tokens 32ks + 8kg + e with e = 4*(mb & 1) + j, ks = mb >> 1
  float x[16];
  float m = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 32 * (mb >> 1) + 8 * kg + 4 * (mb & 1) + j;
      x[4 * mb + j] = sh.ids[t] >= 0 ? sacc[mb][j] * scale_log2 : -INFINITY;
      m = fmaxf(m, x[4 * mb + j]);
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
      const float p0 = exp2f(x[8 * ks + e] - m_use), p1 = exp2f(x[8 * ks + e + 1] - m_use);
      l += p0 + p1;
      pk[ks][e >> 1] = uint32_t(f2bf(p0)) | (uint32_t(f2bf(p1)) << 16);
    }
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  const bf16x8 pb0 = as_bf16x8(u32x4{pk[0][0], pk[0][1], pk[0][2], pk[0][3]});
  const bf16x8 pb1 = as_bf16x8(u32x4{pk[1][0], pk[1][1], pk[1][2], pk[1][3]});

  // O^T[dl, head] += kv^T[dl, tokens] . P^T[tokens, head]
  f32x4 o[32];
#pragma unroll
  for (int blk = 0; blk < 32; ++blk) {
    const int d = blk * 16 + ln;
    const int c = d >> 3, off = d & 7;
    o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int t0 = 32 * ks + 8 * kg + e, t1 = t0 + 1;
        const uint32_t lo = sh.rows[t0][((c ^ row_swz(t0)) << 3) + off];
        const uint32_t hi = sh.rows[t1][((c ^ row_swz(t1)) << 3) + off];
        wv[e >> 1] = lo | (hi << 16);
      }
      o[blk] = mfma16x16x32(as_bf16x8(u32x4{wv[0], wv[1], wv[2], wv[3]}), ks ? pb1 : pb0, o[blk]);
    }
  }

  // o[blk][j] = sum_t p_t kv[t][dl = 16*blk + 4*kg + j] for head h
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const float lse_v = l > 0.f ? (m_use + log2f(l)) * 0.69314718055994531f : -INFINITY;
  if (nsplit == 1) {
    uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + 4 * kg;
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      u32x2 pkd;
      pkd[0] = uint32_t(f2bf(o[blk][0] * inv)) | (uint32_t(f2bf(o[blk][1] * inv)) << 16);
      pkd[1] = uint32_t(f2bf(o[blk][2] * inv)) | (uint32_t(f2bf(o[blk][3] * inv)) << 16);
      *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
    }
    if (kg == 0 && lse) lse[size_t(r) * Hm + h] = lse_v;
  } else {
    float* dst = part_o + ((size_t(r) * nsplit + sp) * Hm + h) * kMlaDl + 4 * kg;
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) *reinterpret_cast<f32x4*>(dst + blk * 16) = o[blk] * inv;
    if (kg == 0) part_lse[(size_t(r) * nsplit + sp) * Hm + h] = lse_v;
  }
}

// Merge split partials: out = sum_s e^{lse_s} O_s / sum_s e^{lse_s}.  The
// split weights are formed once in LDS; the partial loads are independent.
constexpr int kMaxSplit = 256;
__global__ __launch_bounds__(128) void mla_combine(const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse, int nsplit,
                                                   int Hm, uint16_t* __restrict__ out,
                                                   float* __restrict__ lse) {
  __shared__ float wgt[kMaxSplit];
  __shared__ float red[2];
  const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float lv = -INFINITY;
  for (int s = tid; s < nsplit; s += 128) {
    lv = part_lse[(size_t(r) * nsplit + s) * Hm + h];
    wgt[s] = lv;
  }
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += 128) M = fmaxf(M, wgt[s]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  float ws = 0.f;
  for (int s = tid; s < nsplit; s += 128) {
    const float e = M == -INFINITY ? 0.f : expf(wgt[s] - M);
    wgt[s] = e;
    ws += e;
  }
  ws = wave_sum(ws);
  __syncthreads();
  if (lane == 0) red[wave] = ws;
  __syncthreads();
  ws = red[0] + red[1];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* src = part_o + (size_t(r) * nsplit * Hm + h) * kMlaDl + 4 * tid;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + size_t(s) * Hm * kMlaDl);
    acc += wgt[s] * v;
  }
  const float inv = ws > 0.f ? 1.0f / ws : 0.f;
  u32x2 pk;
  pk[0] = uint32_t(f2bf(acc[0] * inv)) | (uint32_t(f2bf(acc[1] * inv)) << 16);
  pk[1] = uint32_t(f2bf(acc[2] * inv)) | (uint32_t(f2bf(acc[3] * inv)) << 16);
  *reinterpret_cast<u32x2*>(out + (size_t(r) * Hm + h) * kMlaDl + 4 * tid) = pk;
  if (tid == 0 && lse) lse[size_t(r) * Hm + h] = ws > 0.f ? M + logf(ws) : -INFINITY;
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
  int nsplit;
};

static MlaPlan mla_plan(int Q, int Hm, int Dl, int W, int dtype) {
  MlaPlan pl{false, 1};
  if (!(dtype == DSA_BF16 && Dl == kMlaDl && Hm % 16 == 0 && Hm <= 128)) return pl;
  pl.mfma = true;
  pl.nsplit = (W + kMlaSplit - 1) / kMlaSplit;
  return pl;
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace dsa

using namespace dsa;

extern "C" size_t dsa_sparse_mla_workspace_bytes(int Q, int Hm, int Dl, int W, int dtype) {
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || W <= 0) return 0;
  const MlaPlan pl = mla_plan(Q, Hm, Dl, W, dtype);
  if (!pl.mfma || pl.nsplit == 1) return 0;
  return align256(size_t(Q) * pl.nsplit * Hm * Dl * sizeof(float)) +
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
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (pl.nsplit > 1) {
    part_o = static_cast<float*>(workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(size_t(Q) * pl.nsplit * Hm * Dl * sizeof(float)));
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  dim3 grid(pl.nsplit, Q);
  const int nw = Hm / 16;
#define DSA_MLA(NW)                                                                               \
  hipLaunchKernelGGL(mla_decode_mfma<NW>, grid, dim3(NW * 64), 0, s, (const uint16_t*)q_lat,     \
                     (const uint16_t*)kv, row_seq, token_ids, Hm, B, T_max, W, scale_log2,        \
                     (uint16_t*)out, lse, part_o, part_lse)
  switch (nw) {
    case 1: DSA_MLA(1); break;
    case 2: DSA_MLA(2); break;
    case 3: DSA_MLA(3); break;
    case 4: DSA_MLA(4); break;
    case 5: DSA_MLA(5); break;
    case 6: DSA_MLA(6); break;
    case 7: DSA_MLA(7); break;
    default: DSA_MLA(8); break;
  }
#undef DSA_MLA
  int st = launch_status();
  if (st || pl.nsplit == 1) return st;
  hipLaunchKernelGGL(mla_combine, dim3(Hm, Q), dim3(kMlaDl / 4), 0, s, part_o, part_lse,
                     pl.nsplit, Hm, (uint16_t*)out, lse);
  return launch_status();
}
