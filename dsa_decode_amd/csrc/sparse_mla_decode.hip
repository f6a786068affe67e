// sparse_mla_decode: absorbed NoPE MLA decode restricted to the selected
// tokens (page "Module glm5next_dsa", "Shape of the pipeline" and "Traps
// carried from Slice 8": NoPE, the rotary slice is zero-width; page "Module
// tp", "Traps this module encodes": one shared latent per token, no head axis).
//
// Absorbed MLA attends with the latent as both key and value: for each head,
// logits sm_scale * <q_lat_h, kv_j> over the listed tokens j, softmax, and the
// softmax-weighted sum of the same kv_j rows.
//
// MFMA path (bf16, Dl = 512, Hm a multiple of 16), few rows (decode).  A
// workgroup of 8 waves handles one row, one group of 16 heads and a slice of
// 128 ids of the row's list, as two halves of 64 ids (waves 0..3 and 4..7):
//   - the ids are requested first, the gather follows as soon as they are in:
//     each half's 64 listed latent rows (64 KiB) go straight into LDS by the
//     load-to-LDS path, one 1 KiB row per instruction (16 bytes per lane, the
//     row swizzle applied through the source addresses); the 16 heads' q_lat
//     rows follow into LDS once per workgroup (padded rows, so that the
//     fragment reads of 16 heads hit distinct banks);
//   - wave w of a half forms the logits of its 16 tokens for the 16 heads
//     over the full latent width on the matrix cores (kv rows and q^T from
//     LDS, every fragment read issued before the first MFMA), so no partial
//     logits cross waves;
//   - softmax: each wave takes its own maximum per head and forms P relative
//     to it; P (bf16) and the per-wave maxima and sums go through LDS, and the
//     value contraction scales the P operand by 2^(m_wave - m_half): no
//     barrier waits for a maximum before P is formed (one barrier publishes P);
//   - wave w of a half accumulates latent quarter w of O^T[dl, head] = kv^T .
//     P^T over its half's 64 tokens, reading kv^T with the transposing LDS
//     reads;
//   - the halves are merged in LDS (half 1 parks its unnormalised O, maximum
//     and sum in its free row buffer; half 0 rescales both to the common
//     maximum), so one partial per 128 ids leaves the workgroup.
// The swizzle spreads both LDS read patterns over the banks.  ~150 KiB of LDS:
// one workgroup per CU.  The head groups of one (row, slice) read the same
// latent rows; their workgroup ids are spaced by a multiple of 8 so that they
// share an XCD and its L2.  Slices write normalised partial outputs, rounded
// to bf16 (in the lanes' order: 512 B per store instruction), and their fp32
// log-sum-exp; a combine launch merges them in fp32.  The gather is the HBM
// traffic (1 KiB per selected token).
#include <mutex>

#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kMlaDl = 512;
constexpr int kMlaSplit = 64;   // ids per workgroup
constexpr int kMlaThreads = 256;

struct alignas(16) MlaShared {
  uint16_t rows[kMlaSplit][kMlaDl];  // latent rows, 16-byte pieces swizzled per row (64 KiB)
  struct {                           // the softmax exchange
    uint16_t p[16][kMlaSplit];       // P[head][token] relative to its wave's maximum, bf16
                                     // (8-token groups swizzled per head, mla_pidx)
    float m[16][4];                  // per head: each wave's maximum (log2 domain)
    float l[16][4];                  // per head: each wave's sum of P
  } x;
};

// LDS banks, as measured on gfx950 with the bank-conflict counter: a 16-byte
// read is served in passes of 16 lanes over 256 bytes (16 slots of 16 bytes),
// each 32-lane half of the wave in two passes that take its lane quads 0, 3,
// 5, 6 and 1, 2, 4, 7 (the parity of lane bits 2..4); 8-byte reads, including
// the transposing ones, in passes of 32 lanes over 256 bytes; writes in passes
// over 128 bytes (8 lanes for 16 bytes, 16 lanes for 8 bytes).  A pass costs
// one extra cycle for every further distinct address in the same slot.
//
// Piece c (16 bytes) of token row t sits at piece c ^ mla_swz(t), with
// mla_swz(t) = rotl4(t) ^ (t & 8) on the low four bits of t.  The logits reads
// (lane (ln, kg) reads piece 4k + kg of row 16w + ln) then fill every slot of
// each 16-lane pass once, and so do the transposing reads of the value
// contraction (rows 8g .. 8g+3 and 8g+8 .. 8g+11 by two adjacent pieces in a
// 32-lane pass): no bank conflicts.  (A swizzle that spreads 16 consecutive
// rows over the slots is not enough: the pass takes lanes of two lane groups.)
__device__ __forceinline__ int mla_swz(int t) { return ((((t << 1) & 14) | ((t >> 3) & 1)) ^ (t & 8)); }

// The softmax weights P of one head: 64 tokens (128 bytes); the 8-token group
// g of head h sits at group g ^ mla_pswz(h), so the 16-byte reads of 16 heads
// (lane (ln, kg) reads group 4ks + kg of head ln) fill every slot of a pass.
__device__ __forceinline__ int mla_pswz(int h) { return (h & 1) | ((h & 2) << 1) | ((h & 4) >> 1); }
// element index of token tok of head h in its P row
__device__ __forceinline__ int mla_pidx(int h, int tok) { return ((((tok >> 3) ^ mla_pswz(h)) << 3) | (tok & 7)); }

// Maximum and sum of v over the four lane groups (kg = 0..3) of the lanes
// that share ln, in every lane: the swaps of 16- and 32-lane rows (the same
// register as both operands, so the two results hold the partner rows'
// values), without a round trip through LDS.
__device__ __forceinline__ float lane_groups_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_groups_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4 16-bit elements read by lanes 4e + (i >> 2), e = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Eight transposing 16-bit LDS reads (as lds_read_tr16, at LDS byte
// addresses a[i]) issued together and waited for within the statement (a
// load written in asm must not be left in flight when the statement ends).
// The compiler does not see these as reads of LDS that a load-to-LDS may be
// writing, so it places no wait for such loads before them.
__device__ __forceinline__ void lds_read_tr16_x8(u32x2 (&v)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// Transposing LDS read of 8-bit elements: within each group of 16 lanes, lane
// i receives byte (i & 7) of the 8-byte words read by lanes 2e + (i >> 3),
// e = 0..7 (so lanes 2e, 2e+1 reading row e's bytes 0..7 and 8..15 of a
// 16-column block give lane i column i of rows 0..7).
typedef int i32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Eight OCP FP8 E4M3 codes (byte i of the pair = element i) -> eight bf16,
// exactly (every E4M3 value is a bf16 value): one scaled convert per two codes.
__device__ __forceinline__ u32x4 widen_fp8x8(u32x2 c) {
  u32x4 v;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    v[2 * h2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[h2], 1.0f, false));
    v[2 * h2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[h2], 1.0f, true));
  }
  return v;
}

// offset (in elements) of partial-output element (head group hg, lane, dl) of a
// (row, split): [hg][dq][blk][lane][j], dl = 128 dq + 16 blk + 4 kg + j
__device__ __forceinline__ size_t part_off(size_t rs, int HG, int hg, int dq, int blk, int lane) {
  return ((((rs * HG + hg) * 4 + dq) * 8 + blk) * 64 + lane) * 4;
}

// Where the latent rows live.  kKvRows: the cache [B, T_max, Dl] bf16 (token t
// of sequence b is row b*T_max + t).  kKvPaged: bf16 pages [num_pages,
// page_size, Dl] behind a page table [B, max_pages] (token t of sequence b is
// row t % page_size of page block_table[b, t / page_size]).  kKvPagedFp8: the
// same pages holding OCP FP8 E4M3 codes with one fp32 scale per row; the codes
// go into LDS as they are (half the bytes of a bf16 row) and are widened to
// bf16 exactly as the fragments are read, and the row's scale multiplies the
// token's logit and its softmax weight in the value sum.
enum KvLayout { kKvRows = 0, kKvPaged = 1, kKvPagedFp8 = 2 };

struct KvPages {
  const int32_t* block_table;
  const float* scale;
  int max_pages, page_size, num_pages;
};

// Few rows (decode): one workgroup of 8 waves per (row, group of 16 heads,
// slice of 128 ids).  The two halves of the slice (waves 0..3: ids 0..63,
// waves 4..7: ids 64..127) each take the steps of mla_decode_mfma on their own
// row buffer, and the halves are merged in LDS before the one partial of the
// slice is written: half the partials of 64-id slices, so half the bytes the
// combine reads.  The 16 heads' q_lat rows go into LDS once per workgroup
// (load-to-LDS, one 1 KiB row per instruction, rows padded so that the
// fragment reads of 16 heads hit distinct banks) instead of once per wave
// into registers: the per-wave q loads were 4x the gathered bytes and held
// back the id loads and the gather behind them.  The ids are requested first,
// then q, then the gather as soon as the ids are in.
constexpr int kMla2Ids = 2 * kMlaSplit;  // ids per workgroup
constexpr int kMla2Threads = 512;

struct alignas(16) Mla2Shared {
  uint16_t rows[2][kMlaSplit][kMlaDl];  // each half's latent rows (swizzled as in MlaShared), 128 KiB
  uint16_t q[16][kMlaDl];               // the 16 heads' q_lat rows (pieces swizzled as the rows)
  struct {
    uint16_t p[16][kMlaSplit];
    float m[16][4];
    float l[16][4];
  } x[2];                               // each half's softmax exchange
  float mh[16], lh[16];                 // half 1's row maximum and sum per head, for the merge
};

template <int KV>
__global__ __launch_bounds__(kMla2Threads) void mla_decode_mfma(
    const uint16_t* __restrict__ q_lat, const void* __restrict__ kv_v, KvPages pages,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int Hm, int B,
    int T_max, int W, int nsplit, int ns8, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse) {
  const uint16_t* __restrict__ kv = static_cast<const uint16_t*>(kv_v);
  __shared__ Mla2Shared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = w8 >> 2, w = w8 & 3;
  const int kg = lane >> 4, ln = lane & 15;
  const int HG = Hm >> 4;
  const int hg = blockIdx.x / ns8, sp = blockIdx.x % ns8;
  if (sp >= nsplit) return;  // padding workgroups (uniform exit)
  const int r = blockIdx.y;
  const int h = hg * 16 + ln;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const size_t seq_base = size_t(bok ? b : 0) * T_max;

  // ids of this wave's 16 tokens (lanes 0..15), -1 when absent or out of range
  int raw = -1;
  const int c = sp * kMla2Ids + kMlaSplit * half + 16 * w + lane;
  if (lane < 16 && c < W) raw = token_ids[size_t(r) * W + c];
  // the token's row in the cache (for a paged cache, its physical row, and
  // for fp8 pages its scale); -1 when absent or out of range
  int myid = -1;
  float mysc = 1.f;
  if (lane < 16) {
    if (KV == kKvRows) {
      myid = (bok && raw >= 0 && raw < T_max) ? raw : -1;
    } else if (bok && raw >= 0 && raw / pages.page_size < pages.max_pages) {
      const int pg = pages.block_table[size_t(b) * pages.max_pages + raw / pages.page_size];
      if (pg >= 0 && pg < pages.num_pages) {
        myid = pg * pages.page_size + raw % pages.page_size;
        if (KV == kKvPagedFp8) mysc = pages.scale[myid];
      }
    }
  }
  uint16_t (*rows)[kMlaDl] = sh.rows[half];
  // fp8 rows: 512 bytes of codes each, the half's 64 rows in the first 32 KiB
  // of its row buffer; the 16-byte piece c of row t sits at piece c ^ (t & 15)
  uint8_t (*rows8)[kMlaDl] = reinterpret_cast<uint8_t (*)[kMlaDl]>(&sh.rows[half][0][0]);
  uint32_t vmask = 0;
  if constexpr (KV != kKvPagedFp8) {
    // one row per instruction: lane i fills piece position i with piece
    // i ^ swz of the token's row; absent ids give a zero row
    const size_t base = KV == kKvRows ? seq_base : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = __builtin_amdgcn_readlane(myid, i);
      const int t = 16 * w + i;
      if (id >= 0) {
        vmask |= 1u << i;
        const uint16_t* src = kv + (base + size_t(id)) * kMlaDl + 8 * (lane ^ mla_swz(t));
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(&rows[t][0]), 16, 0, 0);
      } else {
        *reinterpret_cast<u32x4*>(&rows[t][8 * lane]) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  } else {
    // two rows per instruction (lanes 0..31: row 2i, lanes 32..63: row 2i+1),
    // codes straight into LDS; absent ids give zero rows.  The codes are
    // widened to bf16 when the fragments are read (an E4M3 value is exactly a
    // bf16 value, so nothing is rounded), and the row's scale is applied to
    // the token's logits and to its P instead of to its 512 values
    // (logit_j = scale_j <q, codes_j>, sum_j p_j v_j = sum_j (p_j scale_j) codes_j)
    const uint8_t* kv8 = static_cast<const uint8_t*>(kv_v);
    const int hl = lane >> 5, pl = lane & 31;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id0 = __builtin_amdgcn_readlane(myid, 2 * i), id1 = __builtin_amdgcn_readlane(myid, 2 * i + 1);
      vmask |= (id0 >= 0 ? 1u : 0u) << (2 * i);
      vmask |= (id1 >= 0 ? 1u : 0u) << (2 * i + 1);
      const int id = hl ? id1 : id0;
      const int t = 16 * w + 2 * i + hl;
      if (id >= 0) {
        const uint8_t* src = kv8 + size_t(id) * kMlaDl + 16 * (pl ^ (t & 15));
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(&rows8[16 * w + 2 * i][0]),
                                         16, 0, 0);
      } else {
        *reinterpret_cast<u32x4*>(&rows8[t][16 * pl]) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // q_lat rows of heads 2 w8, 2 w8 + 1 into LDS, after the gather (q is needed
  // only after the barrier; issued before the gather it delayed the gather)
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int hh = 2 * w8 + e;
    __builtin_amdgcn_global_load_lds(q_lat + (size_t(r) * Hm + hg * 16 + hh) * kMlaDl + 8 * (lane ^ mla_swz(hh)),
                                     (__attribute__((address_space(3))) void*)(&sh.q[hh][0]), 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave's rows and the q rows are in LDS

  // logits of tokens 16w + 4kg + j (j < 4) of this half for head ln, full
  // latent width (A = kv rows, B = q^T fragments, both from LDS)
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  {
    // every fragment read is issued before the first MFMA (one LDS round trip)
    const int t = 16 * w + ln, sw = mla_swz(t), swq = mla_swz(ln);
    u32x4 fa[16], fb[16];
    if constexpr (KV != kKvPagedFp8) {
#pragma unroll
      for (int k = 0; k < 16; ++k) fa[k] = *reinterpret_cast<const u32x4*>(&rows[t][((4 * k + kg) ^ sw) * 8]);
    } else {
      // latent columns 32k + 8kg .. +7 of row t: half of piece 2k + (kg >> 1)
      u32x2 c8[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        c8[k] = *reinterpret_cast<const u32x2*>(&rows8[t][(((2 * k + (kg >> 1)) ^ (t & 15)) << 4) + ((kg & 1) << 3)]);
#pragma unroll
      for (int k = 0; k < 16; ++k) fa[k] = widen_fp8x8(c8[k]);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) fb[k] = *reinterpret_cast<const u32x4*>(&sh.q[ln][((4 * k + kg) ^ swq) * 8]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      acc0 = mfma16x16x32(as_bf16x8(fa[k]), as_bf16x8(fb[k]), acc0);
      acc1 = mfma16x16x32(as_bf16x8(fa[k + 1]), as_bf16x8(fb[k + 1]), acc1);
    }
  }
  // fp8 rows: the scale of token 4 kg + j of the wave (its lane < 16 holds it)
  float tsc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tsc[j] = KV == kKvPagedFp8 ? __shfl(mysc, 4 * kg + j, kWave) : 1.f;
  float x[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lg = KV == kKvPagedFp8 ? (acc0[j] + acc1[j]) * tsc[j] : acc0[j] + acc1[j];
    x[j] = (vmask >> (4 * kg + j)) & 1u ? lg * scale_log2 : -INFINITY;
    m = fmaxf(m, x[j]);
  }
  m = lane_groups_max(m);
  const float m_use = m == -INFINITY ? 0.f : m;
  float p[4], l = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
    l += p[j];
  }
  l = lane_groups_sum(l);
  auto& X = sh.x[half];
  // the value operand: P, times the token's scale for fp8 rows (l stays the
  // sum of the unscaled P)
  if (KV == kKvPagedFp8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] *= tsc[j];
  }
  *reinterpret_cast<u32x2*>(&X.p[ln][mla_pidx(ln, 16 * w + 4 * kg)]) = u32x2{pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
  if (kg == 0) {
    X.m[ln][w] = m_use;
    X.l[ln][w] = l;
  }
  __syncthreads();  // P, the maxima and the sums of both halves published

  const f32x4 mv = *reinterpret_cast<const f32x4*>(&X.m[ln][0]);
  const f32x4 lv = *reinterpret_cast<const f32x4*>(&X.l[ln][0]);
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) M = fmaxf(M, lv[v] > 0.f ? mv[v] : -INFINITY);
  const float M_use = M == -INFINITY ? 0.f : M;
  float fv[4];
  l = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    fv[v] = lv[v] > 0.f ? __builtin_amdgcn_exp2f(mv[v] - M_use) : 0.f;
    l = fmaf(fv[v], lv[v], l);
  }
  bf16x8 pb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const u32x4 rw = *reinterpret_cast<const u32x4*>(&X.p[ln][mla_pidx(ln, 32 * ks + 8 * kg)]);
    const float f = fv[2 * ks + (kg >> 1)];
    u32x4 scv;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      scv[e] = pack2bf(__uint_as_float(rw[e] << 16) * f, __uint_as_float(rw[e] & 0xffff0000u) * f);
    pb[ks] = as_bf16x8(scv);
  }
  f32x4 o[8];
  {
    // every transposing read is issued before the first MFMA
    u32x2 tl[8][2], th[8][2];
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (KV != kKvPagedFp8) {
          const int col = 128 * w + 16 * blk + 4 * (ln & 3);
          const int pc = col >> 3, off = col & 7;
          const int t0 = 32 * ks + 8 * kg + (ln >> 2), t1 = t0 + 4;
          tl[blk][ks] = lds_read_tr16(&rows[t0][((pc ^ mla_swz(t0)) << 3) + off]);
          th[blk][ks] = lds_read_tr16(&rows[t1][((pc ^ mla_swz(t1)) << 3) + off]);
        } else {
          // codes of tokens 32ks + 8kg .. +7 at latent column 128w + 16blk + ln:
          // lane 2e + j reads 8 codes of token 32ks + 8kg + e from piece 8w + blk
          const int t0 = 32 * ks + 8 * kg + (ln >> 1);
          tl[blk][ks] = lds_read_tr8(&rows8[t0][(((8 * w + blk) ^ (t0 & 15)) << 4) + ((ln & 1) << 3)]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 av = KV != kKvPagedFp8 ? u32x4{tl[blk][ks][0], tl[blk][ks][1], th[blk][ks][0], th[blk][ks][1]}
                                           : widen_fp8x8(tl[blk][ks]);
        a = mfma16x16x32(as_bf16x8(av), pb[ks], a);
      }
      o[blk] = a;
    }
  }
  // merge the halves: half 1 parks its unnormalised O (relative to its row
  // maximum), maximum and sum in LDS (its row buffer is free once every wave
  // is past the values), half 0 rescales both to the common maximum
  const float Mh = l > 0.f ? M_use : -INFINITY;
  __syncthreads();  // every wave is done reading the rows
  f32x4* park = reinterpret_cast<f32x4*>(&sh.rows[1][0][0]) + (w * 8) * 64 + lane;
  if (half == 1) {
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) park[blk * 64] = o[blk];
    if (w == 0 && kg == 0) {
      sh.mh[ln] = Mh;
      sh.lh[ln] = l;
    }
  }
  __syncthreads();
  if (half == 1) return;
  const float M1 = sh.mh[ln], l1 = sh.lh[ln];
  const float Mt = fmaxf(Mh, M1);
  const float Mt_use = Mt == -INFINITY ? 0.f : Mt;
  const float f0 = l > 0.f ? __builtin_amdgcn_exp2f(M_use - Mt_use) : 0.f;
  const float f1 = l1 > 0.f ? __builtin_amdgcn_exp2f(M1 - Mt_use) : 0.f;
  const float lt = fmaf(l, f0, l1 * f1);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse_v = lt > 0.f ? (Mt_use + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f : -INFINITY;
  const float g0 = f0 * inv, g1 = f1 * inv;
  if (nsplit == 1) {
    uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + w * 128 + 4 * kg;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const f32x4 o1 = park[blk * 64];
      u32x2 pkd;
      pkd[0] = pack2bf(o[blk][0] * g0 + o1[0] * g1, o[blk][1] * g0 + o1[1] * g1);
      pkd[1] = pack2bf(o[blk][2] * g0 + o1[2] * g1, o[blk][3] * g0 + o1[3] * g1);
      *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
    }
    if (w == 0 && kg == 0 && lse) lse[size_t(r) * Hm + h] = lse_v;
  } else {
    const size_t rs = size_t(r) * nsplit + sp;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const f32x4 o1 = park[blk * 64];
      u32x2 pkd;
      pkd[0] = pack2bf(o[blk][0] * g0 + o1[0] * g1, o[blk][1] * g0 + o1[1] * g1);
      pkd[1] = pack2bf(o[blk][2] * g0 + o1[2] * g1, o[blk][3] * g0 + o1[3] * g1);
      __builtin_nontemporal_store(pkd, reinterpret_cast<u32x2*>(part_o + part_off(rs, HG, hg, w, blk, lane)));
    }
    if (w == 0 && kg == 0) part_lse[rs * Hm + h] = lse_v;
  }
}

// Many-rows path (prefill chunks): one workgroup per (row, group of 16 heads)
// runs over all of the row's ids, 64 at a time, with an online softmax, so no
// partial output leaves the workgroup and no combine launch follows.  Each
// 64-id block takes the decode kernel's steps (gather into LDS, full-width
// logits of each wave's 16 tokens, per-wave maxima, the value contraction of
// latent quarter w); the running maximum M, sum l and the O^T accumulators
// carry from block to block, rescaled by 2^(M_old - M_new) as the maximum
// grows.  Workgroup ids put the head groups of a row on one XCD (ids congruent
// mod 8), so a gathered latent row is fetched into that L2 once and read there
// by the other groups.  Used when there are enough (row, head group) pairs to
// fill the chip without splitting the ids.
constexpr int kMlaRowsMinWgs = 1024;

__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_rows_mfma(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int Q, int Hm, int B,
    int T_max, int W, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ MlaShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, ln = lane & 15;
  const int HG = Hm >> 4;
  const int rest = blockIdx.x >> 3;
  const int hg = rest % HG;
  const int r = (rest / HG) * 8 + (blockIdx.x & 7);
  if (r >= Q) return;  // padding workgroups (uniform exit)
  const int h = hg * 16 + ln;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const size_t seq_base = size_t(bok ? b : 0) * T_max;
  const int32_t* ids_row = token_ids + size_t(r) * W;
  const int nblk = (W + kMlaSplit - 1) / kMlaSplit;

  // ids of this wave's 16 tokens of block blk (lanes 0..15), -1 when absent
  auto load_id = [&](int blk) {
    int id = -1;
    if (lane < 16) {
      const int c = blk * kMlaSplit + 16 * w + lane;
      if (c < W) {
        const int v = ids_row[c];
        id = (bok && v >= 0 && v < T_max) ? v : -1;
      }
    }
    return id;
  };
  int myid = load_id(0);
  // q_lat of the 16 heads in registers, matrix-core B layout (as in the decode kernel)
  u32x4 qv[16];
  {
    const uint16_t* qrow = q_lat + (size_t(r) * Hm + h) * kMlaDl + 8 * kg;
#pragma unroll
    for (int j = 0; j < 16; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qrow + 32 * j);
  }
  float M_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) o[blk] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ib = 0; ib < nblk; ++ib) {
    // gather the block's 64 rows (wave w: ids 16w .. 16w+15)
    uint32_t vmask = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = __builtin_amdgcn_readlane(myid, i);
      const int t = 16 * w + i;
      if (id >= 0) {
        vmask |= 1u << i;
        const uint16_t* src = kv + (seq_base + size_t(id)) * kMlaDl + 8 * (lane ^ mla_swz(t));
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(&sh.rows[t][0]), 16, 0, 0);
      } else {
        *reinterpret_cast<u32x4*>(&sh.rows[t][8 * lane]) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int next_id = ib + 1 < nblk ? load_id(ib + 1) : -1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave's rows are in LDS

    // logits of tokens 16w + 4kg + j for head ln over the full latent width
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    {
      const int t = 16 * w + ln, sw = mla_swz(t);
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.rows[t][((4 * k + kg) ^ sw) * 8]));
        const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.rows[t][((4 * k + 4 + kg) ^ sw) * 8]));
        acc0 = mfma16x16x32(a0, as_bf16x8(qv[k]), acc0);
        acc1 = mfma16x16x32(a1, as_bf16x8(qv[k + 1]), acc1);
      }
    }
    // the wave's maximum per head over its 16 tokens and P relative to it
    float x[4];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = (vmask >> (4 * kg + j)) & 1u ? (acc0[j] + acc1[j]) * scale_log2 : -INFINITY;
      m = fmaxf(m, x[j]);
    }
    m = lane_groups_max(m);
    const float m_use = m == -INFINITY ? 0.f : m;
    float p[4], l = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
      l += p[j];
    }
    l = lane_groups_sum(l);
    *reinterpret_cast<u32x2*>(&sh.x.p[ln][mla_pidx(ln, 16 * w + 4 * kg)]) =
        u32x2{pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
    if (kg == 0) {
      sh.x.m[ln][w] = m_use;
      sh.x.l[ln][w] = l;
    }
    __syncthreads();  // P, the maxima and the sums published

    // online merge: new running maximum, rescale of what is accumulated, and
    // the factor 2^(m_v - M) of each wave's tokens
    const f32x4 mv = *reinterpret_cast<const f32x4*>(&sh.x.m[ln][0]);
    const f32x4 lv = *reinterpret_cast<const f32x4*>(&sh.x.l[ln][0]);
    float Mb = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) Mb = fmaxf(Mb, lv[v] > 0.f ? mv[v] : -INFINITY);
    const float M_new = fmaxf(M_run, Mb);
    const float M_use = M_new == -INFINITY ? 0.f : M_new;
    const float alpha = M_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M_run - M_use);
    float fv[4];
    float lb = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      fv[v] = lv[v] > 0.f ? __builtin_amdgcn_exp2f(mv[v] - M_use) : 0.f;
      lb = fmaf(fv[v], lv[v], lb);
    }
    l_run = fmaf(l_run, alpha, lb);
    M_run = M_new;
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(&sh.x.p[ln][mla_pidx(ln, 32 * ks + 8 * kg)]);
      const float f = fv[2 * ks + (kg >> 1)];
      u32x4 sc;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc[e] = pack2bf(__uint_as_float(raw[e] << 16) * f, __uint_as_float(raw[e] & 0xffff0000u) * f);
      pb[ks] = as_bf16x8(sc);
    }
    // O^T over latent quarter w, accumulated on top of the rescaled running sum
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int col = 128 * w + 16 * blk + 4 * (ln & 3);
      const int pc = col >> 3, off = col & 7;
      f32x4 a = o[blk] * alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int t0 = 32 * ks + 8 * kg + (ln >> 2), t1 = t0 + 4;
        const u32x2 lo = lds_read_tr16(&sh.rows[t0][((pc ^ mla_swz(t0)) << 3) + off]);
        const u32x2 hi = lds_read_tr16(&sh.rows[t1][((pc ^ mla_swz(t1)) << 3) + off]);
        a = mfma16x16x32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[ks], a);
      }
      o[blk] = a;
    }
    myid = next_id;
    __syncthreads();  // rows and P are free for the next block
  }

  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + w * 128 + 4 * kg;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    u32x2 pkd;
    pkd[0] = pack2bf(o[blk][0] * inv, o[blk][1] * inv);
    pkd[1] = pack2bf(o[blk][2] * inv, o[blk][3] * inv);
    *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
  }
  if (w == 0 && kg == 0 && lse)
    lse[size_t(r) * Hm + h] = l_run > 0.f ? (M_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
}

// Many-rows path for 64 heads: one workgroup per row holds all 64 heads, so
// each gathered latent row lands in LDS once for every head of the row.  Eight
// waves, two per SIMD (240 registers: each wave holds 64 accumulators, not the
// 128 a latent quarter would need).  Wave w forms the
// logits of heads 16 (w & 3) .. +15 over token half w >> 2 of each 64-id block
// (q^T of its 16 heads in registers), and accumulates latent eighth w of O^T
// for all 64 heads (64 accumulators per lane instead of 128).  The two token
// halves of a head meet in LDS twice per block: first their maxima, so that
// each logits wave forms P against the head's new running maximum M_new (the
// running maximum and both halves' maxima), then P and the halves' sums;
// every wave then forms, for each of the 64 heads, the same M_new from the
// same LDS words, rescales its accumulators by 2^(M_old - M_new) and reads P
// as it is.  (Forming P against each half's own maximum and scaling it by
// 2^(m_half - M_new) as it was read spared a barrier but cost more vector
// work: 1.91 against 1.72 ms per 4096-row chunk.)  Rows are gathered 8 per
// wave, the next block into the second buffer while this one is computed.
struct alignas(16) Mla64x8Shared {
  uint16_t rows[2][kMlaSplit][kMlaDl];  // latent rows, pieces swizzled by mla_swz
  uint16_t p[64][kMlaSplit];            // P[head][token] relative to its half's maximum (mla_pidx)
  float m[64][2];                       // per head and token half: maximum (log2 domain, 0 if none)
  float l[64][2];                       // per head and token half: sum of P
};

constexpr int kMla8Threads = 512;

__global__ __launch_bounds__(kMla8Threads) __attribute__((amdgpu_waves_per_eu(2))) void mla_rows64w8_mfma(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int Q, int B, int T_max,
    int W, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int Hm = 64;
  __shared__ Mla64x8Shared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, ln = lane & 15;
  const int hgw = w & 3, th = w >> 2;
  const int r = blockIdx.x;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const size_t seq_base = size_t(bok ? b : 0) * T_max;
  const int32_t* ids_row = token_ids + size_t(r) * W;
  const int nblk = (W + kMlaSplit - 1) / kMlaSplit;

  auto load_raw = [&](int blk) {
    const int c = blk * kMlaSplit + lane;
    return (blk < nblk && c < W) ? ids_row[c] : -1;
  };
  auto check_id = [&](int v) { return (bok && v >= 0 && v < T_max) ? v : -1; };
  // rows 8w .. 8w+7 of the block whose ids `ids` holds, into buffer `buf`
  auto gather = [&](int ids, int buf) {
    int lg = lane;
    asm volatile("" : "+v"(lg));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 8 * w + i;
      const int id = __builtin_amdgcn_readlane(ids, t);
      if (id >= 0) {
        const uint16_t* src = kv + (seq_base + size_t(id)) * kMlaDl + 8 * (lg ^ mla_swz(t));
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(&sh.rows[buf][t][0]), 16,
                                         0, 0);
      } else {
        *reinterpret_cast<u32x4*>(&sh.rows[buf][t][8 * lane]) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  int cur_id = check_id(load_raw(0));
  const int hq = 16 * hgw + ln;  // the head whose logits this lane forms
  u32x4 qv[16];
  {
    const uint16_t* qrow = q_lat + (size_t(r) * Hm + hq) * kMlaDl + 8 * kg;
#pragma unroll
    for (int j = 0; j < 16; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qrow + 32 * j);
  }
  gather(cur_id, 0);
  int nxt_raw = load_raw(1);
  float M_run[4], l_run[4];  // heads 16 ht + ln
  f32x4 o[4][4];             // [head tile][16-wide latent block of eighth w]
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    M_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[ht][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int swl = mla_swz(ln);
  int lbase[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) lbase[kk] = ln * kMlaDl + (4 * (kk ^ (swl >> 2)) + (kg ^ (swl & 3))) * 8;
  // element offsets of the transposing reads of the value contraction (rows
  // t0 and t0 + 4 of 16-column block blk; +32 rows for the second 32 tokens)
  int voff[2][4];
  {
    const int t0 = 8 * kg + (ln >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int tt = t0 + 4 * e;
        const int col = 64 * w + 16 * blk + 4 * (ln & 3);
        voff[e][blk] = tt * kMlaDl + (((col >> 3) ^ mla_swz(tt)) << 3) + (col & 7);
      }
  }

  for (int ib = 0; ib < nblk; ++ib) {
    const int cur = ib & 1;
    const uint64_t vmask = __ballot(cur_id >= 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // block ib's rows are in LDS; every wave is done with block ib - 1
    if (ib + 1 < nblk) {
      cur_id = check_id(nxt_raw);
      gather(cur_id, cur ^ 1);
      nxt_raw = load_raw(ib + 2);
    }
    const uint16_t* rows = &sh.rows[cur][0][0];

    // logits of tokens 32 th + 16 t + 4 kg + j (t < 2, j < 4) for head hq
    f32x4 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      bf16x8 a[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        a[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(rows + lbase[k & 3] + (32 * th + 16 * t) * kMlaDl +
                                                         (k >> 2) * 128));
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t] = mfma16x16x32(a[t], as_bf16x8(qv[k]), acc[t]);
    }
    float m = -INFINITY;
    const uint32_t vm = uint32_t(vmask >> (32 * th + 4 * kg));  // bit 16 t + j: token 32 th + 16 t + 4 kg + j
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[t][j] = (vm >> (16 * t + j)) & 1u ? acc[t][j] * scale_log2 : -INFINITY;
        m = fmaxf(m, acc[t][j]);
      }
    m = lane_groups_max(m);
    // the two token halves' maxima meet first, so that P is formed against the
    // block's new running maximum and the value contraction reads it as it is
    // (a factor per half applied as P is read cost more than this barrier)
    if (kg == 0) sh.m[hq][th] = m;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float m_other = sh.m[hq][th ^ 1];
    float Mrun_q = M_run[0];  // running maximum of head hq (a select chain, not a dynamic index)
#pragma unroll
    for (int ht = 1; ht < 4; ++ht) Mrun_q = hgw == ht ? M_run[ht] : Mrun_q;
    const float Mq = fmaxf(Mrun_q, fmaxf(m, m_other));
    const float Mq_use = Mq == -INFINITY ? 0.f : Mq;
    float lh = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(acc[t][j] - Mq_use);
        lh += p[j];
      }
      *reinterpret_cast<u32x2*>(&sh.p[hq][mla_pidx(hq, 32 * th + 16 * t + 4 * kg)]) =
          u32x2{pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
    }
    lh = lane_groups_sum(lh);
    if (kg == 0) sh.l[hq][th] = lh;
    // P and the halves' sums of all 64 heads published: LDS writes done, then
    // the barrier alone (the next block's gather stays in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // each head's new running maximum (the same value its logits wave formed,
    // from the same words) and the rescale of what is accumulated
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int h = 16 * ht + ln;
      const f32x2 mh = *reinterpret_cast<const f32x2*>(&sh.m[h][0]);
      const f32x2 lhv = *reinterpret_cast<const f32x2*>(&sh.l[h][0]);
      const float M_new = fmaxf(M_run[ht], fmaxf(mh[0], mh[1]));
      const float M_use = M_new == -INFINITY ? 0.f : M_new;
      const float alpha = M_run[ht] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M_run[ht] - M_use);
      l_run[ht] = fmaf(l_run[ht], alpha, lhv[0] + lhv[1]);
      M_run[ht] = M_new;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) o[ht][kk] *= alpha;
    }
    // O^T over latent eighth w: A = kv^T (16 dl x 32 tokens, two transposing
    // reads), B = P^T (32 tokens x 16 heads)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
        pb[ht] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.p[16 * ht + ln][mla_pidx(ln, 32 * ks + 8 * kg)]));
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const u32x2 lo = lds_read_tr16(rows + 32 * ks * kMlaDl + voff[0][blk]);
        const u32x2 hi = lds_read_tr16(rows + 32 * ks * kMlaDl + voff[1][blk]);
        const bf16x8 av = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) o[ht][blk] = mfma16x16x32(av, pb[ht], o[ht][blk]);
      }
    }
  }

#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int h = 16 * ht + ln;
    const float inv = l_run[ht] > 0.f ? 1.0f / l_run[ht] : 0.f;
    uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + w * 64 + 4 * kg;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      u32x2 pkd;
      pkd[0] = pack2bf(o[ht][blk][0] * inv, o[ht][blk][1] * inv);
      pkd[1] = pack2bf(o[ht][blk][2] * inv, o[ht][blk][3] * inv);
      *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
    }
    if (w == 0 && kg == 0 && lse)
      lse[size_t(r) * Hm + h] =
          l_run[ht] > 0.f ? (M_run[ht] + __builtin_amdgcn_logf(l_run[ht])) * 0.69314718055994531f : -INFINITY;
  }
}

// Many-rows path for 64 heads as a two-stage pipeline over blocks of 32 ids.
// Waves 0..3 form, for block k, the softmax of heads 16w .. 16w+15 (each
// head's running maximum and sum, P, and the factor that rescales what was
// accumulated) while they issue block k + 1's logits (q^T of the 16 heads in
// registers), so that the matrix cores run under the softmax's chain; waves
// 4..7 meanwhile accumulate latent quarter w - 4 of O^T for all 64 heads over
// block k - 1.  Every SIMD holds one wave of each kind and a block needs a
// single barrier.  The row's checked ids go into LDS first; rows pass through
// four LDS buffers, laid out by latent quarter: the value wave of quarter q,
// once it has read its quarter of block k - 1, gathers its quarter of block
// k + 3 into the same buffer (buffer loads to LDS, four rows' quarters per
// load; an absent id reads past the end of the resource and lands as zeros),
// so no wave waits for another before overwriting, and a counted wait finds
// the block needed next.  Each head's P is formed against a reference that
// moves only when a block's maximum exceeds it by more than 8 (log2 units),
// so P <= 2^8 and the rescale factor is exactly 1 for most blocks; O and the
// sum share the reference, so the result and lse are those of the running
// maximum.  A tile of 16 heads whose factors are all exactly 1 is not
// rescaled.
constexpr int kMlaPipeIds = 32;
constexpr int kMlaPipeThreads = 512;
constexpr int kMlaPipeMaxW = 4096;
constexpr long kMlaPipeMaxT = 1L << 21;  // T_max * 1024 bytes of a sequence's rows below 2^31

struct alignas(16) MlaPipeShared {
  uint16_t rows[4][4][kMlaPipeIds][128];  // [buffer][latent quarter][token][128], 16-byte pieces
                                          // swizzled by mla_swz (128 KiB)
  uint16_t p[2][64][kMlaPipeIds];         // P[head][token] of a block (mla_pidx32), two blocks
  float alpha[2][64];                     // per head: the rescale factor a block brings
  float lfin[64];                         // per head: the final sum
  int32_t ids[kMlaPipeMaxW];              // the row's ids, -1 when absent or out of range
};

// element index of token tok (< 32) of head h in its P row: the 8-token group
// g sits at g ^ ((h >> 2) & 3), so the 16-byte reads of 16 heads (lane (ln,
// kg) reads group kg of head ln) fill every slot of a pass
__device__ __forceinline__ int mla_pidx32(int h, int tok) {
  return (((tok >> 3) ^ ((h >> 2) & 3)) << 3) | (tok & 7);
}

// wait until at most 8 (or none) of this wave's vector-memory loads are in flight
__device__ __forceinline__ void wait_vm_at_most(bool eight) {
  if (eight)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ __launch_bounds__(kMlaPipeThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_rows64_pipe(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ token_ids, int B, int T_max, int W,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int Hm = 64, NI = kMlaPipeIds;
  __shared__ MlaPipeShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, ln = lane & 15;
  const int r = blockIdx.x;
  const int b = row_seq[r];
  const bool bok = b >= 0 && b < B;
  const int32_t* ids_row = token_ids + size_t(r) * W;
  const int nblk = (W + NI - 1) / NI;  // the host launches this path for 64 < W <= kMlaPipeMaxW
  for (int c = tid; c < nblk * NI; c += kMlaPipeThreads) {
    const int v = c < W ? ids_row[c] : -1;
    sh.ids[c] = (bok && v >= 0 && v < T_max) ? v : -1;
  }
  __syncthreads();

  if (w < 4) {
    const int hq = 16 * w + ln;  // the head whose logits this lane forms
    u32x4 qv[16];
    {
      const uint16_t* qrow = q_lat + (size_t(r) * Hm + hq) * kMlaDl + 8 * kg;
#pragma unroll
      for (int j = 0; j < 16; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qrow + 32 * j);
    }
    const int swl = mla_swz(ln);
    int lbase[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) lbase[kk] = ln * 128 + (4 * (kk ^ (swl >> 2)) + (kg ^ (swl & 3))) * 8;
    // logits of tokens 16 t + 4 kg + j (t < 2, j < 4) of block blk for head hq
    auto logits = [&](int blk, f32x4 (&acc)[2]) {
      const uint16_t* rows = &sh.rows[blk & 3][0][0][0];
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        bf16x8 a[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          a[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(rows + lbase[kk & 3] + 16 * t * 128 + (kk >> 2) * (NI * 128)));
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma16x16x32(a[t], as_bf16x8(qv[kk]), acc[t]);
      }
    };
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // blocks 0 and 1 are in
    f32x4 cur[2];
    logits(0, cur);
    float M_run = -INFINITY, l_run = 0.f;
    for (int k = 0; k <= nblk; ++k) {
      if (k < nblk) {
        // block k + 1's logits (read from a stale buffer past the last block,
        // and then not used)
        f32x4 nxt[2];
        logits(k + 1, nxt);
        // bit 16 t + j: token 16 t + 4 kg + j
        const uint32_t vm = uint32_t(__ballot(lane < NI && sh.ids[k * NI + (lane & (NI - 1))] >= 0) >> (4 * kg));
        float m = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            cur[t][j] = (vm >> (16 * t + j)) & 1u ? cur[t][j] * scale_log2 : -INFINITY;
            m = fmaxf(m, cur[t][j]);
          }
        m = lane_groups_max(m);
        // the reference moves when the block's maximum exceeds it by more than
        // 8 (M_run = -inf: any finite maximum)
        const bool upd = m > M_run + 8.f;
        const float alpha = !upd ? 1.f : (M_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M_run - m));
        const float M_new = upd ? m : M_run;
        const float M_use = M_new == -INFINITY ? 0.f : M_new;
        float lh = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float p[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = __builtin_amdgcn_exp2f(cur[t][j] - M_use);
            lh += p[j];
          }
          *reinterpret_cast<u32x2*>(&sh.p[k & 1][hq][mla_pidx32(hq, 16 * t + 4 * kg)]) =
              u32x2{pack2bf(p[0], p[1]), pack2bf(p[2], p[3])};
        }
        lh = lane_groups_sum(lh);
        l_run = fmaf(l_run, alpha, lh);
        M_run = M_new;
        if (kg == 0) sh.alpha[k & 1][hq] = alpha;
        cur[0] = nxt[0];
        cur[1] = nxt[1];
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (kg == 0) {
      sh.lfin[hq] = l_run;
      if (lse)
        lse[size_t(r) * Hm + hq] =
            l_run > 0.f ? (M_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
    }
  } else {
    const int vq = w - 4;  // latent quarter
    const auto rs = make_rsrc(kv + size_t(bok ? b : 0) * T_max * kMlaDl, uint32_t(T_max) * (kMlaDl * 2));
    // quarter vq of the 32 rows of block blk, four rows per load (lane i: row
    // 4g + i / 16, piece slot i % 16): 8 loads
    auto gather = [&](int blk) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int t = 4 * g + (lane >> 4);
        const int id = sh.ids[blk * NI + t];
        const uint32_t off = (id >= 0 ? uint32_t(id) * (kMlaDl * 2) : 0x80000000u) +
                             16u * uint32_t(16 * vq + ((lane & 15) ^ mla_swz(t)));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(&sh.rows[blk & 3][vq][4 * g][0]), 16, off, 0, 0, 0);
      }
    };
    f32x4 o[4][8];  // [head tile][16-wide latent block]
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) o[ht][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    // byte offsets (in a buffer) of the transposing reads: rows t0 and t0 + 4,
    // 16-column block blk of quarter vq
    uint32_t voff[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        const int tt = 8 * kg + (ln >> 2) + 4 * e;
        const int col = 16 * blk + 4 * (ln & 3);
        voff[e][blk] = 2u * uint32_t(vq * (NI * 128) + tt * 128 + (((col >> 3) ^ mla_swz(tt)) << 3) + (col & 7));
      }
    gather(0);
    if (nblk > 1) gather(1);
    if (nblk > 2) gather(2);
    wait_vm_at_most(nblk > 2);  // blocks 0 and 1 are in
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int k = 0; k <= nblk; ++k) {
      if (k >= 1) {
        const int kb = k - 1;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const float a = sh.alpha[kb & 1][16 * ht + ln];
          if (__ballot(a != 1.f)) {
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) o[ht][blk] *= a;
          }
        }
        bf16x8 pb[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          pb[ht] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sh.p[kb & 1][16 * ht + ln][mla_pidx32(ln, 8 * kg)]));
        const uint32_t rb = uint32_t(reinterpret_cast<uintptr_t>(&sh.rows[kb & 3][0][0][0]));
        u32x2 tv[2][8];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          uint32_t ad[8];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            ad[2 * bb] = rb + voff[0][4 * hb + bb];
            ad[2 * bb + 1] = rb + voff[1][4 * hb + bb];
          }
          lds_read_tr16_x8(tv[hb], ad);
        }
        // this wave is done with its quarter of the buffer: block k + 3's goes in
        if (kb + 4 < nblk) gather(kb + 4);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          const u32x2 lo = tv[blk >> 2][2 * (blk & 3)], hi = tv[blk >> 2][2 * (blk & 3) + 1];
          const bf16x8 av = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) o[ht][blk] = mfma16x16x32(av, pb[ht], o[ht][blk]);
        }
      } else if (3 < nblk) {
        gather(3);  // the fourth buffer is free from the start
      }
      // block k + 2's quarter is in (the logits waves read it in the next
      // block): only block k + 3's gather may still be in flight
      wait_vm_at_most(k + 3 < nblk);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the sums are in
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int h = 16 * ht + ln;
      const float l = sh.lfin[h];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      uint16_t* dst = out + (size_t(r) * Hm + h) * kMlaDl + 128 * vq + 4 * kg;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        u32x2 pkd;
        pkd[0] = pack2bf(o[ht][blk][0] * inv, o[ht][blk][1] * inv);
        pkd[1] = pack2bf(o[ht][blk][2] * inv, o[ht][blk][3] * inv);
        *reinterpret_cast<u32x2*>(dst + blk * 16) = pkd;
      }
    }
    return;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // (logits waves) the sums are out
}

// Merge split partials: out = sum_s e^{lse_s} O_s / sum_s e^{lse_s}.  One
// wave per (row, head group, latent quarter, 16-channel block): lane (kg, ln)
// owns channels 4kg .. 4kg+3 of the block for head ln.  Splits are taken
// kCombineBatch at a time (16 or 32: the smaller one when it covers the row's
// splits, so that no load is spent on clamped duplicates); within a batch
// every lane issues all its loads (the split weights of its head and its
// slice of every split's partial: one contiguous 512-byte block per split and
// wave) before using any, and batches are merged with a running maximum.
constexpr int kMaxSplit = 256;
template <int kCombineBatch>
__global__ __launch_bounds__(64) void mla_combine(const uint16_t* __restrict__ part_o,
                                                  const float* __restrict__ part_lse, int nsplit,
                                                  int Hm, uint16_t* __restrict__ out,
                                                  float* __restrict__ lse) {
  const int HG = Hm >> 4;
  const int blk = blockIdx.x & 7, dq = (blockIdx.x >> 3) & 3, hg = blockIdx.x >> 5, r = blockIdx.y;
  const int lane = threadIdx.x, kg = lane >> 4, ln = lane & 15;
  const int h = hg * 16 + ln;
  float M = -INFINITY, ws = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += kCombineBatch) {
    float ls[kCombineBatch];
    u32x2 pv[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int sc = min(s0 + i, nsplit - 1);
      ls[i] = part_lse[(size_t(r) * nsplit + sc) * Hm + h];
      pv[i] = *reinterpret_cast<const u32x2*>(part_o + part_off(size_t(r) * nsplit + sc, HG, hg, dq, blk, lane));
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) Mn = s0 + i < nsplit ? fmaxf(Mn, ls[i]) : Mn;
    const float keep = M == -INFINITY ? 0.f : __expf(M - Mn);  // rescale of the earlier batches
    ws *= keep;
    acc *= keep;
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const float wgt = (s0 + i < nsplit && ls[i] != -INFINITY) ? __expf(ls[i] - Mn) : 0.f;
      ws += wgt;
      const f32x4 v = {__uint_as_float(pv[i][0] << 16), __uint_as_float(pv[i][0] & 0xffff0000u),
                       __uint_as_float(pv[i][1] << 16), __uint_as_float(pv[i][1] & 0xffff0000u)};
      acc += wgt * v;
    }
    M = Mn;
  }
  const float inv = ws > 0.f ? 1.0f / ws : 0.f;
  u32x2 pk;
  pk[0] = pack2bf(acc[0] * inv, acc[1] * inv);
  pk[1] = pack2bf(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(out + (size_t(r) * Hm + h) * kMlaDl + dq * 128 + blk * 16 + 4 * kg) = pk;
  if (dq == 0 && blk == 0 && kg == 0 && lse) lse[size_t(r) * Hm + h] = ws > 0.f ? M + logf(ws) : -INFINITY;
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
  bool rows;   // many rows: one workgroup per (row, head group) over all ids
  int nsplit;  // id slices of kMla2Ids per row
  int ns8;     // nsplit rounded up to a multiple of 8 (XCD spacing)
};

static int mla_slices(int W) { return (W + kMla2Ids - 1) / kMla2Ids; }

static MlaPlan mla_plan(int Q, int Hm, int Dl, int W, int dtype) {
  MlaPlan pl{false, false, 1, 1};
  if (!(dtype == DSA_BF16 && Dl == kMlaDl && Hm % 16 == 0 && Hm <= 128)) return pl;
  pl.mfma = true;
  if (W > kMlaSplit && long(Q) * (Hm / 16) >= kMlaRowsMinWgs) {
    pl.rows = true;
    return pl;
  }
  pl.nsplit = mla_slices(W);
  pl.ns8 = (pl.nsplit + 7) / 8 * 8;
  return pl;
}

// the combine of nsplit partials per row
static void launch_combine(int nsplit, int Q, int Hm, const uint16_t* part_o, const float* part_lse, void* out,
                           float* lse, hipStream_t s) {
  const dim3 grid((Hm / 16) * 32, Q);
  if (nsplit <= 16)
    hipLaunchKernelGGL(mla_combine<16>, grid, dim3(64), 0, s, part_o, part_lse, nsplit, Hm, (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL(mla_combine<32>, grid, dim3(64), 0, s, part_o, part_lse, nsplit, Hm, (uint16_t*)out, lse);
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

// Argument checks of dsa_sparse_mla_decode (and its allocation-free variant).
static int mla_check(const void* q_lat, const void* kv, const int32_t* row_seq, const int32_t* token_ids,
                     int Q, int Hm, int Dl, int B, int T_max, int W, int dtype, const void* out) {
  if (!q_lat || !kv || !row_seq || !token_ids || !out) return DSA_ERR_NULL;
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || B <= 0 || T_max <= 0 || W <= 0) return DSA_ERR_SHAPE;
  if (dtype != DSA_F32 && dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  if (Dl != 64 && Dl != 128 && Dl != 256 && Dl != 512) return DSA_ERR_UNSUPPORTED;
  if (Hm > 128 || Q > 65535) return DSA_ERR_UNSUPPORTED;
  if (long(W) > long(kMlaSplit) * kMaxSplit) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// The launches of dsa_sparse_mla_decode on a checked argument set, with the
// split partials in `workspace` (at least dsa_sparse_mla_workspace_bytes).
static int mla_launch(const void* q_lat, const void* kv, const int32_t* row_seq, const int32_t* token_ids, int Q,
                      int Hm, int Dl, int B, int T_max, int W, float sm_scale, int dtype, void* out, float* lse,
                      void* workspace, hipStream_t s) {
  const MlaPlan pl = mla_plan(Q, Hm, Dl, W, dtype);
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
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (pl.rows && Hm == 64 && T_max < kMlaPipeMaxT && W <= kMlaPipeMaxW) {
    hipLaunchKernelGGL(mla_rows64_pipe, dim3(Q), dim3(kMlaPipeThreads), 0, s, (const uint16_t*)q_lat,
                       (const uint16_t*)kv, row_seq, token_ids, B, T_max, W, scale_log2, (uint16_t*)out, lse);
    return launch_status();
  }
  if (pl.rows && Hm == 64) {
    hipLaunchKernelGGL(mla_rows64w8_mfma, dim3(Q), dim3(kMla8Threads), 0, s, (const uint16_t*)q_lat,
                       (const uint16_t*)kv, row_seq, token_ids, Q, B, T_max, W, scale_log2, (uint16_t*)out,
                       lse);
    return launch_status();
  }
  if (pl.rows) {
    const long nwg = (long(Q) + 7) / 8 * 8 * (Hm / 16);
    hipLaunchKernelGGL(mla_rows_mfma, dim3(unsigned(nwg)), dim3(kMlaThreads), 0, s, (const uint16_t*)q_lat,
                       (const uint16_t*)kv, row_seq, token_ids, Q, Hm, B, T_max, W, scale_log2,
                       (uint16_t*)out, lse);
    return launch_status();
  }
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (pl.nsplit > 1) {
    part_o = static_cast<uint16_t*>(workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(size_t(Q) * pl.nsplit * Hm * Dl * sizeof(uint16_t)));
  }
  dim3 grid((Hm / 16) * pl.ns8, Q);
  hipLaunchKernelGGL(mla_decode_mfma<kKvRows>, grid, dim3(kMla2Threads), 0, s, (const uint16_t*)q_lat, kv,
                     KvPages{nullptr, nullptr, 0, 1, 0}, row_seq, token_ids, Hm, B, T_max, W, pl.nsplit, pl.ns8,
                     scale_log2, (uint16_t*)out, lse, part_o, part_lse);
  int st = launch_status();
  if (st || pl.nsplit == 1) return st;
  launch_combine(pl.nsplit, Q, Hm, part_o, part_lse, out, lse, s);
  return launch_status();
}

extern "C" int dsa_sparse_mla_decode(const void* q_lat, const void* kv, const int32_t* row_seq,
                                     const int32_t* token_ids, int Q, int Hm, int Dl, int B,
                                     int T_max, int W, float sm_scale, int dtype, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const int st = mla_check(q_lat, kv, row_seq, token_ids, Q, Hm, Dl, B, T_max, W, dtype, out);
  if (st) return st;
  const size_t need = dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  return mla_launch(q_lat, kv, row_seq, token_ids, Q, Hm, Dl, B, T_max, W, sm_scale, dtype, out, lse, workspace,
                    as_stream(stream));
}

// The allocation-free variant keeps the split partials in this file-scope
// device array: every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol); it passes
// the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[DSA_MLA_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchDevices];

// the current device's address of `scratch` (looked up on the first call there)
static int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  if (dev < 0 || dev >= kScratchDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return DSA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DSA_OK;
}

extern "C" int dsa_sparse_mla_decode_noalloc(const void* q_lat, const void* kv, const int32_t* row_seq,
                                             const int32_t* token_ids, int Q, int Hm, int Dl, int B, int T_max,
                                             int W, float sm_scale, int dtype, void* out, float* lse,
                                             void* stream) {
  int st = mla_check(q_lat, kv, row_seq, token_ids, Q, Hm, Dl, B, T_max, W, dtype, out);
  if (st) return st;
  const size_t need = dsa_sparse_mla_workspace_bytes(Q, Hm, Dl, W, dtype);
  if (need > size_t(DSA_MLA_SCRATCH_BYTES)) return DSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  return mla_launch(q_lat, kv, row_seq, token_ids, Q, Hm, Dl, B, T_max, W, sm_scale, dtype, out, lse, ws,
                    as_stream(stream));
}

extern "C" size_t dsa_sparse_mla_paged_workspace_bytes(int Q, int Hm, int Dl, int W) {
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || W <= 0) return 0;
  const int nsplit = mla_slices(W);
  if (nsplit == 1) return 0;
  return align256(size_t(Q) * nsplit * Hm * Dl * sizeof(uint16_t)) + align256(size_t(Q) * nsplit * Hm * sizeof(float));
}

extern "C" int dsa_sparse_mla_decode_paged(const void* q_lat, const void* kv_pages, const float* kv_scale,
                                           const int32_t* block_table, int max_pages, int page_size,
                                           int num_pages, const int32_t* row_seq, const int32_t* token_ids,
                                           int Q, int Hm, int Dl, int B, int W, float sm_scale, int kv_dtype,
                                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (!q_lat || !kv_pages || !block_table || !row_seq || !token_ids || !out) return DSA_ERR_NULL;
  if (kv_dtype == DSA_FP8_E4M3 && !kv_scale) return DSA_ERR_NULL;
  if (Q <= 0 || Hm <= 0 || Dl <= 0 || B <= 0 || W <= 0 || max_pages <= 0 || page_size <= 0 || num_pages <= 0)
    return DSA_ERR_SHAPE;
  if (kv_dtype != DSA_BF16 && kv_dtype != DSA_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
  if (Dl != kMlaDl || Hm % 16 != 0 || Hm > 128 || Q > 65535) return DSA_ERR_UNSUPPORTED;
  if (long(W) > long(kMlaSplit) * kMaxSplit) return DSA_ERR_UNSUPPORTED;
  if (long(num_pages) * page_size > 2147483647L || long(max_pages) * page_size > 2147483647L)
    return DSA_ERR_UNSUPPORTED;
  const int nsplit = mla_slices(W);
  const int ns8 = (nsplit + 7) / 8 * 8;
  const size_t need = dsa_sparse_mla_paged_workspace_bytes(Q, Hm, Dl, W);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (nsplit > 1) {
    part_o = static_cast<uint16_t*>(workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        align256(size_t(Q) * nsplit * Hm * Dl * sizeof(uint16_t)));
  }
  hipStream_t s = as_stream(stream);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const KvPages pg{block_table, kv_scale, max_pages, page_size, num_pages};
  const int T_logical = max_pages * page_size;
  dim3 grid((Hm / 16) * ns8, Q);
  if (kv_dtype == DSA_BF16)
    hipLaunchKernelGGL(mla_decode_mfma<kKvPaged>, grid, dim3(kMla2Threads), 0, s, (const uint16_t*)q_lat, kv_pages,
                       pg, row_seq, token_ids, Hm, B, T_logical, W, nsplit, ns8, scale_log2, (uint16_t*)out, lse,
                       part_o, part_lse);
  else
    hipLaunchKernelGGL(mla_decode_mfma<kKvPagedFp8>, grid, dim3(kMla2Threads), 0, s, (const uint16_t*)q_lat,
                       kv_pages, pg, row_seq, token_ids, Hm, B, T_logical, W, nsplit, ns8, scale_log2,
                       (uint16_t*)out, lse, part_o, part_lse);
  int st = launch_status();
  if (st || nsplit == 1) return st;
  launch_combine(nsplit, Q, Hm, part_o, part_lse, out, lse, s);
  return launch_status();
}
