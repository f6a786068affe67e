// Shared device helpers for the gfx950 kernels (wave64, MFMA, bf16 bit handling).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is carried as its raw 16 bits (uint16_t) in memory.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// two fp32 -> packed bf16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Activation element access for fp32 and bf16 tensors.
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f2bf(v); }
};

// 8 consecutive activations -> fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack2bf(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<u32x4*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Buffer resource over [p, p + bytes) (bytes < 2^31).  A load whose per-lane
// offset is at or past `bytes` returns 0 (the hardware range check), so loads
// need no clamped addresses and no per-lane 64-bit pointers.  Offsets go in
// the per-lane operand: the range check does not cover the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}

// Pool-cache layout.  The pooled keys [B, P_max, D] are stored tile-interleaved:
// pools are grouped in tiles of 16 (P_tiles = ceil(P_max / 16) per sequence),
// and a tile stores its 16-byte pieces piece-major, so piece c of the tile's
// 16 pools forms 256 contiguous bytes.  For bf16 keys with D = 128 a 16-pool
// tile is 4 KiB and one wave-wide 16-byte load per lane covers pieces 4i ..
// 4i+3 of all 16 pools (1 KiB contiguous), exactly the matrix-core operand
// layout.  E = elements per piece.
template <typename T>
struct KpLayout {
  static constexpr int E = 16 / int(sizeof(T));
  static __host__ __device__ __forceinline__ size_t index(size_t b, int p, int ch, int P_tiles, int D) {
    return (((b * P_tiles + (p >> 4)) * size_t(D / E) + ch / E) * 16 + (p & 15)) * E + ch % E;
  }
};
__host__ __device__ __forceinline__ int pool_tiles(int P_max) { return (P_max + 15) >> 4; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 r) { return __builtin_bit_cast(bf16x8, r); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (l & 15) of A and column (l & 15) of B, each with the 8 k-values of group
// (l >> 4); it receives D rows 4*(l >> 4) + j, j < 4, of column (l & 15).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace dsa
