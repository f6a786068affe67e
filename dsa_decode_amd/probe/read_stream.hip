// A plain HBM read stream: the measured bandwidth ceiling that the score
// kernel's roofline is quoted against besides the 8 TB/s spec figure.  Each
// wave reads one contiguous stretch of the buffer with 16-byte non-temporal
// loads (1 KiB per wave-wide load, 8 loads in flight per lane), the access
// pattern of the pool-cache stream, and folds the words with XOR; one word
// per thread is written only when `sink` is non-null (never in the
// measurement), which keeps the loads from being removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ src, long n16,
                                                              long per_wave, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long wave = long(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const long begin = wave * per_wave;
  long end = begin + per_wave;
  if (end > n16) end = n16;
  uint32_t acc = 0;
  for (long i = begin + lane; i < end; i += 64L * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const long j = i + 64L * u;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (sink) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Reads `bytes` (a multiple of 16) from device pointer p, each wave taking a
// stretch of wave_bytes (a multiple of 1024); 0 on success, -1 on bad
// arguments, -5 on a launch error.
extern "C" int dsa_probe_read_stream(const void* p, long bytes, long wave_bytes, void* stream) {
  if (!p || bytes <= 0 || bytes % 16 || wave_bytes <= 0 || wave_bytes % 1024) return -1;
  const long n16 = bytes / 16, per_wave = wave_bytes / 16;
  const long waves = (n16 + per_wave - 1) / per_wave;
  const long blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7fffffffL) return -1;
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(p), n16, per_wave, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
