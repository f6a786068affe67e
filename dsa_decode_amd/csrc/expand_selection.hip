// expand_selection: pool ids -> token ids (page "Module glm5next_dsa", "Shape
// of the pipeline": -> [Q, out_width] token ids, -1 = invalid; "Traps carried
// from Slice 8": the -1 sentinel destination must be fully written).
//
// One thread per output column; every column of every row is written, so no
// caller-side fill is needed (an unwritten tail is the bug class the page
// warns about).
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ pool_ids, int K,
                                                     const int32_t* __restrict__ row_seq,
                                                     const int32_t* __restrict__ pool_start, int B,
                                                     int P_max, int kp,
                                                     int32_t* __restrict__ token_ids, int W) {
  const int r = blockIdx.y;
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= W) return;
  int32_t tok = -1;
  const int j = col / kp, s = col - j * kp;
  if (j < K) {
    const int b = row_seq[r];
    const int p = pool_ids[size_t(r) * K + j];
    if (p >= 0 && p < P_max && b >= 0 && b < B) {
      const int ps = pool_start[size_t(b) * P_max + p];
      if (ps >= 0) tok = ps + s;
    }
  }
  token_ids[size_t(r) * W + col] = tok;
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_expand_selection(const int32_t* pool_ids, int Q, int K, const int32_t* row_seq,
                                    const int32_t* pool_start, int B, int P_max, int kpool,
                                    int32_t* token_ids, int W, void* stream) {
  if (!pool_ids || !row_seq || !pool_start || !token_ids) return DSA_ERR_NULL;
  if (Q <= 0 || K <= 0 || B <= 0 || P_max <= 0 || kpool <= 0 || W <= 0) return DSA_ERR_SHAPE;
  if (kpool > DSA_MAX_KPOOL) return DSA_ERR_UNSUPPORTED;
  if (long(W) < long(K) * kpool) return DSA_ERR_SHAPE;
  if (Q > 65535) return DSA_ERR_UNSUPPORTED;
  dim3 grid(ceil_div(W, 256), Q);
  hipLaunchKernelGGL(expand_kernel, grid, dim3(256), 0, as_stream(stream), pool_ids, K, row_seq,
                     pool_start, B, P_max, kpool, token_ids, W);
  return launch_status();
}
