// Token-order combine of routed rows, the inverse of the forward's gather
// (the MoE layout of the DeepGEMM issue #10 thread): the rows i with
// gather[i] = t hold token t's copies, one per routed expert; the backward of
// the gather sums their gradients back per token, and the layer's output
// combine sums the experts' outputs with the router's weights:
//   out[t, :] = sum_{j < k} w[t, j] rows[token_rows[t, j], :]   (j ascending)
// fp32 accumulation in that fixed order (bitwise reproducible), one rounding
// to bf16.  HBM-bound: each thread moves 16-byte pieces, the lanes of a wave
// cover consecutive pieces of the same row, four rows' loads in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgemm_launch.h"

namespace mg {

typedef uint32_t u32x4_c __attribute__((ext_vector_type(4)));
typedef float f32x2_c __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_c __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ rows,
                                                          const int32_t* __restrict__ token_rows,
                                                          const float* __restrict__ weights,
                                                          uint16_t* __restrict__ out, int64_t M,
                                                          int64_t T, int32_t k, int64_t D) {
  const int64_t chunks = D / 8;
  const int64_t total = T * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t t = idx / chunks, c = idx - t * chunks;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    // four slots at a time: their indices, then their four loads in flight
    // together, then the adds in slot order
    for (int j0 = 0; j0 < k; j0 += 4) {
      int32_t r[4];
      u32x4_c v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        r[u] = j0 + u < k ? token_rows[t * k + j0 + u] : -1;
        if (r[u] >= M) r[u] = -1;                    // an index out of range: no row
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = r[u] >= 0 ? *reinterpret_cast<const u32x4_c*>(rows + (int64_t)r[u] * D + c * 8)
                         : (u32x4_c){0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (r[u] < 0) continue;
        const float w = weights != nullptr ? weights[t * k + j0 + u] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(w, __builtin_bit_cast(float, v[u][q] << 16), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(w, __builtin_bit_cast(float, v[u][q] & 0xFFFF0000u),
                                          acc[2 * q + 1]);
        }
      }
    }
    u32x4_c o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = __builtin_bit_cast(uint32_t,
                                __builtin_convertvector((f32x2_c){acc[2 * q], acc[2 * q + 1]},
                                                        bf16x2_c));
    *reinterpret_cast<u32x4_c*>(out + t * D + c * 8) = o;
  }
}

int launch_moe_combine(const uint16_t* rows, const int32_t* token_rows, const float* weights,
                       uint16_t* out, int64_t M, int64_t T, int32_t k, int64_t D, hipStream_t s) {
  const int64_t total = T * (D / 8);
  if (total <= 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;                   // grid-stride beyond
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, rows,
                     token_rows, weights, out, M, T, k, D);
  return (int)hipGetLastError();
}

}  // namespace mg
