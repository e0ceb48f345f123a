// Matrix-core ceiling probe (a measurement aid, not part of the grouped GEMM).
//
// Every wave issues only v_mfma_f32_32x32x16_bf16 -- the product the grouped
// kernels use -- on operands held in registers, into eight independent
// accumulators, with no memory traffic and no barrier inside the loop.  The
// operands are pseudo-random bf16 values of unit size, four A and four B
// fragments per wave, so that successive products see different bits as in a
// GEMM on random data.  What it measures: the rate the matrix cores sustain
// on this chip when nothing else runs, under the same power and clock limits
// as the GEMM.  Eight waves per workgroup (two per SIMD), one workgroup per
// compute unit, as the grouped kernels launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgemm_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bits of a value in [-1, 1) from a 32-bit hash (sign, exponent 2^-1
// .. 2^-4, random mantissa): finite, no subnormals.
__device__ __forceinline__ __bf16 hashed_bf16(uint32_t h) {
  const uint32_t e = 126u - ((h >> 8) & 3u);
  const uint16_t bits = (uint16_t)(((h >> 31) << 15) | (e << 7) | (h & 0x7Fu));
  return __builtin_bit_cast(__bf16, bits);
}

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, float* out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[f][e] = hashed_bf16(mix(gid * 64u + (uint32_t)(f * 8 + e)));
      b[f][e] = hashed_bf16(mix(gid * 64u + 32u + (uint32_t)(f * 8 + e)));
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[gid] = s;          // keeps the products live; one vector store per lane
}

}  // namespace

extern "C" int mg_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || out == nullptr) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(512), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" double mg_probe_mfma_bf16_flops(int32_t blocks, int32_t iters) {
  // 8 waves x 8 products x 2 x 32 x 32 x 16 flops per iteration and workgroup
  return (double)blocks * (double)iters * 8.0 * 8.0 * 32768.0;
}
