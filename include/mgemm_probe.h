/* Matrix-core ceiling probe: a measurement aid shipped beside libmgemm.so as
 * libmgemm_probe.so, not part of the grouped GEMM's interface.  It issues only
 * the bf16 matrix-core product the grouped kernels use (v_mfma_f32_32x32x16_bf16)
 * on register-held pseudo-random operands, with no memory traffic, so that the
 * rate it sustains is the practical ceiling of those products on this chip
 * under its power and clock limits (bench.py --ceiling reports it).
 */
#ifndef MGEMM_PROBE_H
#define MGEMM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch of `blocks` workgroups of 512 threads (8 waves; launch
 * one per compute unit to match the grouped kernels), each wave issuing
 * iters x 8 products.  out: fp32 [blocks * 512] DEVICE buffer, written (one
 * checksum per lane, only to keep the products live).  stream: a hipStream_t.
 * Returns 0, 1 for bad arguments (1 <= blocks <= 65536, iters >= 1, out
 * non-NULL) or 2 if the launch failed.  Allocates nothing. */
int mg_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

/* Flops one such launch performs: blocks x iters x 8 waves x 8 products x
 * 2 x 32 x 32 x 16. */
double mg_probe_mfma_bf16_flops(int32_t blocks, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_PROBE_H */
