/* w8a8probe.h -- measured peaks of the device, for the benchmark's report (libw8a8probe.so).
 *
 * Not part of the MoE layer: three small kernels whose rates are the "measured on this chip"
 * counterparts of the published peaks the layer's figures are quoted against.  All calls are
 * asynchronous on `stream` (NULL = default stream); the caller times them (HIP events) and
 * owns every buffer.  Return 0 on success, 1 for a bad argument (null pointer, size not a
 * positive multiple of 16, non-positive count), 5 when the launch fails.
 */
#ifndef W8A8PROBE_H
#define W8A8PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of device memory at `buf` once (16-byte non-temporal loads); writes to the
 * device int32 `sink` only in a case that does not occur in practice. */
int32_t w8a8_probe_read(const void* buf, int64_t bytes, int32_t* sink, hipStream_t stream);

/* Copies `bytes` from device `src` to device `dst` (non-overlapping), 16-byte non-temporal
 * loads and stores. */
int32_t w8a8_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* `workgroups` workgroups of 4 wavefronts, each wavefront issuing `iters` rounds of independent
 * INT8 MFMAs on pseudo-random operands: shape 16 = 8 v_mfma_i32_16x16x64_i8, shape 32 = 4
 * v_mfma_i32_32x32x32_i8 (the same multiply-adds); `sink` as above.  Returns 1 for a null sink,
 * iters or workgroups below 1 or another shape. */
int32_t w8a8_probe_mfma_i8(int64_t iters, int32_t workgroups, int32_t shape, int32_t* sink, hipStream_t stream);

/* `blocks` independent products, one wavefront and one FP8 MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 operands, scales 1.0, zero accumulator) each:
 * c[blk][i][j] = sum over k < 128 of a[blk][i][k] * b[blk][j][k], with a and b device [blocks, 16,
 * 128] E4M3 codes (32-byte aligned) and c device [blocks, 16, 16] fp32.  The operands are fed
 * with the layer's FP8 GEMM layout (lane (g, r): bytes [32 g, 32 g + 32) of row r), so the tests
 * measure the accumulation that GEMM gets. */
int32_t w8a8_probe_mfma_f8_block(const uint8_t* a, const uint8_t* b, float* c, int32_t blocks, hipStream_t stream);

/* Integer operations (2 per multiply-add) of one w8a8_probe_mfma_i8 launch (either shape). */
int64_t w8a8_probe_mfma_i8_ops(int64_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* W8A8PROBE_H */
