/*
 * w8a8moe.h -- C ABI of the MI355X (gfx950) W8A8 INT8 fused Mixture-of-Experts layer.
 *
 * The layer (SGLang PR #3888 "[Feature] DeepSeek V3/R1 INT8 Quantization
 * (channel-wise)", Modifications and Performance; the jiqizhixin article on
 * Meituan's INT8 DeepSeek R1, section "Quantization exploration"):
 *   1. online symmetric INT8 quantization of the activations, one scale per
 *      token (channel-wise) or per token-group of 128 (block-wise);
 *   2. top-k expert routing from fp32 gate logits;
 *   3. grouping of the (token, slot) pairs by expert, with expert offsets equal
 *      to the zero-padded cumulative sum of the per-expert counts (SGLang PR
 *      #8273, review of the m_indices argument);
 *   4. grouped INT8 GEMM with the gate+up weights w13, int32 accumulation,
 *      one dequantization per output (a_scale[token] * w_scale[channel]) or one
 *      per 128-wide K-block (block-wise), SiLU(gate) * up, requantization;
 *   5. grouped INT8 GEMM with the down weights w2 and the top-k weighted
 *      combine of each token's expert outputs (PR #8273 highlights: scatter,
 *      GEMM, activation, GEMM, gather).
 *
 * Conventions for every entry point:
 *  - Pointers named as device buffers must point to device memory of the
 *    current HIP device; the caller owns every buffer.  The library never
 *    allocates, frees or synchronises, and never reads device data on the
 *    host, so every call can be captured into a HIP graph.
 *  - Tensors are dense, row-major and contiguous; strides are implied by the
 *    shapes given in each comment ([E, N, K] = expert, output row, K).
 *  - All work is enqueued on `stream` (NULL = the default stream) and is
 *    asynchronous: errors raised by a kernel while it runs surface at the
 *    caller's next synchronisation.
 *  - Arguments are validated on the host before anything is enqueued.  An
 *    invalid call returns a nonzero status and enqueues nothing.  No C++
 *    exception crosses this interface.
 *  - Sizes are int64_t; T = 0 (no tokens) is a successful no-op wherever the
 *    output is per token.
 *  - Int8 values are symmetric in [-127, 127].  Quantization rule:
 *    scale = max(max|x| / 127, 1e-8), q = round-half-even(x / scale), clamped.
 *
 * Shape limits (W8A8_UNSUPPORTED_SHAPE otherwise): 1 <= E <= 1024;
 * 1 <= k <= E; T * k <= 2^30; H and I multiples of 128, at most 65536;
 * block_m one of 16, 32, 64, 128.
 */
#ifndef W8A8MOE_H
#define W8A8MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  W8A8_OK = 0,
  W8A8_INVALID_ARGUMENT = 1,    /* null pointer, negative size, bad enum value */
  W8A8_UNSUPPORTED_SHAPE = 2,   /* sizes outside the limits above */
  W8A8_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the matching *_workspace_bytes() */
  W8A8_UNSUPPORTED_DTYPE = 4,   /* input dtype is neither fp32 nor bf16 */
  W8A8_HIP_ERROR = 5            /* a kernel launch failed (hipGetLastError) */
};

/* Activation input dtypes. */
enum { W8A8_DTYPE_F32 = 0, W8A8_DTYPE_BF16 = 1 };

/* Routing score functions. */
enum { W8A8_SCORE_SOFTMAX = 0, W8A8_SCORE_SIGMOID = 1 };

/* Scale layouts.  W8A8_SCALE_FP8_BLOCK128: the block-wise layouts with FP8 (E4M3) codes in place
 * of int8 values (see "FP8 block-wise variant" below).  W8A8_SCALE_W4A8: packed int4 weights with
 * one scale per (output row, 128-wide K group) and FP8 activations (see "W4A8 variant" below). */
enum { W8A8_SCALE_CHANNEL = 0, W8A8_SCALE_BLOCK128 = 1, W8A8_SCALE_FP8_BLOCK128 = 2, W8A8_SCALE_W4A8 = 3 };

/* Name of a status code ("W8A8_OK", ...); never NULL. */
const char* w8a8_status_string(int32_t status);

/* ------------------------------------------------------------------ step 1: activation quantization
 * Online symmetric INT8 quantization of activations (article, "Quantization
 * exploration": per token for channel-wise weights, per token-group for
 * block-wise weights).
 *   x      device, [rows, cols] fp32 or bf16 (x_dtype)
 *   group  0 = one scale per row; otherwise the group width (must divide cols)
 *   q      device, [rows, cols] int8 (output)
 *   scale  device, fp32 (output): [rows] if group == 0, else [rows, cols/group]
 */
int32_t w8a8_quant_per_token(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t group,
                             int8_t* q, float* scale, hipStream_t stream);

/* Offline weight quantization with one scale per block_rows x block_cols block
 * of a [rows, cols] matrix (same rule).  Per output channel of an expert's
 * [N, K] weight: block_rows = 1, block_cols = K (article: each weight column,
 * i.e. output channel, is one group).  Block-wise: 128 x 128 (article: DeepSeek's
 * [128, 128] blocks).  Blocks at the right/bottom edge may be partial.
 *   x      device, [rows, cols] fp32 or bf16
 *   q      device, [rows, cols] int8 (output)
 *   scale  device, [ceil(rows/block_rows), ceil(cols/block_cols)] fp32 (output)
 * Shapes (W8A8_UNSUPPORTED_SHAPE otherwise): rows and the block count below 2^31, rows * cols
 * below 2^40, at most 2^20 blocks across a row (w8a8_quant_per_token: the same, with blocks of
 * 1 x group, or 1 x cols for group 0).
 */
int32_t w8a8_quant_blocks(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t block_rows,
                          int64_t block_cols, int8_t* q, float* scale, hipStream_t stream);

/* ------------------------------------------------------------------ step 2: routing
 * Top-k expert selection per token (the pages name only its output, topk_idx,
 * in PR #8273).  Order: larger score first, equal scores to the lower index.
 *   logits          device, [T, E] fp32
 *   score_fn        W8A8_SCORE_SOFTMAX: select on the logits; weights are the
 *                   softmax over the selected logits (renormalize = 1) or the
 *                   softmax probability over all E (renormalize = 0).
 *                   W8A8_SCORE_SIGMOID: s = sigmoid(logit), c = s + bias; with
 *                   n_group > 1, experts are split into n_group equal groups,
 *                   group score = sum of its two best c, only the topk_group
 *                   best groups stay eligible; select the k best c; weights
 *                   s_j (/ sum of the selected s if renormalize).
 *   routed_scaling  every weight is multiplied by it at the end
 *   correction_bias device, [E] fp32, or NULL (sigmoid only)
 *   topk_ids        device, [T, k] int32 (output), slots in selection order
 *   topk_weights    device, [T, k] fp32 (output)
 * Limits: n_group divides E, n_group <= 64, 1 <= topk_group <= n_group,
 * k <= topk_group * E / n_group.
 */
int32_t moe_topk_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn,
                       int64_t n_group, int64_t topk_group, int32_t renormalize, float routed_scaling,
                       const float* correction_bias, int32_t* topk_ids, float* topk_weights,
                       hipStream_t stream);

/* ------------------------------------------------------------------ step 3: align by expert
 * Groups the P = T*k pairs (pair id p = t*k + j) by expert, stably (ascending p
 * within an expert), and pads every expert's segment to a multiple of block_m
 * with the sentinel value P.
 *   topk_ids        device, [T, k] int32; ids outside [0, E) are dropped
 *   expert_counts   device, [E] int32 (output)
 *   expert_offsets  device, [E+1] int32 (output): 0, cumsum(expert_counts)
 *   padded_offsets  device, [E+1] int32 (output): 0, cumsum(padded counts)
 *   sorted_pair_ids device, [w8a8_moe_max_rows()] int32 (output); entries at
 *                   and beyond padded_offsets[E] are left untouched
 *   tile_expert     device, [w8a8_moe_max_rows() / block_m] int32 (output):
 *                   expert of each block_m-row tile
 *   num_tiles       device, [1] int32 (output): padded_offsets[E] / block_m
 *   ws              device workspace of moe_align_workspace_bytes() bytes
 */
int64_t w8a8_moe_max_rows(int64_t T, int64_t k, int64_t E, int64_t block_m);
size_t moe_align_workspace_bytes(int64_t T, int64_t k, int64_t E);
int32_t moe_align_by_expert(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                            int32_t* expert_counts, int32_t* expert_offsets, int32_t* padded_offsets,
                            int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* num_tiles, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* The same align for callers that cannot allocate or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments and outputs as
 * moe_align_by_expert, bit-identical to it; no ws.  Its scratch (the per-chunk histograms and the
 * pairs' ranks, align's workspace) is a device array of moe_align_noalloc_scratch_bytes() = 4 MiB
 * inside the library, one per GPU, held until the process ends; the call allocates nothing and
 * needs nothing cleared (every scratch word it reads, it wrote earlier in the same call).
 * Returns W8A8_UNSUPPORTED_SHAPE when moe_align_workspace_bytes(T, k, E) exceeds that size (for
 * E = 256 up to about 838k pairs; 4*T*k + 4*E*ceil(T*k/1024) bytes, each term rounded up to 256).
 * Calls on one GPU share its array: two calls whose kernels overlap on that GPU (other streams,
 * other host threads) race and give wrong results; calls in one stream order are safe.  The first
 * call on each device resolves the array's device address (hipGetSymbolAddress, no allocation);
 * make that first call outside stream capture. */
int32_t moe_align_by_expert_noalloc(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* padded_offsets,
                                    int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* num_tiles,
                                    hipStream_t stream);
size_t moe_align_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------ steps 4-5: grouped INT8 GEMMs
 * Common arguments (outputs of moe_align_by_expert with the same block_m):
 *   sorted_pair_ids, padded_offsets, tile_expert, num_tiles (device; num_tiles is read on the
 *   device only).  Rows of the intermediate are the padded expert-sorted rows;
 *   rows holding the sentinel are skipped and their outputs are unspecified.
 *
 * Raw int32 accumulators (the exact integer products before any scaling), for checking the
 * integer core of the channel-wise GEMMs bit for bit (PR #3888, Performance: the fused MoE with an
 * int32 accumulator; article, "Quantization exploration": the int8 matmul before its single
 * dequantization).  The call runs the engine, tile shape, gate/up tile pairing and work order that
 * the channel-wise GEMM of the same layer shape runs (w8a8_moe_engine with W8A8_SCALE_CHANNEL);
 * only its epilogue differs, storing the int32 sums instead of scaling them.
 *   gather = 1: the first GEMM of a layer with H = K, I = N / 2: the A row of sorted row r is
 *               a[sorted_pair_ids[r] / k] ([T, K]) and w is w13 [E, N, K];
 *   gather = 0: the second GEMM of a layer with H = N, I = K: the A row of sorted row r is a[r]
 *               ([max_rows, K], the sorted intermediate) and w is w2 [E, N, K].
 *   w    device, [E, N, K] int8
 *   out  device, [max_rows, N] int32 (output; pad rows untouched)
 *   ws   device workspace of w8a8_grouped_gemm_i32_workspace_bytes() bytes (the engine's tile list)
 * Shapes: H and I as for the layer (multiples of 128, at most 65536); N even when gather = 1.
 */
size_t w8a8_grouped_gemm_i32_workspace_bytes(int32_t gather, int64_t N, int64_t K, int64_t T, int64_t k, int64_t E,
                                             int64_t block_m); /* 0 for invalid arguments */
int32_t w8a8_grouped_gemm_i32(const int8_t* a, int32_t gather, const int8_t* w, int64_t N, int64_t K,
                              const int32_t* sorted_pair_ids, const int32_t* padded_offsets,
                              const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int64_t k, int64_t E,
                              int64_t block_m, int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Which GEMM engine the grouped GEMMs of a layer of this shape and scale mode run (both GEMMs of
 * a layer run the same one), decided on the host from the shapes alone: W8A8_ENGINE_STAGED (few
 * rows per expert: register-staged LDS tiles of block_m rows), W8A8_ENGINE_DMA (hundreds of rows
 * per expert: 320 x 256 tiles filled by direct-to-LDS loads), W8A8_ENGINE_RING (tens to ~200 rows
 * per expert at the DeepSeek-V3 shapes, the block-wise and FP8 paths: a 3-stage LDS ring) or
 * W8A8_ENGINE_STREAM (W4A8 with few rows per expert: int4 weights straight to registers).
 * Returns -1 for arguments the GEMM entry points would reject. */
enum { W8A8_ENGINE_STAGED = 0, W8A8_ENGINE_DMA = 1, W8A8_ENGINE_RING = 2, W8A8_ENGINE_STREAM = 3 };
int32_t w8a8_moe_engine(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m, int32_t scale_mode);

/* Channel-wise first GEMM (PR #3888: fused MoE with channel-wise int8 and an
 * int32 accumulator; article: one dequantization after the INT8 matmul):
 *   acc = a_q[t] . w13[e, n]  (int32), g = ((float)acc * a_scale[t]) * w13_scale[e, n]
 *   for n < I, u likewise for row n + I; h = silu(g) * u, silu(g) = g/(1+exp(-g));
 *   h_scale[r] = max(max_n |h| / 127, 1e-8), h_q[r, n] = rne(h / h_scale[r]).
 *   a_q        device, [T, H] int8;  a_scale device, [T] fp32
 *   w13        device, [E, 2I, H] int8 (rows [0, I) gate, [I, 2I) up)
 *   w13_scale  device, [E, 2I] fp32
 *   h_q        device, [max_rows, I] int8 (output, sorted-row order)
 *   h_scale    device, [max_rows] fp32 (output)
 *   ws         device workspace of w8a8_w13_workspace_bytes() bytes
 */
size_t w8a8_w13_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                                int32_t scale_mode);
int32_t w8a8_grouped_gemm_w13_silu(const int8_t* a_q, const float* a_scale, const int8_t* w13,
                                   const float* w13_scale, const int32_t* sorted_pair_ids,
                                   const int32_t* padded_offsets, const int32_t* tile_expert,
                                   const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                   int64_t I, int64_t block_m, int8_t* h_q, float* h_scale, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* Channel-wise second GEMM and combine:
 *   acc = h_q[r] . w2[e, n] (int32), y = ((float)acc * h_scale[r]) * w2_scale[e, n];
 *   out[t, n] = 0, then out = out + topk_weights[t, j] * y(row of pair t*k+j) for j = 0..k-1.
 *   w2         device, [E, H, I] int8;  w2_scale device, [E, H] fp32
 *   topk_weights device, [T, k] fp32
 *   out        device, [T, H] fp32 (output, fully overwritten)
 *   ws         device workspace of w8a8_w2_workspace_bytes() bytes
 */
size_t w8a8_w2_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                               int32_t scale_mode);
int32_t w8a8_grouped_gemm_w2_combine(const int8_t* h_q, const float* h_scale, const int8_t* w2,
                                     const float* w2_scale, const int32_t* sorted_pair_ids,
                                     const int32_t* padded_offsets, const int32_t* tile_expert,
                                     const int32_t* num_tiles, const float* topk_weights, int64_t T,
                                     int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m, float* out,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Block-wise variants (article: [128, 128] weight blocks, activations quantized
 * per token-group of 128; dequantization per 128-wide K-block, accumulated in
 * fp32 in ascending K-block order: acc += ((float)part_kb * a_s[t, kb]) * w_s[e, n/128, kb]).
 * The intermediate is requantized per (row, 128-group).
 *   a_scale    device, [T, H/128];  w13_scale device, [E, 2I/128, H/128]
 *   h_scale    device, [max_rows, I/128]; w2_scale device, [E, H/128, I/128]
 * Other arguments as in the channel-wise entry points; workspaces from the
 * size queries with scale_mode = W8A8_SCALE_BLOCK128. */
int32_t w8a8_block_grouped_gemm_w13_silu(const int8_t* a_q, const float* a_scale, const int8_t* w13,
                                         const float* w13_scale, const int32_t* sorted_pair_ids,
                                         const int32_t* padded_offsets, const int32_t* tile_expert,
                                         const int32_t* num_tiles, int64_t T, int64_t k, int64_t E,
                                         int64_t H, int64_t I, int64_t block_m, int8_t* h_q, float* h_scale,
                                         void* ws, size_t ws_bytes, hipStream_t stream);
int32_t w8a8_block_grouped_gemm_w2_combine(const int8_t* h_q, const float* h_scale, const int8_t* w2,
                                           const float* w2_scale, const int32_t* sorted_pair_ids,
                                           const int32_t* padded_offsets, const int32_t* tile_expert,
                                           const int32_t* num_tiles, const float* topk_weights, int64_t T,
                                           int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ FP8 block-wise variant
 * SGLang PR #8273 (description, "New FP8 MoE Kernel"): an MoE with per-block FP8 weights and
 * per-token-group FP8 activations, multiplied by a block-scaled grouped GEMM.  FP8 here is E4M3
 * as the OCP 8-bit floating-point specification defines it (sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, largest finite value 448, codes 0x7F / 0xFF NaN and never produced); codes are
 * bytes (uint8_t).  Quantization rule: scale = max(max|x| / 448, 1e-8), code = the E4M3 value
 * nearest to x / scale (ties to even) after clamping x / scale to [-448, 448].
 *
 * w8a8_fp8_quant_blocks: arguments as w8a8_quant_blocks, FP8 codes out (block_rows = 1,
 * block_cols = 128: per-token-group activations; 128 x 128: weights).
 *
 * The GEMMs take the block-wise layouts of the INT8 variants (a_scale [T, H/128], w13_scale
 * [E, 2I/128, H/128], h_scale [max_rows, I/128], w2_scale [E, H/128, I/128]) and accumulate each
 * 128-wide K-block's products with the gfx950 FP8 MFMA in fp32, then
 * acc += (part_kb * a_s[t, kb]) * w_s[e, n/128, kb] in fp32, in ascending K-block order.  The
 * products are exact; the MFMA's fp32 summation order inside a K-block is the hardware's, so
 * results agree with an exact per-block sum to within fp32 rounding, not bit for bit.  The first
 * GEMM requantizes SiLU(gate) * up to FP8 per (row, 128-group).  Workspaces from the size queries
 * with scale_mode = W8A8_SCALE_FP8_BLOCK128.
 * Shapes (W8A8_UNSUPPORTED_SHAPE otherwise): H a multiple of 256; H/128 and I/128 each one of
 * 1, 2, 4, 8, 16, 32, 56; T*H, max_rows*I and 2*I*H below 2^32; at most 2^20 work items of 128-row
 * tiles, (ceil(T*k/128) + min(E, T*k)) * max(I/128, H/256).  Operand pointers 16-byte aligned. */
int32_t w8a8_fp8_quant_blocks(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t block_rows,
                              int64_t block_cols, uint8_t* q, float* scale, hipStream_t stream);
int32_t w8a8_fp8_grouped_gemm_w13_silu(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                       const float* w13_scale, const int32_t* sorted_pair_ids,
                                       const int32_t* padded_offsets, const int32_t* tile_expert,
                                       const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                       int64_t I, int64_t block_m, uint8_t* h_q, float* h_scale, void* ws,
                                       size_t ws_bytes, hipStream_t stream);
int32_t w8a8_fp8_grouped_gemm_w2_combine(const uint8_t* h_q, const float* h_scale, const uint8_t* w2,
                                         const float* w2_scale, const int32_t* sorted_pair_ids,
                                         const int32_t* padded_offsets, const int32_t* tile_expert,
                                         const int32_t* num_tiles, const float* topk_weights, int64_t T, int64_t k,
                                         int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                                         size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ W4A8 variant
 * SGLang PR #8311 (w4a8 DeepSeek-R1; its MoE layer enables the path with a w4afp8 flag): 4-bit
 * integer weights, FP8 activations.  Weights: symmetric int4 in [-7, 7], one fp32 scale per (output
 * row, 128-wide K group): scale = max(max|w| / 7, 1e-8), q = clamp(round-half-even(w / scale)).
 * Packing: a row of K values is K/2 bytes; each run of 8 values is 4 bytes, byte b holding value b
 * in its low nibble and value 4 + b in its high nibble; a nibble is sign (bit 3) | magnitude
 * (bits 0-2), zero as 0.  Activations and the intermediate: FP8 codes by the FP8 variant's rule
 * per token-group (w8a8_fp8_quant_blocks with 1 x 128 blocks).  Product: per 128-wide K-block the
 * FP8 MFMA on the activations and the weights widened to E4M3 (exact), then
 * acc += (part_kb * a_s[t, kb]) * w_s[e, n, kb] in fp32, ascending K-blocks; the rest as in the
 * FP8 variant (same summation-order caveat).
 *
 * w8a8_w4a8_quant_weights: x device [rows, cols] fp32 or bf16, cols a multiple of 128 and at most
 *   2^27; rows below 2^31, rows * cols below 2^40;
 *   q device [rows, cols/2] packed (output); scale device [rows, cols/128] fp32 (output).
 * GEMMs: w13 device [E, 2I, H/2] packed, w13_scale [E, 2I, H/128]; w2 [E, H, I/2] packed,
 *   w2_scale [E, H, I/128]; a_q / h_q FP8 codes with a_scale [T, H/128] / h_scale [max_rows, I/128];
 *   other arguments, shape limits and workspaces (scale_mode = W8A8_SCALE_W4A8) as in the FP8
 *   variant. */
int32_t w8a8_w4a8_quant_weights(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                                float* scale, hipStream_t stream);
int32_t w8a8_w4a8_grouped_gemm_w13_silu(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                        const float* w13_scale, const int32_t* sorted_pair_ids,
                                        const int32_t* padded_offsets, const int32_t* tile_expert,
                                        const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                        int64_t I, int64_t block_m, uint8_t* h_q, float* h_scale, void* ws,
                                        size_t ws_bytes, hipStream_t stream);
int32_t w8a8_w4a8_grouped_gemm_w2_combine(const uint8_t* h_q, const float* h_scale, const uint8_t* w2,
                                          const float* w2_scale, const int32_t* sorted_pair_ids,
                                          const int32_t* padded_offsets, const int32_t* tile_expert,
                                          const int32_t* num_tiles, const float* topk_weights, int64_t T, int64_t k,
                                          int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                                          size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ dense linear
 * W8A8 INT8 linear for the model's non-MoE projections (PR #3888 Modifications, "Norm Linear": the
 * dense layers run as w8a8 int8 GEMMs; article, "Quantization exploration": channel-wise weights
 * with online per-token activation scales, one dequantization after the INT8 matmul):
 *   out[m, n] = ((float)(a_q[m] . w[n]) * a_scale[m]) * w_scale[n]   (int32 dot product, fp32 out)
 *   a_q      device, [M, K] int8 (quantize with w8a8_quant_per_token, group 0)
 *   a_scale  device, [M] fp32
 *   w        device, [N, K] int8, K-contiguous;  w_scale device, [N] fp32
 *   out      device, [M, N] fp32 (output, fully overwritten)
 *   ws       device workspace of w8a8_linear_workspace_bytes(M, N, K) bytes (at least 256): when few
 *            rows leave CUs idle, the int32 partial sums of K slices (added exactly, in slice order)
 * Shapes: K and N multiples of 256, M*K and N*K below 2^32, at most 2^20 output tiles (of 320 x 256,
 * or 128-row tiles times K slices for few rows); M = 0 is a no-op.  a_q and w 16-byte
 * aligned.  Returns W8A8_UNSUPPORTED_SHAPE for other shapes, W8A8_WORKSPACE_TOO_SMALL for a short
 * workspace.  Deterministic: every output is one fixed sequence of operations. */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);  /* 0 for an unsupported shape */
int32_t w8a8_linear(const int8_t* a_q, const float* a_scale, const int8_t* w, const float* w_scale, int64_t M,
                    int64_t N, int64_t K, float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ the whole layer
 * Steps 2, 1, 3, 4, 5 on one stream, intermediates carved from `ws`.
 * block_m = 0 picks a tile height from the average rows per expert.  With scale_mode =
 * W8A8_SCALE_FP8_BLOCK128 the w13 / w2 buffers hold FP8 codes and the activations are quantized
 * to FP8 per token-group (the FP8 variant's rule and shape limits); with W8A8_SCALE_W4A8 they hold
 * packed int4 weights with per-(row, K-group) scales and the activations are FP8 as well. */
struct w8a8_moe_args {
  const void* x;               /* device, [T, H] fp32 or bf16 activations */
  int32_t x_dtype;             /* W8A8_DTYPE_* */
  const float* router_logits;  /* device, [T, E] fp32 */
  const int8_t* w13;           /* device, [E, 2I, H] int8 (or FP8 codes; W4A8: [E, 2I, H/2] packed int4) */
  const float* w13_scale;      /* device, [E, 2I], [E, 2I/128, H/128] or (W4A8) [E, 2I, H/128] fp32 */
  const int8_t* w2;            /* device, [E, H, I] int8 (or FP8 codes; W4A8: [E, H, I/2] packed int4) */
  const float* w2_scale;       /* device, [E, H], [E, H/128, I/128] or (W4A8) [E, H, I/128] fp32 */
  const float* correction_bias;/* device, [E] fp32 or NULL */
  float* out;                  /* device, [T, H] fp32 (output) */
  int32_t* topk_ids;           /* device, [T, k] int32 (output), or NULL to keep it in ws */
  float* topk_weights;         /* device, [T, k] fp32 (output), or NULL to keep it in ws */
  int64_t T, H, I, E, k;
  int32_t score_fn;            /* W8A8_SCORE_* */
  int64_t n_group, topk_group;
  int32_t renormalize;
  float routed_scaling;
  int32_t scale_mode;          /* W8A8_SCALE_* */
  int64_t block_m;             /* 0 = automatic */
};
int64_t w8a8_moe_pick_block_m(int64_t T, int64_t k, int64_t E);
size_t w8a8_moe_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                                int32_t scale_mode);
int32_t w8a8_moe_forward(const struct w8a8_moe_args* args, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8MOE_H */
