// kernels.hpp -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

// A dispatch counts the work-items of its x extent in 32 bits, so blocks times threads must stay
// below 2^32 or the grid silently wraps.  Every launch keeps to kMaxGridBlocks workgroups (2^30
// work-items at 1024 threads): the per-row and per-token kernels go in pieces or walk their rows
// with a grid stride, the staged GEMM goes in pieces, and the work-list GEMM engines are chosen
// only for shapes whose grid fits.
constexpr int64_t kMaxGridBlocks = int64_t(1) << 20;

// quant.hip
// fp8: E4M3 codes (as bytes in q) by the FP8 rule instead of the INT8 rule.
hipError_t quant_blocks(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                        int8_t* q, float* scale, hipStream_t stream, bool fp8 = false);
// Packed int4 weights, one scale per (row, 128 columns); cols a multiple of 128.
hipError_t quant_w4(const void* x, int32_t dtype, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                    hipStream_t stream);

// route.hip
hipError_t topk_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn, int64_t n_group,
                      int64_t topk_group, int32_t renormalize, float routed_scaling, const float* bias,
                      int32_t* ids, float* weights, hipStream_t stream);

// align.hip
constexpr int64_t kAlignChunk = 1024;     // pairs per histogram chunk
constexpr int64_t kAlignSmallMax = 4096;  // at most this many pairs: one single-workgroup launch
size_t align_ws_bytes(int64_t P, int64_t E);
// The allocation-free align entry point's scratch: a file-scope device array of this many bytes in
// align.hip; noalloc_scratch gives its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t align_by_expert(const int32_t* ids, int64_t P, int64_t E, int64_t block_m, int32_t* counts,
                           int32_t* offsets, int32_t* padded_offsets, int32_t* sorted, int32_t* tile_expert,
                           int32_t* num_tiles, int64_t max_tiles, void* ws, hipStream_t stream);

// gemm.hip
struct GroupedShape {
  int64_t T, k, E, H, I, block_m;
  int64_t max_rows;  // capacity of the sorted-row buffers
};
// scale_mode: 0 channel-wise INT8, 1 block-wise INT8, 2 block-wise FP8 (E4M3 codes in the int8_t
// buffers), 3 W4A8 (packed int4 weights with per-(row, K-block) scales, FP8 activations).
size_t w13_ws_bytes(const GroupedShape& s, int32_t scale_mode);
bool fp8_supported(const GroupedShape& s);  // the FP8 and W4A8 GEMMs' shape limits
size_t w2_ws_bytes(const GroupedShape& s, int32_t scale_mode);
// GEMM engines (the values of w8a8_moe_engine in the C ABI).
constexpr int32_t kEngineStaged = 0, kEngineDma = 1, kEngineRing = 2, kEngineStream = 3;
int32_t engine_of(const GroupedShape& s, int32_t scale_mode);  // the same engine for both GEMMs of a layer
size_t i32_ws_bytes(const GroupedShape& s);
hipError_t gemm_i32(const GroupedShape& s, int32_t gather, const int8_t* a, const int8_t* w, const int32_t* sorted,
                    const int32_t* padded_offsets, const int32_t* tile_expert, const int32_t* num_tiles, int32_t* out,
                    void* ws, hipStream_t stream);
hipError_t w13_silu(const GroupedShape& s, int32_t scale_mode, const int8_t* a_q, const float* a_s,
                    const int8_t* w13, const float* w13_s, const int32_t* sorted, const int32_t* padded_offsets,
                    const int32_t* tile_expert, const int32_t* num_tiles, int8_t* h_q, float* h_s, void* ws,
                    hipStream_t stream);
hipError_t w2_combine(const GroupedShape& s, int32_t scale_mode, const int8_t* h_q, const float* h_s,
                      const int8_t* w2, const float* w2_s, const int32_t* sorted, const int32_t* padded_offsets,
                      const int32_t* tile_expert, const int32_t* num_tiles, const float* topk_w, float* out,
                      void* ws, hipStream_t stream);

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K);
bool linear_supported(int64_t M, int64_t N, int64_t K);
hipError_t linear(const int8_t* a_q, const float* a_s, const int8_t* w, const float* w_s, int64_t M, int64_t N,
                  int64_t K, float* out, void* ws, hipStream_t stream);

}  // namespace w8a8
