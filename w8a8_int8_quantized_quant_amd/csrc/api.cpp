// api.cpp -- the C ABI (include/w8a8moe.h): host-side validation, workspace
// carving and dispatch to the gfx950 kernels.  Every check runs before anything
// is enqueued, so an invalid call leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/w8a8moe.h"
#include "kernels.hpp"

namespace {

using w8a8::GroupedShape;

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxDim = 65536;
constexpr int64_t kMaxPairs = int64_t(1) << 30;

int32_t hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_HIP_ERROR; }

bool aligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool ok16(const void* p) { return aligned(p, 16); }
bool ok4(const void* p) { return aligned(p, 4); }

bool valid_block_m(int64_t bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

bool valid_dim(int64_t d) { return d >= 128 && d <= kMaxDim && d % 128 == 0; }

bool valid_mode(int32_t m) {
  return m == W8A8_SCALE_CHANNEL || m == W8A8_SCALE_BLOCK128 || m == W8A8_SCALE_FP8_BLOCK128 || m == W8A8_SCALE_W4A8;
}

// FP8 activations (and the ring engine's shape limits): the FP8 and W4A8 modes.
bool fp8_mode(int32_t m) { return m == W8A8_SCALE_FP8_BLOCK128 || m == W8A8_SCALE_W4A8; }

// T, k, E limits shared by every MoE entry point.
int32_t check_tke(int64_t T, int64_t k, int64_t E) {
  if (T < 0 || k < 0 || E < 0) return W8A8_INVALID_ARGUMENT;
  if (E < 1 || E > kMaxE || k < 1 || k > E) return W8A8_UNSUPPORTED_SHAPE;
  if (T > kMaxPairs / k) return W8A8_UNSUPPORTED_SHAPE;
  return W8A8_OK;
}

int64_t max_rows_of(int64_t T, int64_t k, int64_t E, int64_t bm) {
  const int64_t P = T * k;
  const int64_t nonempty = std::min(E, P);
  return (P + nonempty * (bm - 1)) / bm * bm;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Arguments common to the grouped GEMM entry points.
int32_t check_grouped(const int32_t* sorted, const int32_t* padded_offsets, const int32_t* tile_expert,
                      const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H, int64_t I,
                      int64_t block_m) {
  int32_t st = check_tke(T, k, E);
  if (st) return st;
  if (!ok4(sorted) || !ok4(padded_offsets) || !ok4(tile_expert) || !ok4(num_tiles)) return W8A8_INVALID_ARGUMENT;
  if (H < 0 || I < 0 || block_m < 0) return W8A8_INVALID_ARGUMENT;
  if (!valid_dim(H) || !valid_dim(I) || !valid_block_m(block_m)) return W8A8_UNSUPPORTED_SHAPE;
  return W8A8_OK;
}

GroupedShape shape_of(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m) {
  GroupedShape s;
  s.T = T;
  s.k = k;
  s.E = E;
  s.H = H;
  s.I = I;
  s.block_m = block_m;
  s.max_rows = max_rows_of(T, k, E, block_m);
  return s;
}

int32_t route_check(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn, int64_t n_group,
                    int64_t topk_group, const float* bias, const int32_t* ids, const float* w) {
  int32_t st = check_tke(T, k, E);
  if (st) return st;
  if (!ok4(logits) || !ok4(ids) || !ok4(w)) return W8A8_INVALID_ARGUMENT;
  if (bias != nullptr && !ok4(bias)) return W8A8_INVALID_ARGUMENT;
  if (score_fn != W8A8_SCORE_SOFTMAX && score_fn != W8A8_SCORE_SIGMOID) return W8A8_INVALID_ARGUMENT;
  if (n_group < 1 || topk_group < 1) return W8A8_INVALID_ARGUMENT;
  if (score_fn == W8A8_SCORE_SOFTMAX && (n_group != 1 || bias != nullptr)) return W8A8_INVALID_ARGUMENT;
  if (n_group > 64 || E % n_group != 0 || topk_group > n_group) return W8A8_UNSUPPORTED_SHAPE;
  if (k > topk_group * (E / n_group)) return W8A8_UNSUPPORTED_SHAPE;
  return W8A8_OK;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int32_t status) {
  switch (status) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_INVALID_ARGUMENT: return "W8A8_INVALID_ARGUMENT";
    case W8A8_UNSUPPORTED_SHAPE: return "W8A8_UNSUPPORTED_SHAPE";
    case W8A8_WORKSPACE_TOO_SMALL: return "W8A8_WORKSPACE_TOO_SMALL";
    case W8A8_UNSUPPORTED_DTYPE: return "W8A8_UNSUPPORTED_DTYPE";
    case W8A8_HIP_ERROR: return "W8A8_HIP_ERROR";
    default: return "W8A8_UNKNOWN_STATUS";
  }
}

static int32_t quant_entry(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t block_rows,
                           int64_t block_cols, int8_t* q, float* scale, hipStream_t stream, bool fp8) {
  if (rows < 0 || cols < 0 || block_rows < 1 || block_cols < 1) return W8A8_INVALID_ARGUMENT;
  if (x_dtype != W8A8_DTYPE_F32 && x_dtype != W8A8_DTYPE_BF16) return W8A8_UNSUPPORTED_DTYPE;
  if (rows == 0 || cols == 0) return W8A8_OK;
  if (!aligned(x, x_dtype == W8A8_DTYPE_F32 ? 4 : 2) || q == nullptr || !ok4(scale)) return W8A8_INVALID_ARGUMENT;
  const int64_t nb = ((rows + block_rows - 1) / block_rows) * ((cols + block_cols - 1) / block_cols);
  if (rows >= (int64_t(1) << 31) || nb >= (int64_t(1) << 31) || rows * cols >= (int64_t(1) << 40) ||
      (cols + block_cols - 1) / block_cols > w8a8::kMaxGridBlocks)  // one block row fits one launch
    return W8A8_UNSUPPORTED_SHAPE;
  return hip_status(w8a8::quant_blocks(x, x_dtype, rows, cols, block_rows, block_cols, q, scale, stream, fp8));
}

int32_t w8a8_quant_blocks(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t block_rows,
                          int64_t block_cols, int8_t* q, float* scale, hipStream_t stream) {
  return quant_entry(x, x_dtype, rows, cols, block_rows, block_cols, q, scale, stream, false);
}

int32_t w8a8_fp8_quant_blocks(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t block_rows,
                              int64_t block_cols, uint8_t* q, float* scale, hipStream_t stream) {
  return quant_entry(x, x_dtype, rows, cols, block_rows, block_cols, reinterpret_cast<int8_t*>(q), scale, stream,
                     true);
}

int32_t w8a8_w4a8_quant_weights(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, uint8_t* q,
                                float* scale, hipStream_t stream) {
  if (rows < 0 || cols < 0) return W8A8_INVALID_ARGUMENT;
  if (x_dtype != W8A8_DTYPE_F32 && x_dtype != W8A8_DTYPE_BF16) return W8A8_UNSUPPORTED_DTYPE;
  if (cols % 128 != 0) return W8A8_UNSUPPORTED_SHAPE;
  if (rows == 0 || cols == 0) return W8A8_OK;
  if (!aligned(x, x_dtype == W8A8_DTYPE_F32 ? 4 : 2) || q == nullptr || !ok4(scale)) return W8A8_INVALID_ARGUMENT;
  if (rows >= (int64_t(1) << 31) || rows * cols >= (int64_t(1) << 40) || cols / 128 > w8a8::kMaxGridBlocks)
    return W8A8_UNSUPPORTED_SHAPE;
  return hip_status(w8a8::quant_w4(x, x_dtype, rows, cols, q, scale, stream));
}

int32_t w8a8_quant_per_token(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t group, int8_t* q,
                             float* scale, hipStream_t stream) {
  if (group < 0 || cols < 0) return W8A8_INVALID_ARGUMENT;
  if (group > 0 && cols % group != 0) return W8A8_UNSUPPORTED_SHAPE;
  if (cols == 0) return rows < 0 ? W8A8_INVALID_ARGUMENT : W8A8_OK;
  return w8a8_quant_blocks(x, x_dtype, rows, cols, 1, group == 0 ? cols : group, q, scale, stream);
}

int32_t moe_topk_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn, int64_t n_group,
                       int64_t topk_group, int32_t renormalize, float routed_scaling, const float* correction_bias,
                       int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (T == 0 && E >= 1 && k >= 1 && k <= E) return W8A8_OK;
  int32_t st = route_check(logits, T, E, k, score_fn, n_group, topk_group, correction_bias, topk_ids, topk_weights);
  if (st) return st;
  return hip_status(w8a8::topk_route(logits, T, E, k, score_fn, n_group, topk_group, renormalize, routed_scaling,
                                     correction_bias, topk_ids, topk_weights, stream));
}

int64_t w8a8_moe_max_rows(int64_t T, int64_t k, int64_t E, int64_t block_m) {
  if (check_tke(T, k, E) || !valid_block_m(block_m)) return -1;
  return max_rows_of(T, k, E, block_m);
}

size_t moe_align_workspace_bytes(int64_t T, int64_t k, int64_t E) {
  if (check_tke(T, k, E)) return 0;
  return w8a8::align_ws_bytes(T * k, E);
}

int32_t moe_align_by_expert(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                            int32_t* expert_counts, int32_t* expert_offsets, int32_t* padded_offsets,
                            int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* num_tiles, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_tke(T, k, E);
  if (st) return st;
  if (block_m < 0) return W8A8_INVALID_ARGUMENT;
  if (!valid_block_m(block_m)) return W8A8_UNSUPPORTED_SHAPE;
  if (!ok4(expert_counts) || !ok4(expert_offsets) || !ok4(padded_offsets) || !ok4(num_tiles))
    return W8A8_INVALID_ARGUMENT;
  const int64_t P = T * k;
  if (P > 0 && (!ok4(topk_ids) || !ok4(sorted_pair_ids) || !ok4(tile_expert))) return W8A8_INVALID_ARGUMENT;
  const size_t need = w8a8::align_ws_bytes(P, E);
  if (ws_bytes < need) return W8A8_WORKSPACE_TOO_SMALL;
  if (need > 0 && !aligned(ws, 256)) return W8A8_INVALID_ARGUMENT;
  const int64_t mr = max_rows_of(T, k, E, block_m);
  return hip_status(w8a8::align_by_expert(topk_ids, P, E, block_m, expert_counts, expert_offsets, padded_offsets,
                                          sorted_pair_ids, tile_expert, num_tiles, mr / block_m, ws, stream));
}

int32_t moe_align_by_expert_noalloc(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int64_t block_m,
                                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* padded_offsets,
                                    int32_t* sorted_pair_ids, int32_t* tile_expert, int32_t* num_tiles,
                                    hipStream_t stream) {
  int32_t st = check_tke(T, k, E);
  if (st) return st;
  if (block_m < 0) return W8A8_INVALID_ARGUMENT;
  if (!valid_block_m(block_m)) return W8A8_UNSUPPORTED_SHAPE;
  if (!ok4(expert_counts) || !ok4(expert_offsets) || !ok4(padded_offsets) || !ok4(num_tiles))
    return W8A8_INVALID_ARGUMENT;
  const int64_t P = T * k;
  if (P > 0 && (!ok4(topk_ids) || !ok4(sorted_pair_ids) || !ok4(tile_expert))) return W8A8_INVALID_ARGUMENT;
  if (w8a8::align_ws_bytes(P, E) > w8a8::kNoAllocScratchBytes) return W8A8_UNSUPPORTED_SHAPE;
  void* scratch = nullptr;
  hipError_t e = w8a8::noalloc_scratch(&scratch);
  if (e != hipSuccess) return W8A8_HIP_ERROR;
  const int64_t mr = max_rows_of(T, k, E, block_m);
  return hip_status(w8a8::align_by_expert(topk_ids, P, E, block_m, expert_counts, expert_offsets, padded_offsets,
                                          sorted_pair_ids, tile_expert, num_tiles, mr / block_m, scratch, stream));
}

size_t moe_align_noalloc_scratch_bytes(void) { return w8a8::kNoAllocScratchBytes; }

// Shape of the layer whose first (gather = 1: N = 2I, K = H) or second (gather = 0: N = H, K = I) GEMM
// the raw int32 entry runs.
static int32_t i32_shape(int32_t gather, int64_t N, int64_t K, int64_t T, int64_t k, int64_t E, int64_t block_m,
                         GroupedShape* s) {
  int32_t st = check_tke(T, k, E);
  if (st) return st;
  if (N < 0 || K < 0 || block_m < 0 || (gather != 0 && gather != 1)) return W8A8_INVALID_ARGUMENT;
  const int64_t H = gather ? K : N, I = gather ? N / 2 : K;
  if ((gather && N % 2) || !valid_dim(H) || !valid_dim(I) || !valid_block_m(block_m)) return W8A8_UNSUPPORTED_SHAPE;
  *s = shape_of(T, k, E, H, I, block_m);
  return W8A8_OK;
}

size_t w8a8_grouped_gemm_i32_workspace_bytes(int32_t gather, int64_t N, int64_t K, int64_t T, int64_t k, int64_t E,
                                             int64_t block_m) {
  GroupedShape s;
  if (i32_shape(gather, N, K, T, k, E, block_m, &s)) return 0;
  return w8a8::i32_ws_bytes(s);
}

int32_t w8a8_grouped_gemm_i32(const int8_t* a, int32_t gather, const int8_t* w, int64_t N, int64_t K,
                              const int32_t* sorted_pair_ids, const int32_t* padded_offsets,
                              const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int64_t k, int64_t E,
                              int64_t block_m, int32_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  GroupedShape s;
  int32_t st = i32_shape(gather, N, K, T, k, E, block_m, &s);
  if (st) return st;
  if (T == 0) return W8A8_OK;
  if (!ok16(a) || !ok16(w) || !ok16(out) || !ok4(sorted_pair_ids) || !ok4(padded_offsets) || !ok4(tile_expert) ||
      !ok4(num_tiles))
    return W8A8_INVALID_ARGUMENT;
  if (ws_bytes < w8a8::i32_ws_bytes(s)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return W8A8_INVALID_ARGUMENT;
  return hip_status(w8a8::gemm_i32(s, gather, a, w, sorted_pair_ids, padded_offsets, tile_expert, num_tiles, out,
                                   ws, stream));
}

int32_t w8a8_moe_engine(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m, int32_t scale_mode) {
  if (check_tke(T, k, E) || !valid_dim(H) || !valid_dim(I) || !valid_block_m(block_m) || !valid_mode(scale_mode))
    return -1;
  const GroupedShape s = shape_of(T, k, E, H, I, block_m);
  if (fp8_mode(scale_mode) && !w8a8::fp8_supported(s)) return -1;
  return w8a8::engine_of(s, scale_mode);
}

size_t w8a8_w13_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                                int32_t scale_mode) {
  if (check_tke(T, k, E) || !valid_dim(H) || !valid_dim(I) || !valid_block_m(block_m) || !valid_mode(scale_mode))
    return 0;
  const GroupedShape s = shape_of(T, k, E, H, I, block_m);
  if (fp8_mode(scale_mode) && !w8a8::fp8_supported(s)) return 0;
  return w8a8::w13_ws_bytes(s, scale_mode);
}

size_t w8a8_w2_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                               int32_t scale_mode) {
  if (check_tke(T, k, E) || !valid_dim(H) || !valid_dim(I) || !valid_block_m(block_m) || !valid_mode(scale_mode))
    return 0;
  const GroupedShape s = shape_of(T, k, E, H, I, block_m);
  if (fp8_mode(scale_mode) && !w8a8::fp8_supported(s)) return 0;
  return w8a8::w2_ws_bytes(s, scale_mode);
}

static int32_t w13_entry(int32_t mode, const int8_t* a_q, const float* a_scale, const int8_t* w13,
                         const float* w13_scale, const int32_t* sorted, const int32_t* padded_offsets,
                         const int32_t* tile_expert, const int32_t* num_tiles, int64_t T, int64_t k, int64_t E,
                         int64_t H, int64_t I, int64_t block_m, int8_t* h_q, float* h_scale, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_grouped(sorted, padded_offsets, tile_expert, num_tiles, T, k, E, H, I, block_m);
  if (st) return st;
  const GroupedShape s = shape_of(T, k, E, H, I, block_m);
  if (fp8_mode(mode) && !w8a8::fp8_supported(s)) return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!ok16(a_q) || !ok4(a_scale) || !ok16(w13) || !ok4(w13_scale) || !ok16(h_q) || !ok4(h_scale))
    return W8A8_INVALID_ARGUMENT;
  const size_t need = w8a8::w13_ws_bytes(s, mode);
  if (ws_bytes < need) return W8A8_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return W8A8_INVALID_ARGUMENT;
  return hip_status(w8a8::w13_silu(s, mode, a_q, a_scale, w13, w13_scale, sorted, padded_offsets, tile_expert,
                                   num_tiles, h_q, h_scale, ws, stream));
}

static int32_t w2_entry(int32_t mode, const int8_t* h_q, const float* h_scale, const int8_t* w2,
                        const float* w2_scale, const int32_t* sorted, const int32_t* padded_offsets,
                        const int32_t* tile_expert, const int32_t* num_tiles, const float* topk_weights, int64_t T,
                        int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_grouped(sorted, padded_offsets, tile_expert, num_tiles, T, k, E, H, I, block_m);
  if (st) return st;
  const GroupedShape s = shape_of(T, k, E, H, I, block_m);
  if (fp8_mode(mode) && !w8a8::fp8_supported(s)) return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!ok16(h_q) || !ok4(h_scale) || !ok16(w2) || !ok4(w2_scale) || !ok4(topk_weights) || !ok16(out))
    return W8A8_INVALID_ARGUMENT;
  const size_t need = w8a8::w2_ws_bytes(s, mode);
  if (ws_bytes < need) return W8A8_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return W8A8_INVALID_ARGUMENT;
  return hip_status(w8a8::w2_combine(s, mode, h_q, h_scale, w2, w2_scale, sorted, padded_offsets, tile_expert,
                                     num_tiles, topk_weights, out, ws, stream));
}

int32_t w8a8_grouped_gemm_w13_silu(const int8_t* a_q, const float* a_scale, const int8_t* w13,
                                   const float* w13_scale, const int32_t* sorted_pair_ids,
                                   const int32_t* padded_offsets, const int32_t* tile_expert,
                                   const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H, int64_t I,
                                   int64_t block_m, int8_t* h_q, float* h_scale, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return w13_entry(W8A8_SCALE_CHANNEL, a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                   num_tiles, T, k, E, H, I, block_m, h_q, h_scale, ws, ws_bytes, stream);
}

int32_t w8a8_block_grouped_gemm_w13_silu(const int8_t* a_q, const float* a_scale, const int8_t* w13,
                                         const float* w13_scale, const int32_t* sorted_pair_ids,
                                         const int32_t* padded_offsets, const int32_t* tile_expert,
                                         const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                         int64_t I, int64_t block_m, int8_t* h_q, float* h_scale, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return w13_entry(W8A8_SCALE_BLOCK128, a_q, a_scale, w13, w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                   num_tiles, T, k, E, H, I, block_m, h_q, h_scale, ws, ws_bytes, stream);
}

int32_t w8a8_grouped_gemm_w2_combine(const int8_t* h_q, const float* h_scale, const int8_t* w2,
                                     const float* w2_scale, const int32_t* sorted_pair_ids,
                                     const int32_t* padded_offsets, const int32_t* tile_expert,
                                     const int32_t* num_tiles, const float* topk_weights, int64_t T, int64_t k,
                                     int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  return w2_entry(W8A8_SCALE_CHANNEL, h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                  num_tiles, topk_weights, T, k, E, H, I, block_m, out, ws, ws_bytes, stream);
}

int32_t w8a8_block_grouped_gemm_w2_combine(const int8_t* h_q, const float* h_scale, const int8_t* w2,
                                           const float* w2_scale, const int32_t* sorted_pair_ids,
                                           const int32_t* padded_offsets, const int32_t* tile_expert,
                                           const int32_t* num_tiles, const float* topk_weights, int64_t T,
                                           int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m, float* out,
                                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return w2_entry(W8A8_SCALE_BLOCK128, h_q, h_scale, w2, w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                  num_tiles, topk_weights, T, k, E, H, I, block_m, out, ws, ws_bytes, stream);
}

int32_t w8a8_fp8_grouped_gemm_w13_silu(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                       const float* w13_scale, const int32_t* sorted_pair_ids,
                                       const int32_t* padded_offsets, const int32_t* tile_expert,
                                       const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                       int64_t I, int64_t block_m, uint8_t* h_q, float* h_scale, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  return w13_entry(W8A8_SCALE_FP8_BLOCK128, reinterpret_cast<const int8_t*>(a_q), a_scale,
                   reinterpret_cast<const int8_t*>(w13), w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                   num_tiles, T, k, E, H, I, block_m, reinterpret_cast<int8_t*>(h_q), h_scale, ws, ws_bytes, stream);
}

int32_t w8a8_fp8_grouped_gemm_w2_combine(const uint8_t* h_q, const float* h_scale, const uint8_t* w2,
                                         const float* w2_scale, const int32_t* sorted_pair_ids,
                                         const int32_t* padded_offsets, const int32_t* tile_expert,
                                         const int32_t* num_tiles, const float* topk_weights, int64_t T, int64_t k,
                                         int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return w2_entry(W8A8_SCALE_FP8_BLOCK128, reinterpret_cast<const int8_t*>(h_q), h_scale,
                  reinterpret_cast<const int8_t*>(w2), w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                  num_tiles, topk_weights, T, k, E, H, I, block_m, out, ws, ws_bytes, stream);
}

int32_t w8a8_w4a8_grouped_gemm_w13_silu(const uint8_t* a_q, const float* a_scale, const uint8_t* w13,
                                        const float* w13_scale, const int32_t* sorted_pair_ids,
                                        const int32_t* padded_offsets, const int32_t* tile_expert,
                                        const int32_t* num_tiles, int64_t T, int64_t k, int64_t E, int64_t H,
                                        int64_t I, int64_t block_m, uint8_t* h_q, float* h_scale, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  return w13_entry(W8A8_SCALE_W4A8, reinterpret_cast<const int8_t*>(a_q), a_scale,
                   reinterpret_cast<const int8_t*>(w13), w13_scale, sorted_pair_ids, padded_offsets, tile_expert,
                   num_tiles, T, k, E, H, I, block_m, reinterpret_cast<int8_t*>(h_q), h_scale, ws, ws_bytes, stream);
}

int32_t w8a8_w4a8_grouped_gemm_w2_combine(const uint8_t* h_q, const float* h_scale, const uint8_t* w2,
                                          const float* w2_scale, const int32_t* sorted_pair_ids,
                                          const int32_t* padded_offsets, const int32_t* tile_expert,
                                          const int32_t* num_tiles, const float* topk_weights, int64_t T, int64_t k,
                                          int64_t E, int64_t H, int64_t I, int64_t block_m, float* out, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  return w2_entry(W8A8_SCALE_W4A8, reinterpret_cast<const int8_t*>(h_q), h_scale,
                  reinterpret_cast<const int8_t*>(w2), w2_scale, sorted_pair_ids, padded_offsets, tile_expert,
                  num_tiles, topk_weights, T, k, E, H, I, block_m, out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------------------- composite

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 1 || K < 1 || N > kMaxPairs || K > kMaxDim || M > kMaxPairs || !w8a8::linear_supported(M, N, K))
    return 0;
  return w8a8::linear_ws_bytes(M, N, K);
}

int32_t w8a8_linear(const int8_t* a_q, const float* a_scale, const int8_t* w, const float* w_scale, int64_t M,
                    int64_t N, int64_t K, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W8A8_INVALID_ARGUMENT;
  if (N == 0 || K == 0 || N > kMaxPairs || K > kMaxDim || M > kMaxPairs || !w8a8::linear_supported(M, N, K))
    return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!ok16(a_q) || !ok4(a_scale) || !ok16(w) || !ok4(w_scale) || !ok16(out) || !aligned(ws, 4))
    return W8A8_INVALID_ARGUMENT;
  if (ws_bytes < w8a8::linear_ws_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  return hip_status(w8a8::linear(a_q, a_scale, w, w_scale, M, N, K, out, ws, stream));
}

int64_t w8a8_moe_pick_block_m(int64_t T, int64_t k, int64_t E) {
  if (check_tke(T, k, E)) return -1;
  const int64_t avg = (T * k + E - 1) / E;
  if (avg <= 16) return 16;
  if (avg <= 32) return 32;
  if (avg <= 96) return 64;
  return 128;
}

namespace {

struct Layout {
  size_t ids, tw, a_q, a_s, counts, offsets, padded, sorted, tile_expert, num_tiles, align_ws, h_q, h_s, gemm_ws,
      total;
  int64_t max_rows;
};

Layout layout_of(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t bm, int32_t mode) {
  Layout L{};
  const int64_t P = T * k;
  const GroupedShape s = shape_of(T, k, E, H, I, bm);
  L.max_rows = s.max_rows;
  const bool block = mode != W8A8_SCALE_CHANNEL;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += round256(bytes);
    return at;
  };
  L.ids = take(sizeof(int32_t) * P);
  L.tw = take(sizeof(float) * P);
  L.a_q = take((size_t)(T * H));
  L.a_s = take(sizeof(float) * (size_t)(T * (block ? H / 128 : 1)));
  L.counts = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 1));
  L.padded = take(sizeof(int32_t) * (E + 1));
  L.sorted = take(sizeof(int32_t) * (size_t)std::max<int64_t>(s.max_rows, 1));
  L.tile_expert = take(sizeof(int32_t) * (size_t)std::max<int64_t>(s.max_rows / bm, 1));
  L.num_tiles = take(sizeof(int32_t));
  L.align_ws = take(w8a8::align_ws_bytes(P, E));
  L.h_q = take((size_t)(s.max_rows * I));
  L.h_s = take(sizeof(float) * (size_t)(s.max_rows * (block ? I / 128 : 1)));
  L.gemm_ws = take(std::max(w8a8::w13_ws_bytes(s, mode), w8a8::w2_ws_bytes(s, mode)));
  L.total = off;
  return L;
}

}  // namespace

size_t w8a8_moe_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I, int64_t block_m,
                                int32_t scale_mode) {
  if (check_tke(T, k, E) || !valid_dim(H) || !valid_dim(I)) return 0;
  if (block_m == 0) block_m = w8a8_moe_pick_block_m(T, k, E);
  if (!valid_block_m(block_m)) return 0;
  if (!valid_mode(scale_mode)) return 0;
  if (fp8_mode(scale_mode) && !w8a8::fp8_supported(shape_of(T, k, E, H, I, block_m))) return 0;
  return layout_of(T, k, E, H, I, block_m, scale_mode).total;
}

int32_t w8a8_moe_forward(const struct w8a8_moe_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a == nullptr) return W8A8_INVALID_ARGUMENT;
  int32_t st = check_tke(a->T, a->k, a->E);
  if (st) return st;
  if (a->H < 0 || a->I < 0 || a->block_m < 0) return W8A8_INVALID_ARGUMENT;
  if (!valid_dim(a->H) || !valid_dim(a->I)) return W8A8_UNSUPPORTED_SHAPE;
  if (!valid_mode(a->scale_mode)) return W8A8_INVALID_ARGUMENT;
  if (a->x_dtype != W8A8_DTYPE_F32 && a->x_dtype != W8A8_DTYPE_BF16) return W8A8_UNSUPPORTED_DTYPE;
  const int64_t bm = a->block_m == 0 ? w8a8_moe_pick_block_m(a->T, a->k, a->E) : a->block_m;
  if (!valid_block_m(bm)) return W8A8_UNSUPPORTED_SHAPE;
  if (fp8_mode(a->scale_mode) && !w8a8::fp8_supported(shape_of(a->T, a->k, a->E, a->H, a->I, bm)))
    return W8A8_UNSUPPORTED_SHAPE;
  if (a->T == 0) return W8A8_OK;
  st = route_check(a->router_logits, a->T, a->E, a->k, a->score_fn, a->n_group, a->topk_group, a->correction_bias,
                   a->topk_ids ? a->topk_ids : reinterpret_cast<int32_t*>(16),
                   a->topk_weights ? a->topk_weights : reinterpret_cast<float*>(16));
  if (st) return st;
  if (!aligned(a->x, a->x_dtype == W8A8_DTYPE_F32 ? 4 : 2) || !ok16(a->w13) || !ok4(a->w13_scale) || !ok16(a->w2) ||
      !ok4(a->w2_scale) || !ok16(a->out))
    return W8A8_INVALID_ARGUMENT;
  const Layout L = layout_of(a->T, a->k, a->E, a->H, a->I, bm, a->scale_mode);
  if (ws_bytes < L.total) return W8A8_WORKSPACE_TOO_SMALL;
  if (!aligned(ws, 256)) return W8A8_INVALID_ARGUMENT;

  char* base = static_cast<char*>(ws);
  int32_t* ids = a->topk_ids ? a->topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
  float* tw = a->topk_weights ? a->topk_weights : reinterpret_cast<float*>(base + L.tw);
  int8_t* a_q = reinterpret_cast<int8_t*>(base + L.a_q);
  float* a_s = reinterpret_cast<float*>(base + L.a_s);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* padded = reinterpret_cast<int32_t*>(base + L.padded);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  int32_t* tile_expert = reinterpret_cast<int32_t*>(base + L.tile_expert);
  int32_t* num_tiles = reinterpret_cast<int32_t*>(base + L.num_tiles);
  int8_t* h_q = reinterpret_cast<int8_t*>(base + L.h_q);
  float* h_s = reinterpret_cast<float*>(base + L.h_s);
  void* gws = base + L.gemm_ws;
  const bool block = a->scale_mode != W8A8_SCALE_CHANNEL;
  const bool fp8 = fp8_mode(a->scale_mode);
  const GroupedShape s = shape_of(a->T, a->k, a->E, a->H, a->I, bm);

  hipError_t e = w8a8::topk_route(a->router_logits, a->T, a->E, a->k, a->score_fn, a->n_group, a->topk_group,
                                  a->renormalize, a->routed_scaling, a->correction_bias, ids, tw, stream);
  if (e == hipSuccess)
    e = w8a8::quant_blocks(a->x, a->x_dtype, a->T, a->H, 1, block ? 128 : a->H, a_q, a_s, stream, fp8);
  if (e == hipSuccess)
    e = w8a8::align_by_expert(ids, a->T * a->k, a->E, bm, counts, offsets, padded, sorted, tile_expert, num_tiles,
                              L.max_rows / bm, base + L.align_ws, stream);
  if (e == hipSuccess)
    e = w8a8::w13_silu(s, a->scale_mode, a_q, a_s, a->w13, a->w13_scale, sorted, padded, tile_expert, num_tiles,
                       h_q, h_s, gws, stream);
  if (e == hipSuccess)
    e = w8a8::w2_combine(s, a->scale_mode, h_q, h_s, a->w2, a->w2_scale, sorted, padded, tile_expert, num_tiles,
                         tw, a->out, gws, stream);
  return hip_status(e);
}

}  // extern "C"
