// synth_dev.hip -- device (gfx950) fills of the seeded synthetic inputs.
// Same element definitions as synth_host.c (both compile synth_core.h), so a
// tensor drawn here is bit-identical to the host draw; used to fill the
// multi-GB expert weights directly in HBM.
#include <hip/hip_runtime.h>

#include "synth_core.h"

#define SYNTH_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kThreads = 256;

__global__ void fill_normal_kernel(float* __restrict__ out, int64_t n, uint64_t base, int64_t start,
                                   float sigma) {
  int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    out[i] = synth_normal(base, (uint64_t)(start + i)) * sigma;
}

__global__ void fill_logits_kernel(float* __restrict__ out, int64_t T, int64_t E, uint64_t base,
                                   const float* __restrict__ bias, int64_t row_start) {
  int64_t n = T * E;
  int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    int64_t e = i % E;
    float z = synth_normal(base, (uint64_t)(row_start * E + i));
    out[i] = bias ? z + bias[e] : z;
  }
}

__global__ void fill_activation_kernel(void* __restrict__ out, int32_t dtype, int64_t rows, int64_t cols,
                                       uint64_t bx, uint64_t bo, float sigma, uint32_t thr, float mult,
                                       int64_t row_start) {
  int64_t n = rows * cols;
  int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float v = synth_activation(bx, bo, (uint64_t)(row_start * cols + i), sigma, thr, mult);
    if (dtype == 1)
      ((uint16_t*)out)[i] = synth_f32_to_bf16(v);
    else
      ((float*)out)[i] = v;
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : 5; }

}  // namespace

// Returns 0 on success, 5 if the launch failed.
SYNTH_EXPORT int synth_dev_fill_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream,
                                           int64_t start, float sigma, hipStream_t s) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, out, n,
                     synth_base(seed, stream), start, sigma);
  return status_of(hipGetLastError());
}

SYNTH_EXPORT int synth_dev_fill_logits_f32(float* out, int64_t T, int64_t E, uint64_t seed,
                                           const float* bias, int64_t row_start, hipStream_t s) {
  if (T * E <= 0) return 0;
  hipLaunchKernelGGL(fill_logits_kernel, dim3(grid_for(T * E)), dim3(kThreads), 0, s, out, T, E,
                     synth_base(seed, SYNTH_STREAM_LOGITS), bias, row_start);
  return status_of(hipGetLastError());
}

SYNTH_EXPORT int synth_dev_fill_activation(void* out, int32_t dtype, int64_t rows, int64_t cols,
                                           uint64_t seed, float sigma, uint32_t outlier_threshold,
                                           float mult, int64_t row_start, hipStream_t s) {
  if (rows * cols <= 0) return 0;
  hipLaunchKernelGGL(fill_activation_kernel, dim3(grid_for(rows * cols)), dim3(kThreads), 0, s, out,
                     dtype, rows, cols, synth_base(seed, SYNTH_STREAM_X),
                     synth_base(seed, SYNTH_STREAM_X_OUTLIER), sigma, outlier_threshold, mult, row_start);
  return status_of(hipGetLastError());
}
