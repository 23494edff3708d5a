// common.hpp -- device helpers shared by the gfx950 kernels of the W8A8 INT8 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

constexpr int kWave = 64;  // CDNA wavefront width

// Exact widening of a bf16 bit pattern to fp32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Quantization rule shared by activations, weights and the intermediate:
// scale = max(amax / 127, 1e-8); q = clamp(rne(x / scale), -127, 127), IEEE division.
__device__ __forceinline__ float quant_scale(float amax) {
  float s = amax / 127.0f;
  return s < 1e-8f ? 1e-8f : s;
}
__device__ __forceinline__ int8_t quant_value(float x, float s) {
  float v = __builtin_rintf(x / s);
  v = v > 127.0f ? 127.0f : v;
  v = v < -127.0f ? -127.0f : v;
  return (int8_t)(int)v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Mask of lanes below the calling lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace w8a8
