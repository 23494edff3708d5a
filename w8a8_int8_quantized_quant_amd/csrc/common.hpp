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

// FP8 rule (E4M3 as the OCP 8-bit floating-point specification defines it: bias 7, 3 mantissa
// bits, largest finite 448): scale = max(max|x| / 448, 1e-8); code = the E4M3 value nearest to
// x / scale, ties to even, after clamping x / scale to [-448, 448].  v_cvt_pk_fp8_f32 rounds to
// nearest even and keeps the sign of a zero result; the clamp keeps it off the NaN encoding.
__device__ __forceinline__ float fp8_scale(float amax) {
  float s = amax / 448.0f;
  return s < 1e-8f ? 1e-8f : s;
}
__device__ __forceinline__ float fp8_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
// Two codes into bytes 0-1 (HI = false) or 2-3 (HI = true) of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pack2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), (int)old, HI);
}
__device__ __forceinline__ uint8_t fp8_value(float x, float s) {
  const float v = x / s;
  return (uint8_t)(fp8_pack2<false>(v, v, 0u) & 0xFFu);
}

// Int4 weight rule (the W4A8 path): scale = max(max|x| / 7, 1e-8); q = clamp(rne(x / scale), -7, 7),
// IEEE division; stored as a nibble of sign (bit 3) and magnitude (bits 0-2), zero as 0.
__device__ __forceinline__ float w4_scale(float amax) {
  float s = amax / 7.0f;
  return s < 1e-8f ? 1e-8f : s;
}
__device__ __forceinline__ uint32_t w4_nibble(float x, float s) {
  float v = __builtin_rintf(x / s);
  v = v > 7.0f ? 7.0f : v;
  v = v < -7.0f ? -7.0f : v;
  const int q = (int)v;
  return q < 0 ? (uint32_t)(8 | -q) : (uint32_t)q;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Maximum over each 16-lane DPP row, left in every lane of the row: partner lanes l^1 and l^2 (quad
// permutes), then the mirrored lane in the 8-lane half and in the row.  Max is order-free, so this
// equals any other reduction order.  The whole wavefront must be active.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_max_step(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF,
                                                             false)));
}
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  return dpp_max_step<0x140>(v);  // row_mirror
}

// Mask of lanes below the calling lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace w8a8
