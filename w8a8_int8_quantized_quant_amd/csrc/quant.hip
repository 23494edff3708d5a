// quant.hip -- symmetric INT8, FP8 (E4M3) and packed int4 quantization kernels (gfx950).
//
// Online activation quantization, one scale per token or per token-group
// (jiqizhixin article on Meituan's INT8 DeepSeek R1, "Quantization
// exploration"), and the offline weight quantization with one scale per
// output channel or per 128 x 128 block.  INT8 rule: scale = max(max|x|/127,
// 1e-8), q = clamp(rne(x / scale)).  FP8 (SGLang PR #8273: per-block FP8
// weights, per-token-group FP8 activations): scale = max(max|x|/448, 1e-8), q =
// the nearest E4M3 code of x / scale.  Int4 weights (SGLang PR #8311, w4a8):
// scale = max(max|x|/7, 1e-8) per (row, 128 columns), q = clamp(rne(x / scale)).
// The max is order-independent and the division is IEEE, so results are
// bit-exact regardless of how lanes split the work.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) m = fmaxf(m, red[i]);
  return m;
}

// Eight consecutive inputs as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The two code formats: scale rule, one code, four codes packed into a word.
struct Int8Codec {
  static __device__ __forceinline__ float scale(float amax) { return quant_scale(amax); }
  static __device__ __forceinline__ int8_t code(float x, float s) { return quant_value(x, s); }
  static __device__ __forceinline__ uint32_t pack4(const float* v, float s) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (uint32_t)(uint8_t)quant_value(v[i], s) << (8 * i);
    return w;
  }
};
struct Fp8Codec {
  static __device__ __forceinline__ float scale(float amax) { return fp8_scale(amax); }
  static __device__ __forceinline__ int8_t code(float x, float s) { return (int8_t)fp8_value(x, s); }
  static __device__ __forceinline__ uint32_t pack4(const float* v, float s) {
    const uint32_t w = fp8_pack2<false>(v[0] / s, v[1] / s, 0u);
    return fp8_pack2<true>(v[2] / s, v[3] / s, w);
  }
};

// One workgroup per row; cols % 8 == 0 and 16-byte aligned rows: 16-byte loads, 8-byte stores.
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void quant_rows_vec_kernel(const T* __restrict__ x, int64_t cols,
                                                                  int8_t* __restrict__ q,
                                                                  float* __restrict__ scale) {
  __shared__ float red[kThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * cols;
  int8_t* qr = q + row * cols;
  const int64_t nchunk = cols / 8;
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < nchunk; c += kThreads) {
    float v[8];
    load8(xr + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  const float s = C::scale(block_max(amax, red));
  if (threadIdx.x == 0) scale[row] = s;
  for (int64_t c = threadIdx.x; c < nchunk; c += kThreads) {
    float v[8];
    load8(xr + c * 8, v);
    *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(C::pack4(v, s), C::pack4(v + 4, s));
  }
}

// One workgroup per row of at most kRegChunks * kThreads * 8 columns (8192): every thread loads
// all of its 16-byte chunks before the row maximum, and quantizes them from registers, so a row
// costs one round of loads instead of a dependent load per chunk and a second pass.
constexpr int kRegChunks = 4;
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void quant_rows_reg_kernel(const T* __restrict__ x, int64_t cols,
                                                                  int8_t* __restrict__ q,
                                                                  float* __restrict__ scale) {
  __shared__ float red[kThreads / kWave];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * cols;
  int8_t* qr = q + row * cols;
  const int nchunk = (int)(cols / 8);
  float v[kRegChunks][8];
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < nchunk) {
      load8(xr + (int64_t)c * 8, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
  const float s = C::scale(block_max(amax, red));
  if (threadIdx.x == 0) scale[row] = s;
#pragma unroll
  for (int i = 0; i < kRegChunks; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < nchunk)
      *reinterpret_cast<uint2*>(qr + (int64_t)c * 8) = make_uint2(C::pack4(v[i], s), C::pack4(v[i] + 4, s));
  }
}

// Groups of 128 columns (the per-token groups of the block-wise layouts): a group is one 16-lane
// DPP row, each lane holding 8 consecutive values from one 16-byte load, so the group maximum is
// four DPP steps inside the row and the values are quantized from registers (one pass, 8-byte
// stores).  cols % 128 == 0, 16-byte aligned rows.
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void quant_group128_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                                  int8_t* __restrict__ q,
                                                                  float* __restrict__ scale) {
  const int64_t ngroups = cols / 128;
  const int64_t g = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / 16;  // group, row-major
  const int j = (int)(threadIdx.x % 16);
  const bool in = g < rows * ngroups;
  const int64_t base = in ? (g / ngroups) * cols + (g % ngroups) * 128 + j * 8 : 0;
  float v[8];
  if (in) {
    load8(x + base, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const float s = C::scale(row16_max(amax));  // every lane takes part in the DPP steps
  if (in) {
    if (j == 0) scale[g] = s;
    *reinterpret_cast<uint2*>(q + base) = make_uint2(C::pack4(v, s), C::pack4(v + 4, s));
  }
}

// One wave per (row, group) for groups of up to a few hundred columns.
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void quant_groups_kernel(const T* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t group,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
  const int64_t ngroups = cols / group;
  const int64_t gid = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (gid >= rows * ngroups) return;
  const int64_t row = gid / ngroups, g = gid % ngroups;
  const int64_t base = row * cols + g * group;
  float amax = 0.0f;
  for (int64_t c = lane_id(); c < group; c += kWave) amax = fmaxf(amax, fabsf(load_as_f32(x, base + c)));
  const float s = C::scale(wave_max(amax));
  if (lane_id() == 0) scale[gid] = s;
  for (int64_t c = lane_id(); c < group; c += kWave) q[base + c] = C::code(load_as_f32(x, base + c), s);
}

// General case: one workgroup per br x bc block (edge blocks may be partial).
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void quant_blocks_kernel(const T* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t br, int64_t bc,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
  __shared__ float red[kThreads / kWave];
  const int64_t nbc = (cols + bc - 1) / bc;
  const int64_t bi = blockIdx.x / nbc, bj = blockIdx.x % nbc;
  const int64_t r0 = bi * br, r1 = min(r0 + br, rows);
  const int64_t c0 = bj * bc, c1 = min(c0 + bc, cols);
  const int64_t w = c1 - c0, n = (r1 - r0) * w;
  float amax = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += kThreads)
    amax = fmaxf(amax, fabsf(load_as_f32(x, (r0 + i / w) * cols + c0 + i % w)));
  const float s = C::scale(block_max(amax, red));
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) {
    const int64_t off = (r0 + i / w) * cols + c0 + i % w;
    q[off] = C::code(load_as_f32(x, off), s);
  }
}

// Packed int4 weights: one wavefront per (row, 128 columns); lane l builds byte l of the group's
// 64, holding value 8 (l / 4) + l % 4 in its low nibble and value 8 (l / 4) + 4 + l % 4 in its
// high nibble (the W4A8 GEMM's packing: 8 consecutive values per 4 bytes).
template <typename T>
__global__ __launch_bounds__(kThreads) void quant_w4_kernel(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t ngroups = cols / 128;
  const int64_t gid = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (gid >= rows * ngroups) return;
  const int64_t row = gid / ngroups, gi = gid % ngroups;
  const int l = lane_id();
  const int64_t base = row * cols + gi * 128 + (l / 4) * 8 + (l % 4);
  const float v0 = load_as_f32(x, base), v1 = load_as_f32(x, base + 4);
  const float s = w4_scale(wave_max(fmaxf(fabsf(v0), fabsf(v1))));
  if (l == 0) scale[gid] = s;
  q[row * (cols / 2) + gi * 64 + l] = (uint8_t)(w4_nibble(v0, s) | (w4_nibble(v1, s) << 4));
}

// Rows go in pieces of at most kMaxGridBlocks workgroups; each piece starts on a row (and on a
// row block), so it is the same quantization of its rows with offset pointers.
template <typename T, typename C>
hipError_t launch_quant(const void* xv, int64_t rows, int64_t cols, int64_t br, int64_t bc, int8_t* q,
                        float* scale, hipStream_t stream) {
  const T* x = static_cast<const T*>(xv);
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(q) % 8 == 0);
  if (br == 1 && bc == cols && cols % 8 == 0 && aligned) {
    const bool reg = cols <= 8 * kThreads * kRegChunks;
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxGridBlocks) {
      const int64_t n = std::min(rows - r0, kMaxGridBlocks);
      if (reg)
        hipLaunchKernelGGL((quant_rows_reg_kernel<T, C>), dim3((uint32_t)n), dim3(kThreads), 0, stream, x + r0 * cols,
                           cols, q + r0 * cols, scale + r0);
      else
        hipLaunchKernelGGL((quant_rows_vec_kernel<T, C>), dim3((uint32_t)n), dim3(kThreads), 0, stream, x + r0 * cols,
                           cols, q + r0 * cols, scale + r0);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  } else if (br == 1 && bc == 128 && cols % 128 == 0 && aligned) {
    const int64_t ngroups = cols / 128;
    const int64_t step = kMaxGridBlocks * (kThreads / 16) / ngroups;  // rows per launch (ngroups <= 2^20)
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
      const int64_t n = std::min(rows - r0, step);
      const int64_t blocks = (n * ngroups * 16 + kThreads - 1) / kThreads;
      hipLaunchKernelGGL((quant_group128_kernel<T, C>), dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                         x + r0 * cols, n, cols, q + r0 * cols, scale + r0 * ngroups);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  } else if (br == 1 && bc <= 512 && cols % bc == 0) {
    const int64_t per_row = cols / bc;  // wavefronts (groups) per row
    const int64_t step = std::max<int64_t>(1, kMaxGridBlocks * (kThreads / kWave) / per_row);
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
      const int64_t n = std::min(rows - r0, step);
      const int64_t blocks = (n * per_row + kThreads / kWave - 1) / (kThreads / kWave);
      hipLaunchKernelGGL((quant_groups_kernel<T, C>), dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                         x + r0 * cols, n, cols, bc, q + r0 * cols, scale + r0 * per_row);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  } else {
    const int64_t nbr = (rows + br - 1) / br, nbc = (cols + bc - 1) / bc;
    const int64_t step = std::max<int64_t>(1, kMaxGridBlocks / nbc);  // row blocks per piece
    for (int64_t b0 = 0; b0 < nbr; b0 += step) {
      const int64_t nb = std::min(nbr - b0, step), r0 = b0 * br;
      hipLaunchKernelGGL((quant_blocks_kernel<T, C>), dim3((uint32_t)(nb * nbc)), dim3(kThreads), 0, stream,
                         x + r0 * cols, std::min(rows - r0, nb * br), cols, br, bc, q + r0 * cols, scale + b0 * nbc);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t quant_w4(const void* x, int32_t dtype, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                    hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t per_row = cols / 128;  // wavefronts (groups) per row
  const int64_t step = std::max<int64_t>(1, kMaxGridBlocks * (kThreads / kWave) / per_row);
  const size_t esize = dtype == 1 ? 2 : 4;
  for (int64_t r0 = 0; r0 < rows; r0 += step) {
    const int64_t n = std::min(rows - r0, step);
    const int64_t blocks = (n * per_row + kThreads / kWave - 1) / (kThreads / kWave);
    const void* xr = static_cast<const char*>(x) + (size_t)(r0 * cols) * esize;
    if (dtype == 1)
      hipLaunchKernelGGL(quant_w4_kernel<uint16_t>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                         static_cast<const uint16_t*>(xr), n, cols, q + r0 * (cols / 2), scale + r0 * per_row);
    else
      hipLaunchKernelGGL(quant_w4_kernel<float>, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                         static_cast<const float*>(xr), n, cols, q + r0 * (cols / 2), scale + r0 * per_row);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t quant_blocks(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                        int8_t* q, float* scale, hipStream_t stream, bool fp8) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (fp8) {
    if (dtype == 1) return launch_quant<uint16_t, Fp8Codec>(x, rows, cols, br, bc, q, scale, stream);
    return launch_quant<float, Fp8Codec>(x, rows, cols, br, bc, q, scale, stream);
  }
  if (dtype == 1) return launch_quant<uint16_t, Int8Codec>(x, rows, cols, br, bc, q, scale, stream);
  return launch_quant<float, Int8Codec>(x, rows, cols, br, bc, q, scale, stream);
}

}  // namespace w8a8
