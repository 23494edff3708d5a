// probe.hip -- measured peaks of the chip the layer runs on, for the benchmark's report: a
// streaming HBM read, a streaming HBM copy and an INT8 MFMA loop; and one FP8 MFMA on given
// operands, whose sums the tests compare with exact ones.  Not part of the layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w8a8probe.h"

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Every thread reads kUnroll 16-byte chunks per round, non-temporal (the weights of the layer are
// streamed the same way); the XOR of everything read decides a store that never happens in
// practice, so the loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void read_kernel(const i32x4* __restrict__ p, int64_t n,
                                                        int32_t* __restrict__ sink) {
  i32x4 acc = {0, 0, 0, 0};
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n; i += stride) {
    i32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kThreads;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x7f3a5c11) sink[0] = 1;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const i32x4* __restrict__ src, i32x4* __restrict__ dst,
                                                        int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n; i += stride) {
    i32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kThreads;
      v[u] = j < n ? __builtin_nontemporal_load(src + j) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kThreads;
      if (j < n) __builtin_nontemporal_store(v[u], dst + j);
    }
  }
}

// Each wavefront keeps independent accumulators busy with one INT8 MFMA form on operands of
// pseudo-random bytes (a multiply-xorshift of the lane id: all-equal operands would draw less power
// and clock higher than real data): 8 chains of v_mfma_i32_16x16x64_i8 (FR = 16) or 4 of
// v_mfma_i32_32x32x32_i8 (FR = 32), the same multiply-adds per round.
constexpr int kChains = 8;  // 16 x 16 x 64 chains per round (4 of 32 x 32 x 32)
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
template <int FR>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int64_t iters, int32_t* __restrict__ sink) {
  const uint32_t l = threadIdx.x + blockIdx.x * kThreads;
  auto mix = [](uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    return x ^ (x >> 16);
  };
  i32x4 a = {(int32_t)mix(l), (int32_t)mix(l + 1u), (int32_t)mix(l + 2u), (int32_t)mix(l + 3u)};
  i32x4 b = {(int32_t)mix(~l), (int32_t)mix(~l + 7u), (int32_t)mix(~l + 9u), (int32_t)mix(~l + 11u)};
  int32_t s = 0;
  if constexpr (FR == 16) {
    i32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = i32x4{0, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) s ^= acc[c][0] ^ acc[c][1] ^ acc[c][2] ^ acc[c][3];
  } else {
    i32x16 acc[kChains / 2];
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c) acc[c] = i32x16{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains / 2; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains / 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s ^= acc[c][r];
  }
  if (s == 0x13572468) sink[0] = s;
}

// One v_mfma_scale_f32_16x16x128_f8f6f4 per wavefront (scales 1.0, C = 0) on one [16, 128] A block
// and one [16, 128] B block of E4M3 codes, K-contiguous rows, with the operand layout of the
// layer's FP8 GEMM: lane (g, r) holds bytes [32 g, 32 g + 32) of row r of each operand.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(64) void mfma_f8_block_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                           float* __restrict__ c) {
  const int l = threadIdx.x, g = l >> 4, r = l & 15;
  const int64_t blk = blockIdx.x;
  const i32x8 av = *reinterpret_cast<const i32x8*>(a + blk * 2048 + r * 128 + g * 32);
  const i32x8 bv = *reinterpret_cast<const i32x8*>(b + blk * 2048 + r * 128 + g * 32);
  const f32x4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                                      0, 127, 0, 127);
#pragma unroll
  for (int i = 0; i < 4; ++i) c[blk * 256 + (g * 4 + i) * 16 + r] = acc[i];
}

}  // namespace

extern "C" {

// 8192 workgroups: the fastest of the read patterns tried on this chip (grid-stride or per-workgroup
// chunks, 4 / 8 / 16 loads in flight per thread, plain or non-temporal, 1024 to 16384 workgroups)
int32_t w8a8_probe_read(const void* buf, int64_t bytes, int32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(8192), dim3(kThreads), 0, stream, static_cast<const i32x4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int32_t w8a8_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes < 16 || bytes % 16) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(kThreads), 0, stream, static_cast<const i32x4*>(src),
                     static_cast<i32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int32_t w8a8_probe_mfma_i8(int64_t iters, int32_t workgroups, int32_t shape, int32_t* sink, hipStream_t stream) {
  if (!sink || iters < 1 || workgroups < 1 || (shape != 16 && shape != 32)) return 1;
  if (shape == 16)
    hipLaunchKernelGGL(mfma_kernel<16>, dim3((uint32_t)workgroups), dim3(kThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_kernel<32>, dim3((uint32_t)workgroups), dim3(kThreads), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int32_t w8a8_probe_mfma_f8_block(const uint8_t* a, const uint8_t* b, float* c, int32_t blocks, hipStream_t stream) {
  if (!a || !b || !c || blocks < 1) return 1;
  hipLaunchKernelGGL(mfma_f8_block_kernel, dim3((uint32_t)blocks), dim3(64), 0, stream, a, b, c);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int64_t w8a8_probe_mfma_i8_ops(int64_t iters, int32_t workgroups) {
  // per wavefront and iteration: kChains MFMAs of 16 x 16 x 64 multiply-adds (either shape)
  return (int64_t)workgroups * (kThreads / 64) * iters * kChains * 2 * 16 * 16 * 64;
}

}  // extern "C"
