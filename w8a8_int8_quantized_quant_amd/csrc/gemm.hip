// gemm.hip -- grouped INT8 GEMMs of the MoE layer on gfx950 INT8 MFMA.
//
// First GEMM: gathered int8 token rows x w13[e] (gate rows [0,I), up rows
// [I,2I)), int32 accumulation (SGLang PR #3888: the fused MoE kernel with
// channel-wise int8 and an int32 accumulator), one dequantization per output
// ((float)acc * a_scale[token]) * w_scale[channel] (jiqizhixin article,
// "Quantization exploration", channel-wise: a single dequantization after the
// INT8 matmul), SiLU(gate) * up, requantization of each row.
// Second GEMM: the int8 intermediate x w2[e], dequantization, and the top-k
// weighted combine of each token's expert outputs (PR #8273 highlights:
// GEMM, activation, GEMM, gather).
// Block-wise (article: [128,128] weight blocks, per-token-group activation
// scales): int32 partial per 128-wide K-block, acc += ((float)part * a_s) * w_s
// in ascending K-block order, requantization per (row, 128-group).
//
// Tiling: one workgroup = 4 wavefronts computes a BM x BN tile of one expert;
// K advances 128 bytes per stage through a double-buffered LDS tile (A: the
// tile's token rows gathered through the sorted pair list; B: BN weight rows),
// each wavefront issuing v_mfma_i32_16x16x64_i8 on 16 x 16 sub-tiles.  In the
// first GEMM the B tile holds BN/2 gate rows and the matching BN/2 up rows, so
// every lane owns both operands of SiLU(gate) * up.  The grid covers the
// worst-case tile count; workgroups past the device-side tile count exit at once.
#include "common.hpp"
#include "kernels.hpp"

namespace w8a8 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 128;                // K bytes per stage (= one block-wise K-block)
constexpr int kLdsStride = kBK + 16;    // padded LDS row (bytes)

enum class BMap { Plain, Split };
enum class Epi { I32, W13Channel, W2Channel, W13Block, W2Block };

struct Params {
  const int8_t* a;
  int32_t gather;
  const int8_t* w;
  int64_t N, K;
  const int32_t* sorted;
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  int64_t P, k, block_m, n_tiles, I;
  const float* a_s;    // activation / intermediate scales
  const float* w_s;    // weight scales
  int32_t* out_i32;
  float* out_f32;      // hf (first GEMM, channel) or y (second GEMM)
  float* part_amax;    // [rows, n_tiles] per-tile row maxima (first GEMM, channel)
  int8_t* h_q;
  float* h_s;
};

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// B-tile row of fragment fn of wavefront column wn: plain tiles split BN evenly over the WN
// wavefronts; split tiles give each wavefront FN/2 gate fragments and the matching up fragments.
template <int BN, int WN, int FN, BMap MAP>
__device__ __forceinline__ int brow_of(int wn, int fn) {
  if (MAP == BMap::Plain) return wn * (BN / WN) + fn * 16;
  return (fn < FN / 2 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (fn % (FN / 2)) * 16;
}

template <int BM, int BN, int WM, int WN, BMap MAP, Epi EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(const Params p) {
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int FNH = FN / 2;
  constexpr int A_CH = (BM * 8 + kThreads - 1) / kThreads;
  constexpr int B_CH = BN * 8 / kThreads;
  constexpr bool kBlock = EPI == Epi::W13Block || EPI == Epi::W2Block;
  static_assert(WM * WN == kThreads / kWave, "4 wavefronts");
  static_assert(FM >= 1 && FN >= 1 && B_CH >= 1, "tile too small");
  static_assert(MAP == BMap::Plain || FN % 2 == 0, "split tiles need gate and up fragments");

  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kLdsStride];
  __shared__ int32_t sh_pid[BM];
  __shared__ float sh_red[WN][BM];

  const int64_t mt = blockIdx.x / p.n_tiles, nt = blockIdx.x % p.n_tiles;
  const int64_t row0 = mt * BM;
  if (row0 >= (int64_t)p.num_tiles[0] * p.block_m) return;
  const int64_t e = p.tile_expert[row0 / p.block_m];
  const int8_t* wexp = p.w + e * p.N * p.K;

  const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
  const int wm = wv / WN, wn = wv % WN;

  for (int i = tid; i < BM; i += kThreads) sh_pid[i] = p.sorted[row0 + i];

  // Global sources of this thread's 16-byte chunks (row-major chunks of 8 per 128-byte row).
  const int8_t* a_src[A_CH];
  bool a_ok[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int idx = tid + c * kThreads, row = idx / 8, part = idx % 8;
    a_ok[c] = false;
    a_src[c] = p.a;
    if (idx < BM * 8) {
      const int32_t pid = p.sorted[row0 + row];
      if (pid < p.P) {
        a_ok[c] = true;
        a_src[c] = (p.gather ? p.a + (int64_t)(pid / p.k) * p.K : p.a + (row0 + row) * p.K) + part * 16;
      }
    }
  }
  const int8_t* b_src[B_CH];
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int idx = tid + c * kThreads, j = idx / 8, part = idx % 8;
    int64_t wrow;
    if (MAP == BMap::Plain)
      wrow = nt * BN + j;
    else
      wrow = j < BN / 2 ? nt * (BN / 2) + j : p.I + nt * (BN / 2) + (j - BN / 2);
    b_src[c] = wexp + wrow * p.K + part * 16;
  }

  i32x4 ra[A_CH], rb[B_CH];  // native vectors: HIP's uint4 struct would be copied through scratch
// Global -> registers for the K-stage at byte offset k0, and registers -> LDS buffer `buf`.
#define W8A8_GLOAD(k0)                                                                                         \
  do {                                                                                                         \
    _Pragma("unroll") for (int c = 0; c < A_CH; ++c) ra[c] =                                                   \
        a_ok[c] ? *reinterpret_cast<const i32x4*>(a_src[c] + (k0)) : i32x4{0, 0, 0, 0};                       \
    _Pragma("unroll") for (int c = 0; c < B_CH; ++c) rb[c] = *reinterpret_cast<const i32x4*>(b_src[c] + (k0)); \
  } while (0)
#define W8A8_SSTORE(buf)                                                                                       \
  do {                                                                                                         \
    _Pragma("unroll") for (int c = 0; c < A_CH; ++c) {                                                         \
      const int idx = tid + c * kThreads;                                                                      \
      if (idx < BM * 8) *reinterpret_cast<i32x4*>(&lds[buf][(idx / 8) * kLdsStride + (idx % 8) * 16]) = ra[c]; \
    }                                                                                                          \
    _Pragma("unroll") for (int c = 0; c < B_CH; ++c) {                                                         \
      const int idx = tid + c * kThreads;                                                                      \
      *reinterpret_cast<i32x4*>(&lds[buf][(BM + idx / 8) * kLdsStride + (idx % 8) * 16]) = rb[c];              \
    }                                                                                                          \
  } while (0)

  i32x4 acc[FM][FN];
  float accf[kBlock ? FM : 1][kBlock ? FN : 1][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  if (kBlock) {
#pragma unroll
    for (int i = 0; i < (kBlock ? FM : 1); ++i)
#pragma unroll
      for (int j = 0; j < (kBlock ? FN : 1); ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[i][j][r] = 0.0f;
  }

  const int64_t KT = p.K / kBK;
  const int64_t nkb = p.K / 128;  // block-wise scale columns
  W8A8_GLOAD(0);
  W8A8_SSTORE(0);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < KT) W8A8_GLOAD((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 64; ++kk) {
      i32x4 af[FM], bf[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const i32x4*>(
            &lds[buf][(wm * (BM / WM) + fm * 16 + (l % 16)) * kLdsStride + kk * 64 + (l / 16) * 16]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bf[fn] = *reinterpret_cast<const i32x4*>(
            &lds[buf][(BM + brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16)) * kLdsStride + kk * 64 + (l / 16) * 16]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
    }
    if constexpr (kBlock) {
      // Dequantize this K-block's integer partials and fold them into the fp32 sums.
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
          const int32_t pid = sh_pid[trow];
          float as = 0.0f;
          if (pid < p.P)
            as = EPI == Epi::W13Block ? p.a_s[(int64_t)(pid / p.k) * nkb + kt] : p.a_s[(row0 + trow) * nkb + kt];
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int br = brow_of<BN, WN, FN, MAP>(wn, fn);
            int64_t wrow;
            if (MAP == BMap::Plain)
              wrow = nt * BN + br;
            else
              wrow = br < BN / 2 ? nt * (BN / 2) + br : p.I + nt * (BN / 2) + (br - BN / 2);
            const float ws = p.w_s[(e * (p.N / 128) + wrow / 128) * nkb + kt];
            accf[fm][fn][r] = accf[fm][fn][r] + (((float)acc[fm][fn][r] * as) * ws);
          }
        }
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = i32x4{0, 0, 0, 0};
    }
    if (kt + 1 < KT) W8A8_SSTORE(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  // Accumulator element r of fragment (fm, fn) sits at tile row
  // wm*(BM/WM) + fm*16 + (l/16)*4 + r and tile column brow_of<BN, WN, FN, MAP>(wn, fn) + l%16.
  if constexpr (EPI == Epi::I32) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
        if (sh_pid[trow] >= p.P) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          p.out_i32[(row0 + trow) * p.N + nt * BN + brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16)] = acc[fm][fn][r];
      }
  } else if constexpr (EPI == Epi::W2Channel || EPI == Epi::W2Block) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
        if (sh_pid[trow] >= p.P) continue;
        const int64_t grow = row0 + trow;
        const float hs = kBlock ? 0.0f : p.a_s[grow];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int64_t n = nt * BN + brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16);
          float y;
          if constexpr (kBlock)
            y = accf[fm][fn][r];
          else
            y = ((float)acc[fm][fn][r] * hs) * p.w_s[e * p.N + n];
          p.out_f32[grow * p.N + n] = y;
        }
      }
  } else {
    // First GEMM: SiLU(gate) * up, then the row maxima of |h|.
    const int64_t I = p.I;
    float hf[FM][FNH][4];
    float rmax[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
        const int32_t pid = sh_pid[trow];
        const bool valid = pid < p.P;
        const float as = (!kBlock && valid) ? p.a_s[pid / p.k] : 0.0f;
        rmax[fm][r] = 0.0f;
#pragma unroll
        for (int f = 0; f < FNH; ++f) {
          const int64_t n = nt * (BN / 2) + brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16);
          float g, u;
          if constexpr (kBlock) {
            g = accf[fm][f][r];
            u = accf[fm][f + FNH][r];
          } else {
            g = ((float)acc[fm][f][r] * as) * p.w_s[e * 2 * I + n];
            u = ((float)acc[fm][f + FNH][r] * as) * p.w_s[e * 2 * I + I + n];
          }
          const float h = silu_mul(g, u);
          hf[fm][f][r] = h;
          if (valid) rmax[fm][r] = fmaxf(rmax[fm][r], fabsf(h));
        }
      }
    // reduce over the 16 lanes that share a row, then over the WN wavefronts
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = rmax[fm][r];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        if ((l % 16) == 0) sh_red[wn][wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r] = m;
      }
    __syncthreads();
    if constexpr (EPI == Epi::W13Channel) {
      // write h (fp32) and this tile's row maxima; the requant pass finishes the row
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
          if (sh_pid[trow] >= p.P) continue;
#pragma unroll
          for (int f = 0; f < FNH; ++f)
            p.out_f32[(row0 + trow) * I + nt * (BN / 2) + brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16)] = hf[fm][f][r];
        }
      for (int i = tid; i < BM; i += kThreads) {
        if (sh_pid[i] >= p.P) continue;
        float m = sh_red[0][i];
#pragma unroll
        for (int w = 1; w < WN; ++w) m = fmaxf(m, sh_red[w][i]);
        p.part_amax[(row0 + i) * p.n_tiles + nt] = m;
      }
    } else {
      // block-wise: this tile's BN/2 = 128 gate columns are exactly one requant group
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r;
          if (sh_pid[trow] >= p.P) continue;
          float m = sh_red[0][trow];
#pragma unroll
          for (int w = 1; w < WN; ++w) m = fmaxf(m, sh_red[w][trow]);
          const float s = quant_scale(m);
          const int64_t grow = row0 + trow;
          if (wn == 0 && (l % 16) == 0) p.h_s[grow * (I / 128) + nt] = s;
#pragma unroll
          for (int f = 0; f < FNH; ++f)
            p.h_q[grow * I + nt * (BN / 2) + brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16)] = quant_value(hf[fm][f][r], s);
        }
    }
  }
}

#undef W8A8_GLOAD
#undef W8A8_SSTORE

// Channel-wise requantization of the first GEMM's rows: one wavefront per row.
__global__ __launch_bounds__(kThreads) void requant_rows_kernel(const float* __restrict__ hf,
                                                                const float* __restrict__ part_amax,
                                                                const int32_t* __restrict__ sorted,
                                                                const int32_t* __restrict__ num_tiles, int64_t block_m,
                                                                int64_t P, int64_t I, int64_t n_tiles,
                                                                int8_t* __restrict__ h_q, float* __restrict__ h_s) {
  const int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (r >= (int64_t)num_tiles[0] * block_m) return;
  if (sorted[r] >= P) return;
  const int l = lane_id();
  float m = 0.0f;
  for (int64_t i = l; i < n_tiles; i += kWave) m = fmaxf(m, part_amax[r * n_tiles + i]);
  const float s = quant_scale(wave_max(m));
  if (l == 0) h_s[r] = s;
  const float4* src = reinterpret_cast<const float4*>(hf + r * I);
  uint32_t* dst = reinterpret_cast<uint32_t*>(h_q + r * I);
  for (int64_t c = l; c < I / 4; c += kWave) {
    const float4 v = src[c];
    dst[c] = (uint32_t)(uint8_t)quant_value(v.x, s) | ((uint32_t)(uint8_t)quant_value(v.y, s) << 8) |
             ((uint32_t)(uint8_t)quant_value(v.z, s) << 16) | ((uint32_t)(uint8_t)quant_value(v.w, s) << 24);
  }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = v;
}

// pair_row[sorted[r]] = r for the real rows.
__global__ void pair_row_kernel(const int32_t* __restrict__ sorted, const int32_t* __restrict__ num_tiles,
                                int64_t block_m, int64_t P, int32_t* __restrict__ pair_row, int64_t max_rows) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= max_rows || r >= (int64_t)num_tiles[0] * block_m) return;
  const int32_t pid = sorted[r];
  if (pid >= 0 && pid < P) pair_row[pid] = (int32_t)r;
}

// out[t, n] = 0 + w[t,0] * y0 + w[t,1] * y1 + ... in slot order; 4 columns per thread.
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y,
                                                           const int32_t* __restrict__ pair_row,
                                                           const float* __restrict__ topk_w, int64_t T, int64_t k,
                                                           int64_t H, float* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t H4 = H / 4;
  if (q >= T * H4) return;
  const int64_t t = q / H4, c = q % H4;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t j = 0; j < k; ++j) {
    const int32_t r = pair_row[t * k + j];
    if (r < 0) continue;
    const float wj = topk_w[t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + (int64_t)r * H)[c];
    o.x = o.x + wj * v.x;
    o.y = o.y + wj * v.y;
    o.z = o.z + wj * v.z;
    o.w = o.w + wj * v.w;
  }
  reinterpret_cast<float4*>(out + t * H)[c] = o;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

template <int BM, int BN, int WM, int WN, BMap MAP, Epi EPI>
hipError_t launch(const Params& prm, int64_t max_rows, hipStream_t stream) {
  const int64_t mtiles = max_rows / BM;
  const int64_t grid = mtiles * prm.n_tiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, MAP, EPI>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     stream, prm);
  return hipGetLastError();
}

// Tile height of the kernel for a given align block_m (a divisor of block_m).
template <BMap MAP, Epi EPI, int BN>
hipError_t launch_bm(Params prm, int64_t max_rows, hipStream_t stream) {
  prm.n_tiles = MAP == BMap::Plain ? prm.N / BN : prm.I / (BN / 2);
  switch (prm.block_m) {
    case 16: return launch<16, BN, 1, 4, MAP, EPI>(prm, max_rows, stream);
    case 32: return launch<32, BN, 1, 4, MAP, EPI>(prm, max_rows, stream);
    case 64: return launch<64, BN, 2, 2, MAP, EPI>(prm, max_rows, stream);
    default: return launch<(EPI == Epi::W13Block ? 64 : 128), BN, 2, 2, MAP, EPI>(prm, max_rows, stream);
  }
}

constexpr int kBNChannel = 128;  // first GEMM: 64 gate + 64 up rows; second GEMM: 128 output columns
constexpr int kBNBlock13 = 256;  // block-wise first GEMM: 128 gate + 128 up rows (one requant group)

}  // namespace

size_t w13_ws_bytes(const GroupedShape& s, int32_t scale_mode) {
  if (scale_mode == 1) return 256;
  const int64_t n_tiles = s.I / (kBNChannel / 2);
  return round256(sizeof(float) * (size_t)(s.max_rows * s.I)) + round256(sizeof(float) * (size_t)(s.max_rows * n_tiles));
}

size_t w2_ws_bytes(const GroupedShape& s, int32_t scale_mode) {
  (void)scale_mode;
  return round256(sizeof(float) * (size_t)(s.max_rows * s.H)) + round256(sizeof(int32_t) * (size_t)(s.T * s.k));
}

hipError_t gemm_i32(const int8_t* a, int32_t gather, const int8_t* w, int64_t N, int64_t K, const int32_t* sorted,
                    const int32_t* tile_expert, const int32_t* num_tiles, int64_t P, int64_t k, int64_t block_m,
                    int64_t max_rows, int32_t* out, hipStream_t stream) {
  Params prm{};
  prm.a = a;
  prm.gather = gather;
  prm.w = w;
  prm.N = N;
  prm.K = K;
  prm.sorted = sorted;
  prm.tile_expert = tile_expert;
  prm.num_tiles = num_tiles;
  prm.P = P;
  prm.k = k;
  prm.block_m = block_m;
  prm.out_i32 = out;
  return launch_bm<BMap::Plain, Epi::I32, kBNChannel>(prm, max_rows, stream);
}

hipError_t w13_silu(const GroupedShape& s, int32_t scale_mode, const int8_t* a_q, const float* a_s,
                    const int8_t* w13, const float* w13_s, const int32_t* sorted, const int32_t* tile_expert,
                    const int32_t* num_tiles, int8_t* h_q, float* h_s, void* ws, hipStream_t stream) {
  Params prm{};
  prm.a = a_q;
  prm.gather = 1;
  prm.w = w13;
  prm.N = 2 * s.I;
  prm.K = s.H;
  prm.sorted = sorted;
  prm.tile_expert = tile_expert;
  prm.num_tiles = num_tiles;
  prm.P = s.T * s.k;
  prm.k = s.k;
  prm.block_m = s.block_m;
  prm.I = s.I;
  prm.a_s = a_s;
  prm.w_s = w13_s;
  prm.h_q = h_q;
  prm.h_s = h_s;
  if (scale_mode == 1) return launch_bm<BMap::Split, Epi::W13Block, kBNBlock13>(prm, s.max_rows, stream);
  float* hf = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + round256(sizeof(float) * (size_t)(s.max_rows * s.I)));
  prm.out_f32 = hf;
  prm.part_amax = part;
  hipError_t err = launch_bm<BMap::Split, Epi::W13Channel, kBNChannel>(prm, s.max_rows, stream);
  if (err != hipSuccess) return err;
  const int64_t n_tiles = s.I / (kBNChannel / 2);
  const int64_t blocks = (s.max_rows + kThreads / kWave - 1) / (kThreads / kWave);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(requant_rows_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, hf, part, sorted,
                     num_tiles, s.block_m, s.T * s.k, s.I, n_tiles, h_q, h_s);
  return hipGetLastError();
}

hipError_t w2_combine(const GroupedShape& s, int32_t scale_mode, const int8_t* h_q, const float* h_s,
                      const int8_t* w2, const float* w2_s, const int32_t* sorted, const int32_t* tile_expert,
                      const int32_t* num_tiles, const float* topk_w, float* out, void* ws, hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  const int64_t P = s.T * s.k;
  float* y = static_cast<float*>(ws);
  int32_t* pair_row =
      reinterpret_cast<int32_t*>(static_cast<char*>(ws) + round256(sizeof(float) * (size_t)(s.max_rows * s.H)));
  Params prm{};
  prm.a = h_q;
  prm.gather = 0;
  prm.w = w2;
  prm.N = s.H;
  prm.K = s.I;
  prm.sorted = sorted;
  prm.tile_expert = tile_expert;
  prm.num_tiles = num_tiles;
  prm.P = P;
  prm.k = s.k;
  prm.block_m = s.block_m;
  prm.a_s = h_s;
  prm.w_s = w2_s;
  prm.out_f32 = y;
  hipError_t err = scale_mode == 1 ? launch_bm<BMap::Plain, Epi::W2Block, kBNChannel>(prm, s.max_rows, stream)
                                   : launch_bm<BMap::Plain, Epi::W2Channel, kBNChannel>(prm, s.max_rows, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((uint32_t)((P + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     pair_row, P, -1);
  if (s.max_rows > 0)
    hipLaunchKernelGGL(pair_row_kernel, dim3((uint32_t)((s.max_rows + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, sorted, num_tiles, s.block_m, P, pair_row, s.max_rows);
  const int64_t q = s.T * (s.H / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((q + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream, y,
                     pair_row, topk_w, s.T, s.k, s.H, out);
  return hipGetLastError();
}

}  // namespace w8a8
