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
// Three tile engines.  All issue v_mfma_i32_16x16x64_i8 on 16 x 16 sub-tiles;
// accumulator element r of a fragment sits at fragment row (lane/16)*4 + r and
// fragment column lane%16.  In the first GEMM a B tile holds BN/2 gate rows and
// the matching BN/2 up rows, so the lane that owns gate column n also owns up
// column n and forms SiLU(gate) * up in registers.
//  - Staged engine (few rows per expert, weight streaming): tiles of block_m
//    rows from the align step, K advances 128 bytes per stage through a double
//    buffered LDS tile loaded via registers.  Many small workgroups keep many
//    weight bytes in flight.
//  - DMA engine (hundreds of rows per expert, MFMA-bound): 320 x 256 tiles of
//    real rows only (a device-built work list, so align padding costs no MFMA
//    work), two LDS stages of 128-byte K-slices (whole L2 lines) filled by
//    global_load_lds_dwordx4, XOR-swizzled 16-byte chunks so fragment reads are
//    conflict-free, and an XCD-aware order in which each XCD walks a contiguous
//    stretch of (tile, N-tile) work so the A rows and the expert's weights are
//    reused from its own L2.
//  - Ring engine (tens to a couple of hundred rows per expert, and every
//    block-wise batch past decode): the DMA engine's work list and order with
//    128 x 256 tiles and a 3-stage LDS ring whose K loop is unrolled for the
//    layer's K sizes, so two stages are always in flight.
// Grids cover the worst case; workgroups past the device-side tile count exit
// at once (no host read, graph-capturable).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace w8a8 {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));  // native vector: the non-temporal builtins take it
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));  // 32 FP8 codes: one lane's MFMA operand

constexpr int kThreads = 256;

enum class BMap { Plain, Split };
// W13Fp8 / W2Fp8: the block-wise epilogues for FP8 (E4M3) operands, whose per-K-block partial
// sums come from the FP8 MFMA in fp32; the first GEMM requantizes to E4M3.  W13W4 / W2W4: the
// same with packed int4 weights (widened to E4M3 codes on the way to the MFMA) and one weight
// scale per (output row, K-block).
enum class Epi { I32, W13Channel, W2Channel, W13Block, W2Block, W13Fp8, W2Fp8, W13W4, W2W4 };

template <Epi EPI>
constexpr bool is_w4() {
  return EPI == Epi::W13W4 || EPI == Epi::W2W4;
}
template <Epi EPI>
constexpr bool is_fp8() {
  return EPI == Epi::W13Fp8 || EPI == Epi::W2Fp8 || is_w4<EPI>();
}
template <Epi EPI>
constexpr bool is_block() {
  return EPI == Epi::W13Block || EPI == Epi::W2Block || is_fp8<EPI>();
}

struct Params {
  const int8_t* a;
  int32_t gather;
  const int8_t* w;
  int64_t N, K;
  const int32_t* sorted;  // null: rows in their own order (the dense linear), row r = pair r
  const int32_t* tile_expert;
  const int32_t* num_tiles;
  int64_t P, k, block_m, n_tiles, I;
  const float* a_s;    // activation / intermediate scales
  const float* w_s;    // weight scales
  int32_t* out_i32;
  float* out_f32;      // fp32 h (first GEMM, channel) or y (second GEMM)
  float* part_amax;    // [rows, n_tiles] per-tile row maxima of |h| (first GEMM, channel)
  int8_t* h_q;
  float* h_s;
  int64_t ksplit;  // DMA engine, Epi::I32: K slices per tile (1 = none); slice s writes out_i32 + s*P*N
  int32_t* pair_row;  // second GEMM: the workgroups of N-tile 0 store pair_row[pair] = sorted row
  int64_t block0;     // staged engine: the (row tile, N-tile) item of this launch's workgroup 0
};

// pair_row[pid] = row for a real row of the tile (only the N-tile 0 workgroups call it, so each
// real row is written once).
__device__ __forceinline__ void note_pair_row(const Params& p, int32_t pid, int64_t row) {
  if (pid >= 0 && pid < p.P) p.pair_row[pid] = (int32_t)row;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// B-tile row of fragment fn of wavefront column wn: plain tiles split BN evenly over the WN
// wavefronts; split tiles give each wavefront FN/2 gate fragments and the matching up fragments.
template <int BN, int WN, int FN, BMap MAP>
__device__ __forceinline__ int brow_of(int wn, int fn) {
  if (MAP == BMap::Plain) return wn * (BN / WN) + fn * 16;
  return (fn < FN / 2 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (fn % (FN / 2)) * 16;
}

// Weight row of B-tile row br in N-tile nt.
template <int BN, BMap MAP>
__device__ __forceinline__ int64_t wrow_of(int64_t nt, int br, int64_t I) {
  if (MAP == BMap::Plain) return nt * BN + br;
  return br < BN / 2 ? nt * (BN / 2) + br : I + nt * (BN / 2) + (br - BN / 2);
}

// Tile row block (16 rows) of fragment row fm of wavefront row wm: the FM fragment rows of a
// wavefront row one after another (contiguous bands), or interleaved, fragment fm of wavefront row
// wm at block fm * WM + wm, so that a tile holding fewer real rows than BM still gives every
// wavefront row a share of them.
template <int WM, int FM, bool ILV>
__device__ __forceinline__ int rblk(int wm, int fm) {
  return ILV ? fm * WM + wm : wm * FM + fm;
}
// Fragment rows (bit fm) of wavefront row wm that hold real rows of a tile with nrows of them.
template <int WM, int FM, bool ILV>
__device__ __forceinline__ uint32_t real_frags(int wm, int nrows) {
  uint32_t m = 0;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
    if (rblk<WM, FM, ILV>(wm, fm) * 16 < nrows) m |= 1u << fm;
  return m;
}

// Block-wise scales of K-block kb for this lane's accumulators: the activation (or intermediate)
// scale of each of its rows (sh_arow: the row's index into the scale matrix, -1 past the real
// rows) and the weight scale of each of its fragments' 128-row weight block.
template <int BM, int BN, int WM, int WN, int FM, int FN, BMap MAP>
__device__ __forceinline__ void block_scales(const Params& p, const int32_t* sh_arow, int64_t nt, int64_t e, int wm,
                                             int wn, int l, int64_t kb, int64_t nkb, float (&as)[FM][4],
                                             float (&ws)[FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t ar = sh_arow[wm * (BM / WM) + fm * 16 + (l / 16) * 4 + r];
      as[fm][r] = ar >= 0 ? p.a_s[(int64_t)ar * nkb + kb] : 0.0f;
    }
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int64_t wrow = wrow_of<BN, MAP>(nt, brow_of<BN, WN, FN, MAP>(wn, fn), p.I);
    ws[fn] = p.w_s[(e * (p.N / 128) + wrow / 128) * nkb + kb];
  }
}

// Block-wise: fold the int32 partials of one K-block into the fp32 sums, in the written order
// acc_f = acc_f + (((float)part * a_s) * w_s), and clear them.
// Fragment rows outside `fmask` (no real rows) hold zero partials and are skipped.
template <int FM, int FN, typename AccT>
__device__ __forceinline__ void block_flush(AccT (&acc)[FM][FN], float (&accf)[FM][FN][4], const float (&as)[FM][4],
                                            const float (&ws)[FN], uint32_t fmask = ~0u) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (!((fmask >> fm) & 1u)) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) accf[fm][fn][r] = accf[fm][fn][r] + (((float)acc[fm][fn][r] * as[fm][r]) * ws[fn]);
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = AccT{0, 0, 0, 0};
}

// The channel-wise epilogues scale each tile row by one activation scale: the token's (first GEMM,
// rows gathered from tokens) or the sorted row's own (second GEMM); 0 for rows that hold no pair.
// The kernels gather it into LDS (sh_as) while their first stage loads, so the epilogue reads it
// there: a global load per row inside the epilogue left the wavefronts waiting on one round trip
// after another (with the prologue's pair ids also read from LDS, the gate+up stage at 8192 tokens
// went from 2.39 to 2.24 ms and the down stage from 1.73 to 1.69 ms).
template <Epi EPI>
constexpr bool has_row_scale() {
  return EPI == Epi::W13Channel || EPI == Epi::W2Channel;
}
template <Epi EPI>
__device__ __forceinline__ float row_scale(const Params& p, int32_t pid, int64_t row) {
  if constexpr (EPI == Epi::W13Channel) return pid < p.P ? p.a_s[pid / p.k] : 0.0f;
  else if constexpr (EPI == Epi::W2Channel) return pid < p.P ? p.a_s[row] : 0.0f;
  else return 0.0f;
}

// Epilogues.  Rows whose sh_pid is the sentinel (>= P) are skipped; sh_as holds the channel-wise
// row scales (row_scale).
template <int BM, int BN, int WM, int WN, int FM, int FN, BMap MAP, Epi EPI, bool ILV = false, typename AccT>
__device__ __forceinline__ void epilogue(const Params& p, const AccT (&acc)[FM][FN], const float (&accf)[FM][FN][4],
                                         const int32_t* sh_pid, const float* sh_as, float (*sh_red)[BM], int64_t row0,
                                         int64_t nt, int64_t e, int wm, int wn, int l, int tid) {
  constexpr int FNH = FN / 2;
  constexpr bool kBlock = is_block<EPI>();
  if constexpr (EPI == Epi::I32) {
    // raw accumulators at their weight rows (gate and up halves of a split tile go to their own columns)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        if (sh_pid[trow] >= p.P) continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          p.out_i32[(row0 + trow) * p.N + wrow_of<BN, MAP>(nt, brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16), p.I)] =
              acc[fm][fn][r];
      }
  } else if constexpr (EPI == Epi::W2Channel || EPI == Epi::W2Block || EPI == Epi::W2Fp8 || EPI == Epi::W2W4) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        if (sh_pid[trow] >= p.P) continue;
        const int64_t grow = row0 + trow;
        const float hs = kBlock ? 0.0f : sh_as[trow];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int64_t n = nt * BN + brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16);
          float y;
          if constexpr (kBlock)
            y = accf[fm][fn][r];
          else
            y = ((float)acc[fm][fn][r] * hs) * p.w_s[e * p.N + n];
          if constexpr (kBlock)  // y of a mid-size batch (470 MB at 2048 tokens): read once, by the combine
            __builtin_nontemporal_store(y, p.out_f32 + grow * p.N + n);
          else
            p.out_f32[grow * p.N + n] = y;
        }
      }
  } else if constexpr (EPI == Epi::W13Channel) {
    // First GEMM, channel-wise: SiLU(gate) * up stored as fp32 h, one fragment row at a time
    // (few live registers), plus this tile's per-row maxima of |h|; the requant pass finishes
    // each row once all its N-tiles are in.
    const int64_t I = p.I;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      float rmax[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        const bool valid = sh_pid[trow] < p.P;
        const float as = sh_as[trow];
        rmax[r] = 0.0f;
#pragma unroll
        for (int f = 0; f < FNH; ++f) {
          const int64_t n = nt * (BN / 2) + brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16);
          const float g = ((float)acc[fm][f][r] * as) * p.w_s[e * 2 * I + n];
          const float u = ((float)acc[fm][f + FNH][r] * as) * p.w_s[e * 2 * I + I + n];
          const float h = silu_mul(g, u);
          if (valid) {
            p.out_f32[(row0 + trow) * I + n] = h;
            rmax[r] = fmaxf(rmax[r], fabsf(h));
          }
        }
      }
      // reduce over the 16 lanes that share a row
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = row16_max(rmax[r]);  // over the 16 lanes that share a row
        if ((l % 16) == 0) sh_red[wn][rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r] = m;
      }
    }
    __syncthreads();
    for (int i = tid; i < BM; i += WM * WN * kWave) {
      if (sh_pid[i] >= p.P) continue;
      float m = sh_red[0][i];
#pragma unroll
      for (int w = 1; w < WN; ++w) m = fmaxf(m, sh_red[w][i]);
      p.part_amax[(row0 + i) * p.n_tiles + nt] = m;
    }
  } else {
    // First GEMM, block-wise: SiLU(gate) * up, then requantization in the tile, whose BN/2 = 128
    // gate columns are exactly one 128-wide requant group (INT8, or E4M3 for FP8 operands).
    const int64_t I = p.I;
    float hf[FM][FNH][4];
    float rmax[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        const bool valid = sh_pid[trow] < p.P;
        rmax[fm][r] = 0.0f;
#pragma unroll
        for (int f = 0; f < FNH; ++f) {
          const float h = silu_mul(accf[fm][f][r], accf[fm][f + FNH][r]);
          hf[fm][f][r] = h;
          if (valid) rmax[fm][r] = fmaxf(rmax[fm][r], fabsf(h));
        }
      }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = row16_max(rmax[fm][r]);  // over the 16 lanes that share a row
        if ((l % 16) == 0) sh_red[wn][rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r] = m;
      }
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        if (sh_pid[trow] >= p.P) continue;
        float m = sh_red[0][trow];
#pragma unroll
        for (int w = 1; w < WN; ++w) m = fmaxf(m, sh_red[w][trow]);
        const float s = is_fp8<EPI>() ? fp8_scale(m) : quant_scale(m);
        const int64_t grow = row0 + trow;
        if (wn == 0 && (l % 16) == 0) p.h_s[grow * (I / 128) + nt] = s;
#pragma unroll
        for (int f = 0; f < FNH; ++f)
          p.h_q[grow * I + nt * (BN / 2) + brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16)] =
              is_fp8<EPI>() ? (int8_t)fp8_value(hf[fm][f][r], s) : quant_value(hf[fm][f][r], s);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Staged engine: tiles of BM rows (BM divides block_m), BK = 128 bytes per stage, register-staged
// global loads into a double-buffered, padded LDS tile.

constexpr int kBK = 128;
constexpr int kLdsStride = kBK + 16;  // padded LDS row (bytes)

template <int BM, int BN, int WM, int WN, BMap MAP, Epi EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(const Params p) {
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int A_CH = (BM * 8 + kThreads - 1) / kThreads;
  constexpr int B_CH = BN * 8 / kThreads;
  constexpr bool kBlock = is_block<EPI>();
  static_assert(WM * WN == kThreads / kWave, "4 wavefronts");
  static_assert(FM >= 1 && FN >= 1 && B_CH >= 1, "tile too small");
  static_assert(MAP == BMap::Plain || FN % 2 == 0, "split tiles need gate and up fragments");

  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kLdsStride];
  __shared__ int32_t sh_pid[BM];
  __shared__ int32_t sh_arow[kBlock ? BM : 1];  // block-wise: row index into the activation scales
  __shared__ float sh_as[has_row_scale<EPI>() ? BM : 1];
  __shared__ float sh_red[WN][BM];

  const int64_t v = p.block0 + blockIdx.x;
  const int64_t mt = v / p.n_tiles, nt = v % p.n_tiles;
  const int64_t row0 = mt * BM;
  if (row0 >= (int64_t)p.num_tiles[0] * p.block_m) return;
  const int64_t e = p.tile_expert[row0 / p.block_m];
  const int8_t* wexp = p.w + e * p.N * p.K;

  const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
  const int wm = wv / WN, wn = wv % WN;

  for (int i = tid; i < BM; i += kThreads) {
    const int32_t pid = p.sorted[row0 + i];
    sh_pid[i] = pid;
    if (p.pair_row && nt == 0) note_pair_row(p, pid, row0 + i);
    if constexpr (kBlock) sh_arow[i] = pid < p.P ? (p.gather ? (int32_t)(pid / p.k) : (int32_t)(row0 + i)) : -1;
    if constexpr (has_row_scale<EPI>()) sh_as[i] = row_scale<EPI>(p, pid, row0 + i);
  }

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
    b_src[c] = wexp + wrow_of<BN, MAP>(nt, j, p.I) * p.K + part * 16;
  }

  i32x4 ra[A_CH], rb[B_CH];  // native vectors: HIP's uint4 struct would be copied through scratch
// Global -> registers for the K-stage at byte offset k0, and registers -> LDS buffer `buf`.  The
// weights stream through with non-temporal loads (each weight tile is read by few workgroups; the
// streaming hint measured about 15% more read bandwidth than plain loads on a pure read stream).
#define W8A8_GLOAD(k0)                                                                                         \
  do {                                                                                                         \
    _Pragma("unroll") for (int c = 0; c < A_CH; ++c) ra[c] =                                                   \
        a_ok[c] ? *reinterpret_cast<const i32x4*>(a_src[c] + (k0)) : i32x4{0, 0, 0, 0};                       \
    _Pragma("unroll") for (int c = 0; c < B_CH; ++c) rb[c] =                                                   \
        __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(b_src[c] + (k0)));                           \
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
  float accf[FM][FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][j][r] = 0.0f;
    }

  const int64_t KT = p.K / kBK;
  const int64_t nkb = p.K / 128;  // block-wise scale columns
  W8A8_GLOAD(0);
  W8A8_SSTORE(0);
  __syncthreads();
  // Block-wise: the scales of K-block kt + 1 are loaded during step kt, a full step ahead of use,
  // into the other of two register sets (the loop is unrolled by two, so no copy waits on them).
  float sa0[kBlock ? FM : 1][4], sw0[kBlock ? FN : 1], sa1[kBlock ? FM : 1][4], sw1[kBlock ? FN : 1];
  if constexpr (kBlock) block_scales<BM, BN, WM, WN, FM, FN, MAP>(p, sh_arow, nt, e, wm, wn, l, 0, nkb, sa0, sw0);
  auto step = [&](int64_t kt, float (&as_c)[kBlock ? FM : 1][4], float (&ws_c)[kBlock ? FN : 1],
                  float (&as_n)[kBlock ? FM : 1][4], float (&ws_n)[kBlock ? FN : 1]) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < KT) W8A8_GLOAD((kt + 1) * kBK);
    if constexpr (kBlock) {
      if (kt + 1 < KT) block_scales<BM, BN, WM, WN, FM, FN, MAP>(p, sh_arow, nt, e, wm, wn, l, kt + 1, nkb, as_n, ws_n);
    }
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
    if constexpr (kBlock) block_flush<FM, FN>(acc, accf, as_c, ws_c);
    if (kt + 1 < KT) W8A8_SSTORE(buf ^ 1);
    __syncthreads();
  };
  if constexpr (kBlock) {
    for (int64_t kt = 0; kt < KT; kt += 2) {
      step(kt, sa0, sw0, sa1, sw1);
      if (kt + 1 < KT) step(kt + 1, sa1, sw1, sa0, sw0);
    }
  } else {
    for (int64_t kt = 0; kt < KT; ++kt) step(kt, sa0, sw0, sa1, sw1);
  }
#undef W8A8_GLOAD
#undef W8A8_SSTORE
  epilogue<BM, BN, WM, WN, FM, FN, MAP, EPI>(p, acc, accf, sh_pid, sh_as, sh_red, row0, nt, e, wm, wn, l, tid);
}

// ---------------------------------------------------------------------------------------------
// DMA engine.

constexpr int kWorkFields = 5;  // ints per work-list tile
constexpr int64_t kSuperRows = 4;  // row tiles per super-row of the DMA engine's work order
// The ring engine's super-rows hold up to 16 row tiles: with skewed routing a hot expert has ~13
// 128-row tiles, and one super-row streams each of its weight tiles once instead of once per 4 row
// tiles (its activation rows are re-read per N-tile instead).  Experts with one row tile, the
// common case at mid-size batches, are unaffected.
constexpr int64_t kRingSuperRows = 16;
constexpr int kDmaBK = 128;  // K bytes per LDS stage: two MFMA K-steps, whole 128-byte L2 lines

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 encoding) waiting until at most n vector-memory operations of this
// wavefront are outstanding, without waiting on LDS or export counters.
template <int n>
constexpr int vmcnt_imm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}
constexpr int kLgkm0Imm = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0) only

// vmcnt(n) for an n that is a constant once the K loop is unrolled (the switch folds away).
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
#define W8A8_VMW(i) \
  case i: __builtin_amdgcn_s_waitcnt(vmcnt_imm<i>()); break;
    W8A8_VMW(0) W8A8_VMW(1) W8A8_VMW(2) W8A8_VMW(3) W8A8_VMW(4) W8A8_VMW(5) W8A8_VMW(6) W8A8_VMW(7)
    W8A8_VMW(8) W8A8_VMW(9) W8A8_VMW(10) W8A8_VMW(11) W8A8_VMW(12) W8A8_VMW(13) W8A8_VMW(14) W8A8_VMW(15)
    W8A8_VMW(16) W8A8_VMW(17) W8A8_VMW(18) W8A8_VMW(19) W8A8_VMW(20) W8A8_VMW(21) W8A8_VMW(22) W8A8_VMW(23)
    W8A8_VMW(24) W8A8_VMW(25) W8A8_VMW(26) W8A8_VMW(27) W8A8_VMW(28) W8A8_VMW(29) W8A8_VMW(30) W8A8_VMW(31)
#undef W8A8_VMW
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>()); break;
  }
}

// Workgroup barrier without a memory fence: LDS data written by the DMA is published by the
// explicit vmcnt wait that precedes it, and a fence would drain every stage still in flight.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte-per-lane DMA (global_load_lds_dwordx4): lane i's 16 bytes land at lds + 16 i.
// (A plain device function: calling the builtin directly inside the kernel template kept the
// host compiler from emitting the kernel's launch stub.)
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}
// The same with the non-temporal (streaming) cache policy, for the weights: each weight tile is
// read by the few row tiles of its expert, side by side.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16_nt(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, kCachePolicyNT);
}

// 16-byte chunk swizzle of a 128-byte LDS row: chunk c of row r sits in slot c ^ ((r >> 1) & 7).
// Sixteen consecutive rows reading the same chunk then hit sixteen different 16-byte bank groups
// of a 256-byte window.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// The DMA engine's K loop.  Each stage holds 128 bytes of K (two MFMA K-steps) for BM A rows and
// BN B rows.  A wavefront works through its stage in groups (K-step kk, fragment row fm) of FN
// MFMAs and issues the next stage's DMA instructions between the first SPREAD groups (0: between
// all of them, evenly), A before B.  Scheduling barriers keep the compiler from regrouping them.
template <int BM, int BN, int WM, int WN, int A_LD, int LD, BMap MAP, bool ILV = false, int SPREAD = 0>
__device__ __forceinline__ void dma_stage(const int8_t* stage, int8_t* next, const int8_t* a_base,
                                          const int8_t* b_base, const uint32_t (&off)[LD], int a_dst, int b_dst,
                                          uint32_t next_off, bool prefetch, i32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                          int wm, int wn, int g, int fr, uint32_t fmask) {
  constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  constexpr int GROUPS = (kDmaBK / 64) * FM;
  constexpr int SLOTS = SPREAD > 0 ? SPREAD : GROUPS;
  static_assert(GROUPS >= LD && SLOTS <= GROUPS, "DMA slots");  // DMA c goes out before group c SLOTS / LD
#pragma unroll
  for (int kk = 0; kk < kDmaBK / 64; ++kk) {
    const int lane = fr * kDmaBK + (((kk * 4 + g) ^ swz(fr)) << 4);
    i32x4 af[FM], bf[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      af[fm] = *reinterpret_cast<const i32x4*>(stage + lane + rblk<WM, FM, ILV>(wm, fm) * 16 * kDmaBK);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      bf[fn] = *reinterpret_cast<const i32x4*>(stage + BM * kDmaBK + lane + brow_of<BN, WN, FN, MAP>(wn, fn) * kDmaBK);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int grp = kk * FM + fm;
#pragma unroll
      for (int c = 0; c < LD; ++c)
        if ((c * SLOTS) / LD == grp && prefetch) {
          if (c < A_LD)
            dma16(a_base + (off[c] + next_off), next + a_dst + c * 1024);
          else
            dma16_nt(b_base + (off[c] + next_off), next + b_dst + (c - A_LD) * 1024);
        }
      if ((fmask >> fm) & 1u) {  // fragment rows past the tile's real rows are never stored
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[fm], bf[fn], acc[fm][fn], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The same K loop step for FP8 (E4M3) operands: one v_mfma_scale_f32_16x16x128_f8f6f4 per
// fragment covers the stage's 128 K-bytes (the scale operands are E8M0 127, i.e. 1.0).  Lane
// (g, fr) takes the 16-byte chunks 2g and 2g+1 of row fr, and the same chunks of both operands, so
// A and B hold the same K-elements at the same register positions.  Groups are (fragment row,
// half of the fragment columns), two MFMAs each, with the next stage's DMA spread between them as
// in dma_stage.
template <int BM, int BN, int WM, int WN, int A_LD, int LD, BMap MAP, bool ILV = false>
__device__ __forceinline__ void dma_stage_f8(const int8_t* stage, int8_t* next, const int8_t* a_base,
                                             const int8_t* b_base, const uint32_t (&off)[LD], int a_dst, int b_dst,
                                             uint32_t next_off, bool prefetch, f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                             int wm, int wn, int g, int fr, uint32_t fmask) {
  constexpr int FM = BM / WM / 16, FN = BN / WN / 16, FNH = FN / 2;
  constexpr int GROUPS = 2 * FM;
  static_assert(FN % 2 == 0, "gate and up fragments");  // DMA c goes out before group (c * GROUPS) / LD
  constexpr int kScaleOne = 127;                         // E8M0 exponent of 1.0
  const int c0 = fr * kDmaBK + (((2 * g) ^ swz(fr)) << 4);
  const int c1 = fr * kDmaBK + (((2 * g + 1) ^ swz(fr)) << 4);
  auto ld32 = [&](const int8_t* rowbase) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(rowbase + c0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(rowbase + c1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  i32x8 bf[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) bf[fn] = ld32(stage + BM * kDmaBK + brow_of<BN, WN, FN, MAP>(wn, fn) * kDmaBK);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    i32x8 af;
    if ((fmask >> fm) & 1u) af = ld32(stage + rblk<WM, FM, ILV>(wm, fm) * 16 * kDmaBK);  // rows past the real ones: no read
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int grp = fm * 2 + h;
#pragma unroll
      for (int c = 0; c < LD; ++c)
        if ((c * GROUPS) / LD == grp && prefetch) {
          if (c < A_LD)
            dma16(a_base + (off[c] + next_off), next + a_dst + c * 1024);
          else
            dma16_nt(b_base + (off[c] + next_off), next + b_dst + (c - A_LD) * 1024);
        }
      if ((fmask >> fm) & 1u) {
#pragma unroll
        for (int f = 0; f < FNH; ++f)
          acc[fm][h * FNH + f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[h * FNH + f], acc[fm][h * FNH + f], 0, 0, 0, kScaleOne, 0, kScaleOne);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Packed int4 -> E4M3 codes.  One dword holds 8 consecutive K values: byte b carries value b in
// its low nibble and value 4 + b in its high nibble, each nibble sign (bit 3) and magnitude
// (bits 0-2).  The magnitudes 0..7 are exact E4M3 values: a byte permute looks their codes up,
// and the sign moves to bit 7.  Out: codes of values 0-3 (first) and 4-7 (second).
constexpr uint32_t kW4CodesLo = 0x44403800u;  // E4M3 codes of 0, 1, 2, 3
constexpr uint32_t kW4CodesHi = 0x4E4C4A48u;  // E4M3 codes of 4, 5, 6, 7
__device__ __forceinline__ uint32_t w4_codes4(uint32_t nib) {  // nibble per byte -> code per byte
  return __builtin_amdgcn_perm(kW4CodesHi, kW4CodesLo, nib & 0x07070707u) | ((nib & 0x08080808u) << 4);
}
__device__ __forceinline__ void w4_to_fp8(uint32_t x, int32_t& lo, int32_t& hi) {
  lo = (int32_t)w4_codes4(x & 0x0F0F0F0Fu);
  hi = (int32_t)w4_codes4((x >> 4) & 0x0F0F0F0Fu);
}

// The K loop step for FP8 activations against packed int4 weights: as dma_stage_f8, with B rows
// of 64 bytes (128 int4 values) whose 16-byte chunks are swizzled by (row / 4) mod 4; lane (g, fr)
// widens chunk g of B row fr (values 32 g .. 32 g + 31) into the 32 E4M3 codes of its operand.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
template <int BM, int BN, int WM, int WN, int A_LD, int LD, BMap MAP, bool ILV = false>
__device__ __forceinline__ void dma_stage_w4(const int8_t* stage, int8_t* next, const int8_t* a_base,
                                             const int8_t* b_base, const uint32_t (&off)[LD], int a_dst, int b_dst,
                                             uint32_t next_off, bool prefetch, f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                             int wm, int wn, int g, int fr, uint32_t fmask) {
  constexpr int FM = BM / WM / 16, FN = BN / WN / 16, FNH = FN / 2;
  constexpr int GROUPS = 2 * FM;
  constexpr int BROW = kDmaBK / 2;  // bytes of one B row in a stage
  static_assert(FN % 2 == 0, "gate and up fragments");  // DMA c goes out before group (c * GROUPS) / LD
  constexpr int kScaleOne = 127;
  const int c0 = fr * kDmaBK + (((2 * g) ^ swz(fr)) << 4);
  const int c1 = fr * kDmaBK + (((2 * g + 1) ^ swz(fr)) << 4);
  i32x8 bf[FN];
  if (fmask != 0u) {  // wavefronts whose rows are all past the tile's real rows widen nothing
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int j = brow_of<BN, WN, FN, MAP>(wn, fn) + fr;
      const i32x4 v = *reinterpret_cast<const i32x4*>(stage + BM * kDmaBK + j * BROW + ((g ^ swz4(j)) << 4));
      int32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) w4_to_fp8((uint32_t)v[d], o[2 * d], o[2 * d + 1]);
      bf[fn] = i32x8{o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
    }
  }
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    i32x8 af;
    if ((fmask >> fm) & 1u) {  // rows past the real ones: no read
      const int8_t* arow = stage + rblk<WM, FM, ILV>(wm, fm) * 16 * kDmaBK;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(arow + c0);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(arow + c1);
      af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int grp = fm * 2 + h;
#pragma unroll
      for (int c = 0; c < LD; ++c)
        if ((c * GROUPS) / LD == grp && prefetch) {
          if (c < A_LD)
            dma16(a_base + (off[c] + next_off), next + a_dst + c * 1024);
          else
            // int4 stages are half a 128-byte line of each weight row; the normal cache policy keeps
            // the line in L2 for the next step's half (2.59 -> 2.52 ms at T = 2048)
            dma16(b_base + (off[c] + next_off), next + b_dst + (c - A_LD) * 1024);
        }
      if ((fmask >> fm) & 1u) {
#pragma unroll
        for (int f = 0; f < FNH; ++f)
          acc[fm][h * FNH + f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[h * FNH + f], acc[fm][h * FNH + f], 0, 0, 0, kScaleOne, 0, kScaleOne);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Maximum over each half wavefront (32 lanes), held by the half's upper 16 lanes: the 16-lane row
// maximum, then row_bcast:15 brings lane 15 of rows 0 and 2 to rows 1 and 3.  VALU only: the xor
// shuffles it replaces went through the LDS crossbar, five dependent round trips per row.  The whole
// wavefront must be active.
__device__ __forceinline__ float half_wave_max(float v) {
  return dpp_max_step<0x142, 0xA>(row16_max(v));  // row_bcast:15 into rows 1 and 3
}

// Channel-wise epilogues of the DMA engine, staged through the (then idle) stage buffers: each
// pass turns the accumulators of a band of fragment rows into fp32 values in LDS (wavefront-half
// wm in buffer wm), then whole rows leave as contiguous float4 stores.  Second GEMM: y rows of BN
// columns.  First GEMM: SiLU(gate) * up rows of BN / 2 columns, plus the row maximum of |h| over
// them, which a half wavefront reduces while it stores the row.  The fp32 rows are stored with
// the non-temporal policy: in the layer they are read back once, by the requantization or the
// combine pass after the whole GEMM (at 8192 tokens 0.5 and 1.9 GB, more than the caches hold);
// the dense linear's rows are its output.
template <int BM, int BN, int WM, int WN, int STAGE_BYTES, BMap MAP, Epi EPI, bool ILV = false>
__device__ __forceinline__ void dma_epilogue(const Params& p, const i32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                             const int32_t* sh_pid, const float* sh_as, int8_t* buf0, int8_t* buf1,
                                             int64_t row0, int64_t nt, int64_t e, int wm, int wn, int wv, int l,
                                             int64_t i32_off) {
  constexpr int FM = BM / WM / 16, FN = BN / WN / 16, FNH = FN / 2;
  constexpr int NW = WM * WN;
  constexpr bool kW13 = EPI == Epi::W13Channel;
  static_assert(WM == 2 && (EPI == Epi::W2Channel || EPI == Epi::W13Channel || EPI == Epi::I32),
                "two LDS halves, channel-wise or raw int32");
  constexpr int COLS = kW13 ? BN / 2 : BN;  // fp32 columns per row
  constexpr int STRIDE = COLS * 4 + 16;     // padded LDS row: the 4 row groups of a store hit distinct banks
  constexpr int F = STAGE_BYTES / (16 * STRIDE) < FM ? STAGE_BYTES / (16 * STRIDE) : FM;  // fragment rows per pass
  static_assert(F >= 1, "an LDS half holds at least one fragment row of values");
  int8_t* half = wm == 0 ? buf0 : buf1;
  const int64_t I = p.I;
#pragma unroll
  for (int f0 = 0; f0 < FM; f0 += F) {
    // accumulators -> LDS
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm < f0 || fm >= f0 + F) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rblk<WM, FM, ILV>(wm, fm) * 16 + (l / 16) * 4 + r;
        float* dst = reinterpret_cast<float*>(half + ((fm - f0) * 16 + (l / 16) * 4 + r) * STRIDE);
        if constexpr (kW13) {
          const float as = sh_as[trow];
#pragma unroll
          for (int f = 0; f < FNH; ++f) {
            const int col = brow_of<BN, WN, FN, MAP>(wn, f) + (l % 16);
            const int64_t n = nt * (BN / 2) + col;
            const float g = ((float)acc[fm][f][r] * as) * p.w_s[e * 2 * I + n];
            const float u = ((float)acc[fm][f + FNH][r] * as) * p.w_s[e * 2 * I + I + n];
            dst[col] = silu_mul(g, u);
          }
        } else if constexpr (EPI == Epi::I32) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int col = brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16);
            reinterpret_cast<int32_t*>(dst)[col] = acc[fm][fn][r];
          }
        } else {
          const float hs = sh_as[trow];
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int col = brow_of<BN, WN, FN, MAP>(wn, fn) + (l % 16);
            dst[col] = ((float)acc[fm][fn][r] * hs) * p.w_s[e * p.N + nt * BN + col];
          }
        }
      }
    }
    __syncthreads();
    // LDS -> global, whole rows
    const int rows = 2 * F * 16;
    if constexpr (kW13) {
      // a half wavefront per row: 32 lanes x float4 = 128 columns
      const int hl = l % 32;
      for (int idx = wv * 2 + l / 32; idx < rows; idx += NW * 2) {
        const int hf = idx / (F * 16), lr = idx % (F * 16);
        const bool in = f0 * 16 + lr < FM * 16;  // the last pass may hold fewer fragment rows
        const int trow = rblk<WM, FM, ILV>(hf, f0 + (in ? lr : 0) / 16) * 16 + (in ? lr : 0) % 16;
        const int32_t pid = in ? sh_pid[trow] : (int32_t)p.P;
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (in) v = *reinterpret_cast<const float4*>((hf == 0 ? buf0 : buf1) + lr * STRIDE + hl * 16);
        const float m = half_wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        if (pid < p.P) {
          __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<f32x4*>(p.out_f32 + (row0 + trow) * I + nt * (BN / 2)) + hl);
          if (hl == 16) p.part_amax[(row0 + trow) * p.n_tiles + nt] = m;  // lanes 16..31 of a half hold its max
        }
      }
    } else {
      // a wavefront per row: 64 lanes x float4 = 256 columns
      for (int idx = wv; idx < rows; idx += NW) {
        const int hf = idx / (F * 16), lr = idx % (F * 16);
        if (f0 * 16 + lr >= FM * 16) continue;
        const int trow = rblk<WM, FM, ILV>(hf, f0 + lr / 16) * 16 + lr % 16;
        if (sh_pid[trow] >= p.P) continue;
#pragma unroll
        for (int c = l; c < COLS / 4; c += kWave) {
          const float4 v = *reinterpret_cast<const float4*>((hf == 0 ? buf0 : buf1) + lr * STRIDE + c * 16);
          if constexpr (EPI == Epi::I32)  // int32 bits; a split tile's 4 columns lie in one half (BN / 2 % 4 == 0)
            *reinterpret_cast<float4*>(p.out_i32 + i32_off + (row0 + trow) * p.N + wrow_of<BN, MAP>(nt, 4 * c, I)) = v;
          else
            __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w},
                                        reinterpret_cast<f32x4*>(p.out_f32 + (row0 + trow) * p.N + nt * BN) + c);
        }
      }
    }
    __syncthreads();
  }
}

// BM x BN tiles on WM x WN wavefronts (two per SIMD), two LDS stages: while the MFMAs read one,
// the DMA fills the other.  The K loop runs two steps per iteration, one per stage buffer, so every
// stage index is known at compile time and the compiler tells the buffer being read from the one
// being filled; every step ends with all its DMA landed, so nothing is in flight across the loop's
// back edge.  K is a multiple of 256 (an even number of 128-byte steps).
template <int BM, int BN, int WM, int WN, BMap MAP, Epi EPI>
__global__ __launch_bounds__(WM * WN * kWave, 1) void grouped_gemm_dma_kernel(const Params p,
                                                                             const int32_t* __restrict__ work) {
  constexpr int NT = WM * WN * kWave;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int CPR = kDmaBK / 16;    // 16-byte chunks per row and stage
  constexpr int A_LD = BM * CPR / NT;  // DMA instructions per thread per stage (A tile)
  constexpr int B_LD = BN * CPR / NT;  // (B tile)
  constexpr int LD = A_LD + B_LD;
  constexpr int STAGE = (BM + BN) * kDmaBK;
  static_assert(!is_block<EPI>(), "channel-wise epilogues only");
  static_assert(A_LD >= 1 && B_LD >= 1 && (BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile shape");
  static_assert(MAP == BMap::Plain || FN % 2 == 0, "split tiles need gate and up fragments");

  __shared__ __attribute__((aligned(1024))) int8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) int8_t st1[STAGE];
  __shared__ int32_t sh_pid[BM];
  __shared__ float sh_as[has_row_scale<EPI>() ? BM : 1];

  // Work order: expert-major, then (super-row, N-tile, row tile), so the row tiles that share a
  // weight tile run side by side and the weights come from HBM once.  XCD-aware: workgroups are
  // dispatched round-robin over the 8 XCDs; each XCD gets a contiguous stretch of that order.
  const int64_t ntl = work ? (int64_t)work[0] : (p.P + BM - 1) / BM;  // row tiles
  const int64_t total = ntl * p.n_tiles * p.ksplit;
  const int64_t per = (total + 7) / 8;
  const int64_t v = blockIdx.x;
  if (v >= 8 * per) return;
  const int64_t item = (v % 8) * per + v / 8;
  if (item >= total) return;
  const int64_t ks = item % p.ksplit, logical = item / p.ksplit;  // K slice, then the (tile, N-tile) item
  const int64_t kslice = p.K / p.ksplit;                           // bytes of K per slice
  int64_t first = 0, count = ntl;  // the expert's first tile and its tile count
  if (work) {
    const int32_t* any = work + 1 + kWorkFields * (logical / p.n_tiles);  // a tile of the same expert
    first = any[3];
    count = any[4];
  }
  // Within the expert: super-rows of up to kSuperRows row tiles, N-tile-major inside each, so the
  // workgroups running together share a few row tiles and a few weight tiles (an expert with at
  // most kSuperRows row tiles is one super-row: all its row tiles of an N-tile side by side).
  const int64_t local = logical - p.n_tiles * first;
  const int64_t sr = local / (kSuperRows * p.n_tiles);
  const int64_t in_sr = count - sr * kSuperRows < kSuperRows ? count - sr * kSuperRows : kSuperRows;
  const int64_t rem = local - sr * kSuperRows * p.n_tiles;
  const int64_t nt = rem / in_sr, ti = first + sr * kSuperRows + rem % in_sr;
  int64_t e = 0, row0 = ti * BM;
  int nrows = (int)(p.P - row0 < BM ? p.P - row0 : BM);
  if (work) {
    e = work[1 + kWorkFields * ti];
    row0 = work[2 + kWorkFields * ti];
    nrows = work[3 + kWorkFields * ti];
  }
  const int8_t* wexp = p.w + e * p.N * p.K;

  const int tid = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave), wm = wv / WN, wn = wv % WN;
  static_assert(BM <= NT, "one tile row per thread");
  float my_as = 0.0f;  // row tid's scale, into LDS once the first stage has landed
  if (tid < BM) {
    const int32_t pid = tid < nrows ? (p.sorted ? p.sorted[row0 + tid] : (int32_t)(row0 + tid)) : (int32_t)p.P;
    sh_pid[tid] = pid;
    if (p.pair_row && nt == 0 && ks == 0 && tid < nrows) note_pair_row(p, pid, row0 + tid);
    if constexpr (has_row_scale<EPI>()) my_as = row_scale<EPI>(p, pid, row0 + tid);
  }

  // This thread's DMA chunks: stage chunk q holds row q / CPR, K-chunk (q % CPR) ^ swz(row); lane i
  // of an instruction lands 16 i bytes after the instruction's 1 KB slot.  Sources are 32-bit
  // offsets from the A matrix and from the expert's weights (the host checks they fit).  Rows past
  // the tile read row 0 (their results are never stored).  Gathered rows come from sh_pid: reading
  // the ids from global memory cost a round trip per chunk before the first DMA could go out.
  __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
  barrier_no_fence();  // sh_pid complete (the scale loads stay in flight)
  uint32_t off[LD];
#pragma unroll
  for (int c = 0; c < A_LD; ++c) {
    const int q = (wv * A_LD + c) * kWave + l, r = q / CPR, kc = (q % CPR) ^ swz(r);
    int64_t row = 0;
    if (r < nrows) row = p.gather ? (int64_t)(sh_pid[r] / p.k) : row0 + r;
    off[c] = (uint32_t)(row * p.K + ks * kslice + kc * 16);
  }
#pragma unroll
  for (int c = 0; c < B_LD; ++c) {
    const int q = (wv * B_LD + c) * kWave + l, j = q / CPR, kc = (q % CPR) ^ swz(j);
    off[A_LD + c] = (uint32_t)(wrow_of<BN, MAP>(nt, j, p.I) * p.K + ks * kslice + kc * 16);
  }
  const int a_dst = wv * A_LD * 1024, b_dst = BM * kDmaBK + wv * B_LD * 1024;

  i32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  const int g = l >> 4, fr = l & 15;
  const uint32_t fmask = real_frags<WM, BM / WM / 16, false>(wm, nrows);  // fragment rows with real rows

  // Prologue: stage 0 lands before the loop.
#pragma unroll
  for (int c = 0; c < LD; ++c) {
    if (c < A_LD)
      dma16(p.a + off[c], st0 + a_dst + c * 1024);
    else
      dma16_nt(wexp + off[c], st0 + b_dst + (c - A_LD) * 1024);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  if (has_row_scale<EPI>() && tid < BM) sh_as[tid] = my_as;  // read after the K loop's barriers

  // Step kt: every wavefront is done with step kt - 1 (barrier), so the other buffer is free; the
  // MFMAs read stage kt while the DMA of step kt + 1 goes out between them; then wait until it
  // has landed.  The step ends waiting on the last of those loads (the weights stream from HBM
  // once), so they all go out within the step's first kDmaSlots MFMA groups, activation rows
  // first: the gate+up GEMM at 8192 tokens took 2.59 ms with the loads spread over all 20 groups,
  // 2.40 ms within the first two, 2.44 ms all before the first group, 2.52 ms weights first.
  constexpr int kDmaSlots = 2;
  const int64_t KT = kslice / kDmaBK;
  for (int64_t kt = 0; kt < KT; kt += 2) {
    __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
    barrier_no_fence();
    dma_stage<BM, BN, WM, WN, A_LD, LD, MAP, false, kDmaSlots>(st0, st1, p.a, wexp, off, a_dst, b_dst,
                                                               (uint32_t)(kt + 1) * kDmaBK, true, acc, wm, wn, g, fr,
                                                               fmask);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
    __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
    barrier_no_fence();
    dma_stage<BM, BN, WM, WN, A_LD, LD, MAP, false, kDmaSlots>(st1, st0, p.a, wexp, off, a_dst, b_dst,
                                                               (uint32_t)(kt + 2) * kDmaBK, kt + 2 < KT, acc, wm, wn, g,
                                                               fr, fmask);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  }
  __syncthreads();
  dma_epilogue<BM, BN, WM, WN, STAGE, MAP, EPI>(p, acc, sh_pid, sh_as, st0, st1, row0, nt, e, wm, wn, wv, l,
                                                ks * p.P * p.N);
}

// One 4-byte-per-lane DMA (global_load_lds_dword): lane i's value lands at lds + 4 i.
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 4, 0, 0);
}

// Ring engine: the DMA engine's tiles and work order with an NS-stage LDS ring (NS = 3 for 8-bit
// weights: 128 x 256 tiles, 48 KB a stage; deeper for the half-size int4 stages).  Step kt reads
// stage kt, the DMA of stage kt + NS - 1 goes out between its MFMA groups, and at its end only
// stage kt + 1 must have landed, so NS - 1 stages stay in flight at all times.  The K loop (KT steps of 128 bytes, a compile-time count) is fully unrolled: every
// stage index and wait count is known, so the compiler tells the buffer being read from the two
// being filled, and no loop back edge joins in-flight DMA.
// Block-wise scales: each step is one 128-wide K-block, whose int32 partials are folded into the
// fp32 sums at the end of the step.  The tile's activation scales travel by DMA too, four K-blocks
// at a time next to the data stage of their first block (each wavefront brings 16 rows x 4 blocks
// into one of two buffers), so the data waits cover them; the weight scales of the tile's two
// 128-row weight blocks (every K-block) are read into LDS once, before the loop.
// Channel-wise: int32 sums over all of K, then the DMA engine's LDS-staged epilogue.
template <int BM, int BN, int WM, int WN, int KT, BMap MAP, Epi EPI, int NS = 3>
__global__ __launch_bounds__(WM * WN * kWave, 1) void grouped_gemm_ring_kernel(const Params p,
                                                                              const int32_t* __restrict__ work) {
  constexpr bool kBlock = is_block<EPI>();
  constexpr bool kFp8 = is_fp8<EPI>();
  constexpr bool kW4 = is_w4<EPI>();          // packed int4 weights, one scale per (row, K-block)
  constexpr bool kBlkScales = kBlock && !kW4;  // 128 x 128 weight-scale blocks
  using AccT = typename std::conditional<kFp8, f32x4, i32x4>::type;
  constexpr int NT = WM * WN * kWave;
  constexpr int NW = WM * WN;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr int CPR = kDmaBK / 16;
  constexpr int BKB = kW4 ? kDmaBK / 2 : kDmaBK;  // bytes of one B row per stage
  constexpr int CPRB = BKB / 16;
  constexpr int A_LD = BM * CPR / NT;
  constexpr int B_LD = BN * CPRB / NT;
  constexpr int LD = A_LD + B_LD;
  constexpr int STAGE = BM * kDmaBK + BN * BKB;
  constexpr int SG = 4;  // K-blocks per activation-scale DMA
  static_assert(EPI != Epi::I32 || !kW4, "raw int32 sums of 8-bit operands");
  static_assert(A_LD >= 1 && B_LD >= 1 && (BM * CPR) % NT == 0 && (BN * CPRB) % NT == 0, "tile shape");
  static_assert(KT >= 1 && (NS - 2) * (LD + 1) < 32, "K steps");
  // NS <= 5: the scale group a DMA overwrites was last read before the step that issues it
  static_assert(NS >= 3 && NS <= 5 && (NS == 3 || kW4), "ring depth");
  static_assert(!kW4 || (BN * KT) % kWave == 0, "scale table in whole 64-float chunks");
  // one scale DMA per wavefront: 16 rows x SG blocks (wavefronts past BM rows bring the first row's)
  static_assert(!kBlock || (NW * 16 >= BM && kWave == 16 * SG), "scale DMA shape");
  static_assert(!kBlkScales || BN == 256, "two 128-row weight-scale blocks per tile");
  static_assert(MAP == BMap::Plain || FN % 2 == 0, "split tiles need gate and up fragments");

  __shared__ __attribute__((aligned(1024))) int8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) int8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) int8_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) int8_t st3[NS > 3 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) int8_t st4[NS > 4 ? STAGE : 1];
  __shared__ __attribute__((aligned(16))) float sas0[kBlock ? NW * kWave : 1];  // activation scales, even groups
  __shared__ __attribute__((aligned(16))) float sas1[kBlock ? NW * kWave : 1];  // odd groups
  __shared__ float sh_ws[kBlkScales ? 2 : 1][kBlkScales ? KT : 1];
  __shared__ __attribute__((aligned(16))) float sh_wst[kW4 ? BN * KT : 1];  // int4: the tile rows' scales
  __shared__ int32_t sh_pid[BM];
  __shared__ float sh_as[has_row_scale<EPI>() ? BM : 1];
  __shared__ float sh_red[kBlock ? WN : 1][BM];

  // Raw int32 sums may split K into p.ksplit slices of KT steps (slice ks writes out_i32 + ks P N);
  // the other epilogues run over all of K (p.ksplit = 1, K = KT steps).
  const int64_t ksplit = EPI == Epi::I32 ? p.ksplit : 1;
  const int64_t ntl = work ? (int64_t)work[0] : (p.P + BM - 1) / BM;  // row tiles
  const int64_t total = ntl * p.n_tiles * ksplit;
  const int64_t per = (total + 7) / 8;
  const int64_t v = blockIdx.x;
  if (v >= 8 * per) return;
  const int64_t item = (v % 8) * per + v / 8;
  if (item >= total) return;
  const int64_t ks = item % ksplit, logical = item / ksplit;
  int64_t first = 0, count = ntl;
  if (work) {
    const int32_t* any = work + 1 + kWorkFields * (logical / p.n_tiles);
    first = any[3];
    count = any[4];
  }
  const int64_t local = logical - p.n_tiles * first;
  const int64_t sr = local / (kRingSuperRows * p.n_tiles);
  const int64_t in_sr =
      count - sr * kRingSuperRows < kRingSuperRows ? count - sr * kRingSuperRows : kRingSuperRows;
  const int64_t rem = local - sr * kRingSuperRows * p.n_tiles;
  const int64_t nt = rem / in_sr, ti = first + sr * kRingSuperRows + rem % in_sr;
  int64_t e = 0, row0 = ti * BM;
  int nrows = (int)(p.P - row0 < BM ? p.P - row0 : BM);
  if (work) {
    e = work[1 + kWorkFields * ti];
    row0 = work[2 + kWorkFields * ti];
    nrows = work[3 + kWorkFields * ti];
  }
  const int64_t wrow_bytes = kW4 ? p.K / 2 : p.K;
  const int64_t k0 = ks * KT * kDmaBK;  // first K byte of this slice (8-bit operands)
  const int8_t* wexp = p.w + e * p.N * wrow_bytes + k0;
  const int8_t* abase = p.a + k0;

  const int tid = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave), wm = wv / WN, wn = wv % WN;
  const int g = l >> 4, fr = l & 15;
  static_assert(BM <= NT, "one tile row per thread");
  float my_as = 0.0f;  // row tid's scale, into LDS once the first stage has landed
  if (tid < BM) {
    const int32_t pid = tid < nrows ? (p.sorted ? p.sorted[row0 + tid] : (int32_t)(row0 + tid)) : (int32_t)p.P;
    sh_pid[tid] = pid;
    if (p.pair_row && nt == 0 && ks == 0 && tid < nrows) note_pair_row(p, pid, row0 + tid);
    if constexpr (has_row_scale<EPI>()) my_as = row_scale<EPI>(p, pid, row0 + tid);
  }
  if constexpr (kBlkScales) {
    for (int i = tid; i < 2 * KT; i += NT) {
      const int64_t blk = wrow_of<BN, MAP>(nt, (i / KT) * 128, p.I) / 128;
      sh_ws[i / KT][i % KT] = p.w_s[(e * (p.N / 128) + blk) * KT + i % KT];
    }
  }
  __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
  barrier_no_fence();  // sh_pid, sh_ws complete (the row-scale loads stay in flight)
  // Source row of a tile row; rows past the real ones read the first row (finite values whose
  // results are never stored).  Gathered rows come from sh_pid, not from global memory (a round
  // trip per DMA chunk before the first stage could go out).
  auto src_row = [&](int r) -> int64_t {
    const int64_t rr = r < nrows ? r : 0;
    return p.gather ? (int64_t)(sh_pid[rr] / p.k) : row0 + rr;
  };

  uint32_t off[LD];
#pragma unroll
  for (int c = 0; c < A_LD; ++c) {
    const int q = (wv * A_LD + c) * kWave + l, r = q / CPR, kc = (q % CPR) ^ swz(r);
    off[c] = (uint32_t)(src_row(r) * p.K + kc * 16);
  }
#pragma unroll
  for (int c = 0; c < B_LD; ++c) {
    const int q = (wv * B_LD + c) * kWave + l, j = q / CPRB, kc = (q % CPRB) ^ (kW4 ? swz4(j) : swz(j));
    off[A_LD + c] = (uint32_t)(wrow_of<BN, MAP>(nt, j, p.I) * wrow_bytes + kc * 16);
  }

  // activation-scale DMA: lane l brings row wv * 16 + (l & 15) of K-block group * SG + l / 16
  // (the last K-block again where a group runs past K)
  const uint32_t s_off = kBlock ? (uint32_t)(src_row(wv * 16 + (l & 15)) * KT) : 0u;
  auto s_blk = [&](int q) { return (uint32_t)min(q * SG + (l >> 4), KT - 1); };
  const int a_dst = wv * A_LD * 1024, b_dst = BM * kDmaBK + wv * B_LD * 1024;

  AccT acc[FM][FN];
  float accf[FM][FN][kBlock ? 4 : 1];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[i][j] = AccT{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < (kBlock ? 4 : 1); ++r) accf[i][j][r] = 0.0f;
    }
  // fragment rows interleaved over the two wavefront rows, so a tile with fewer real rows than BM (an
  // expert's last tile, or experts with about BM / 2 rows) keeps both wavefront rows busy (block-wise
  // T = 2048: 2.46 -> 2.41 ms INT8, 2.44 -> 2.40 ms FP8); not for int4 weights, whose widening both
  // wavefront rows would then repeat (2.57 -> 2.69 ms)
  constexpr bool ILV = WM > 1 && !kW4;
  const uint32_t fmask = real_frags<WM, FM, ILV>(wm, nrows);  // fragment rows with real rows

#define W8A8_RSTG(j) ((j) % NS == 0 ? st0 : (j) % NS == 1 ? st1 : (j) % NS == 2 ? st2 : (j) % NS == 3 ? st3 : st4)
  // VMEM operations that stage st brings: its DMAs, and with every SG-th stage its scale group
  auto stage_ops = [&](int st) { return st < KT ? LD + ((kBlock && st % SG == 0) ? 1 : 0) : 0; };
#define W8A8_RSAS(q) (((q) & 1) ? sas1 : sas0)
  if constexpr (kW4) {
    // int4 weights: the scales of the tile's BN weight rows for every K-block ([BN][KT], one per
    // (row, K-block)) go to LDS by DMA ahead of the first stage, so the prologue wait covers them;
    // chunk c of 64 floats is table entries 64 c .. 64 c + 63
    for (int c = wv; c < (BN * KT) / kWave; c += NW) {
      const int f = c * kWave + l, j = f / KT;
      dma4(p.w_s + ((e * p.N + wrow_of<BN, MAP>(nt, j, p.I)) * KT + (f - j * KT)), sh_wst + c * kWave);
    }
  }
  constexpr int PRE = KT < NS - 1 ? KT : NS - 1;  // stages loaded before the loop
#pragma unroll
  for (int st = 0; st < PRE; ++st) {
#pragma unroll
    for (int c = 0; c < LD; ++c) {
      if (c < A_LD)
        dma16(abase + (off[c] + (uint32_t)(st * kDmaBK)), W8A8_RSTG(st) + a_dst + c * 1024);
      else
        (kW4 ? dma16 : dma16_nt)(wexp + (off[c] + (uint32_t)(st * BKB)), W8A8_RSTG(st) + b_dst + (c - A_LD) * 1024);
    }
    if (kBlock && st % SG == 0) dma4(p.a_s + (s_off + s_blk(st / SG)), W8A8_RSAS(st / SG) + wv * kWave);
  }
  {  // stage 0 (and the first scale group) landed: only stages 1 .. PRE - 1 may be outstanding
    int later = 0;
#pragma unroll
    for (int st = 1; st < PRE; ++st) later += stage_ops(st);
    vm_wait(later);
  }
  if (has_row_scale<EPI>() && tid < BM) sh_as[tid] = my_as;  // read after the K loop's barriers

  // Uniform bases of the stage two steps ahead, advanced one step at a time; the empty asm keeps
  // the compiler from precomputing every step's address up front.
  const int8_t* a_next = abase + (NS - 1) * kDmaBK;
  const int8_t* b_next = wexp + (NS - 1) * BKB;
#pragma clang loop unroll(full)
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
    barrier_no_fence();
    const int nxt = kt + NS - 1;  // the stage whose DMA goes out in this step
    const bool more = nxt < KT;
    const bool sdma = kBlock && more && nxt % SG == 0;  // with its scale group
    if (sdma) dma4(p.a_s + (s_off + s_blk(nxt / SG)), W8A8_RSAS(nxt / SG) + wv * kWave);
    if constexpr (kW4)
      dma_stage_w4<BM, BN, WM, WN, A_LD, LD, MAP, ILV>(W8A8_RSTG(kt), W8A8_RSTG(nxt), a_next, b_next, off, a_dst,
                                                       b_dst, 0u, more, acc, wm, wn, g, fr, fmask);
    else if constexpr (kFp8)
      dma_stage_f8<BM, BN, WM, WN, A_LD, LD, MAP, ILV>(W8A8_RSTG(kt), W8A8_RSTG(nxt), a_next, b_next, off, a_dst,
                                                       b_dst, 0u, more, acc, wm, wn, g, fr, fmask);
    else
      dma_stage<BM, BN, WM, WN, A_LD, LD, MAP, ILV>(W8A8_RSTG(kt), W8A8_RSTG(nxt), a_next, b_next, off, a_dst, b_dst,
                                                    0u, more, acc, wm, wn, g, fr, fmask);
    a_next += kDmaBK;
    b_next += BKB;
    asm volatile("" : "+s"(a_next), "+s"(b_next));
    if constexpr (kBlock) {
      if (fmask != 0u) {
        float as[FM][4], ws[FN];
        const float* sa = W8A8_RSAS(kt / SG) + (kt % SG) * 16 + (l >> 4) * 4;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(sa + rblk<WM, FM, ILV>(wm, fm) * kWave);
#pragma unroll
          for (int r = 0; r < 4; ++r) as[fm][r] = s4[r];
        }
        if constexpr (kW4) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) ws[fn] = sh_wst[(brow_of<BN, WN, FN, MAP>(wn, fn) + (l & 15)) * KT + kt];
        } else {
          const float w0 = sh_ws[0][kt], w1 = sh_ws[1][kt];
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) ws[fn] = brow_of<BN, WN, FN, MAP>(wn, fn) >= 128 ? w1 : w0;
        }
        block_flush<FM, FN, AccT>(acc, accf, as, ws, fmask);
      }
    }
    {  // stage kt + 1 landed: only the stages after it may be outstanding
      int later = 0;
#pragma unroll
      for (int st = kt + 2; st < kt + NS; ++st) later += stage_ops(st);
      vm_wait(later);
    }
  }
#undef W8A8_RSAS
#undef W8A8_RSTG
  __syncthreads();
  if constexpr (kBlock)
    epilogue<BM, BN, WM, WN, FM, FN, MAP, EPI, ILV>(p, acc, accf, sh_pid, sh_as, sh_red, row0, nt, e, wm, wn, l, tid);
  else
    dma_epilogue<BM, BN, WM, WN, STAGE, MAP, EPI, ILV>(p, acc, sh_pid, sh_as, st0, st1, row0, nt, e, wm, wn, wv, l,
                                                       ks * p.P * p.N);
}

// Streaming engine for packed int4 weights when experts hold few rows (decode): tiles of 16 rows
// x 256 weight rows on four wavefronts that share nothing until the epilogue.  Wavefront wn owns
// 64 weight rows (FN = 4 fragments); for each 128-wide K-block lane (g, fr) needs the 16 bytes
// (32 int4 values, K values 32 g .. 32 g + 31 of the block) of weight row fr of each fragment, widens
// them to E4M3 codes, and takes the matching 32 activation codes of tile row fr from the (L1/L2-
// resident) activation rows.  The weights are loaded straight into registers with the non-temporal
// policy, two K-blocks (one 128-byte line of each row) per pair of load instructions that each cover
// whole lines, and put in place by one DPP row shift per dword (see the loads); loading each lane's
// own 16 bytes instead covered half of each line per instruction and ran the weight stream at 4.9
// instead of 5.7 TB/s.  PD pairs of K-blocks are in flight ahead of the pair being multiplied, and no
// barrier or LDS round trip sits between a load and its MFMA.
// Scales: lane (g, fr) holds four consecutive K-blocks (4 g .. 4 g + 3 of a 16-block window) of
// the weight scale of row fr of each fragment and of the activation scale of tile row fr; each
// K-block's values are fetched from the owning lane by a cross-lane read (ds_bpermute).  Each
// K-block's FP8 MFMA sum starts from zero and is folded into the fp32 sums as
// acc + ((part * a_s) * w_s), in ascending K-block order.
constexpr int kStreamBM = 16, kStreamBN = 256, kStreamWN = 4;
template <int KT, BMap MAP, Epi EPI>
__global__ __launch_bounds__(kStreamWN * kWave) void grouped_gemm_w4_stream_kernel(const Params p,
                                                                                  const int32_t* __restrict__ work) {
  static_assert(is_w4<EPI>(), "packed int4 weights");
  constexpr int BM = kStreamBM, BN = kStreamBN, WN = kStreamWN;
  constexpr int FN = BN / WN / 16, FNH = FN / 2;
  constexpr int PD = 1, NB = PD + 1;  // K-block pairs in flight ahead of the current one; register slots
  constexpr int WIN = 16;             // K-blocks per scale window (four per lane group)
  constexpr int NWIN = (KT + WIN - 1) / WIN;
  constexpr int kScaleOne = 127;
  static_assert(KT >= 1 && (MAP == BMap::Plain || FN % 2 == 0), "shape");
  __shared__ int32_t sh_pid[BM];
  __shared__ float sh_red[WN][BM];

  const int64_t total = (int64_t)work[0] * p.n_tiles;
  const int64_t per = (total + 7) / 8;
  const int64_t v = blockIdx.x;
  if (v >= 8 * per) return;
  // consecutive items on one XCD (workgroups are dealt round-robin over the 8 XCDs), so the row
  // tiles of one expert that read the same weight rows meet in that XCD's L2
  const int64_t logical = (v % 8) * per + v / 8;
  if (logical >= total) return;
  const int64_t ti = logical / p.n_tiles, nt = logical % p.n_tiles;
  const int64_t e = work[1 + kWorkFields * ti];
  const int64_t row0 = work[2 + kWorkFields * ti];
  const int nrows = work[3 + kWorkFields * ti];
  const int64_t KB = p.K / 2;  // bytes of one packed weight row
  const int8_t* wexp = p.w + e * p.N * KB;

  const int tid = threadIdx.x, l = lane_id();
  const int wn = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = l >> 4, fr = l & 15;
  for (int i = tid; i < BM; i += WN * kWave) {
    sh_pid[i] = i < nrows ? p.sorted[row0 + i] : (int32_t)p.P;
    if (p.pair_row && nt == 0 && i < nrows) note_pair_row(p, sh_pid[i], row0 + i);
  }

  // tile row fr (rows past the real ones read the first row: finite values, never stored)
  const int64_t rr = fr < nrows ? fr : 0;
  const int64_t arow = p.gather ? (int64_t)(p.sorted[row0 + rr] / p.k) : row0 + rr;
  const int8_t* a_src = p.a + arow * p.K + g * 32;
  const float* as_src = p.a_s + arow * KT;
  // Weights go in whole 128-byte lines: a K-block pair (2q, 2q + 1) is one line of each row.  Load X
  // covers the fragment's rows 0-7, load Y rows 8-15; lane (g, fr) takes row fr % 8 (resp. 8 + fr % 8)
  // and 16-byte chunk g + 4 (fr / 8) of the line.  X then holds in lanes fr < 8 exactly the MFMA
  // operand of K-block 2q (row fr, chunk g) and Y in lanes fr >= 8 that of K-block 2q + 1; the other
  // halves come one DPP row shift by 8 lanes away (see below).
  const int8_t* b_src[FN];
  const float* ws_src[FN];
  const int bchunk = g + 4 * (fr >> 3);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int brow = brow_of<BN, WN, FN, MAP>(wn, fn);
    b_src[fn] = wexp + wrow_of<BN, MAP>(nt, brow + (fr & 7), p.I) * KB;
    ws_src[fn] = p.w_s + (e * p.N + wrow_of<BN, MAP>(nt, brow + fr, p.I)) * KT;
  }
  const int64_t y_off = 8 * KB;  // rows 8-15 of a fragment (the fragment's 16 rows are consecutive)

  i32x4 bx[NB][FN], by[NB][FN], aq[NB][2][2];
  // pair q into register slot `slot`; with an odd KT the last pair has one K-block, whose line half
  // is read twice (the second copy is never used)
  auto load = [&](int q, int slot) {
    const int chunk = 2 * q + 1 < KT ? bchunk : (bchunk & 3);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int8_t* src = b_src[fn] + q * kDmaBK + chunk * 16;
      bx[slot][fn] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src));
      by[slot][fn] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src + y_off));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (2 * q + h >= KT) break;
      aq[slot][h][0] = *reinterpret_cast<const i32x4*>(a_src + (2 * q + h) * kDmaBK);
      aq[slot][h][1] = *reinterpret_cast<const i32x4*>(a_src + (2 * q + h) * kDmaBK + 16);
    }
  };
  float wsw[2][FN][4], asw[2][4];
  auto load_scales = [&](int w, int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kb = min(w * WIN + 4 * g + i, KT - 1);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) wsw[set][fn][i] = ws_src[fn][kb];
      asw[set][i] = as_src[kb];
    }
  };

  float accf[1][FN][4];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int r = 0; r < 4; ++r) accf[0][fn][r] = 0.0f;

  constexpr int NP = (KT + 1) / 2;  // K-block pairs
#pragma unroll
  for (int s = 0; s < PD; ++s)
    if (s < NP) load(s, s);
  load_scales(0, 0);
#pragma clang loop unroll(full)
  for (int kb = 0; kb < KT; ++kb) {
    const int q = kb / 2, h = kb % 2;
    if (h == 0 && q + PD < NP) load(q + PD, (q + PD) % NB);
    if (kb % WIN == 0 && kb / WIN + 1 < NWIN) load_scales(kb / WIN + 1, (kb / WIN + 1) & 1);
    const int slot = q % NB, set = (kb / WIN) & 1;
    const int src = ((kb % WIN) / 4) * 16;  // lane group holding this K-block's scales
    i32x8 bf[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // K-block 2q: X, lanes 8-15 of each 16-lane row from Y 8 lanes down (row_shr:8, banks 2-3);
        // K-block 2q + 1: Y, lanes 0-7 from X 8 lanes up (row_shl:8, banks 0-1)
        const int32_t w = h == 0 ? __builtin_amdgcn_update_dpp(bx[slot][fn][d], by[slot][fn][d], 0x118, 0xF, 0xC, false)
                                 : __builtin_amdgcn_update_dpp(by[slot][fn][d], bx[slot][fn][d], 0x108, 0xF, 0x3, false);
        w4_to_fp8((uint32_t)w, o[2 * d], o[2 * d + 1]);
      }
      bf[fn] = i32x8{o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
    }
    const i32x8 af = i32x8{aq[slot][h][0][0], aq[slot][h][0][1], aq[slot][h][0][2], aq[slot][h][0][3],
                           aq[slot][h][1][0], aq[slot][h][1][1], aq[slot][h][1][2], aq[slot][h][1][3]};
    f32x4 part[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      part[fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[fn], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                                  0, kScaleOne, 0, kScaleOne);
    float as[4], ws[FN];
#pragma unroll
    for (int r = 0; r < 4; ++r) as[r] = __shfl(asw[set][kb % 4], src + g * 4 + r, kWave);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) ws[fn] = __shfl(wsw[set][fn][kb % 4], src + fr, kWave);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[0][fn][r] = accf[0][fn][r] + ((part[fn][r] * as[r]) * ws[fn]);
  }
  // The down GEMM's epilogue reads the sums only inside per-row conditional stores; this empty
  // asm takes them as operands after the loop, so the compiler cannot sink every fold into those
  // stores (keeping all K-blocks' partial sums live to the end), while the loop itself stays one
  // scheduling region.
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
    asm volatile("" : "+v"(accf[0][fn][0]), "+v"(accf[0][fn][1]), "+v"(accf[0][fn][2]), "+v"(accf[0][fn][3]));
  (void)FNH;
  i32x4 unused[1][FN] = {};  // the block-wise epilogues read only the fp32 sums
  __syncthreads();  // sh_pid
  static_assert(!has_row_scale<EPI>(), "block-wise epilogues take no row scales");
  epilogue<BM, BN, 1, WN, 1, FN, MAP, EPI>(p, unused, accf, sh_pid, nullptr, sh_red, row0, nt, e, 0, wn, l, tid);
}

// Work list of the DMA engine: per expert, tiles of up to bmk real rows of its sorted segment.
// work[0] = number of tiles; tile i = (expert, first sorted row, rows, index of the expert's
// first tile, number of the expert's tiles) at work[1 + kWorkFields * i].
constexpr int kListThreads = 1024;

__device__ int list_exclusive_scan(int v, int* wsum, int& total) {
  const int l = lane_id(), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (l >= o) x += y;
  }
  if (l == kWave - 1) wsum[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int i = 0; i < kListThreads / kWave; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kListThreads) void build_tiles_kernel(const int32_t* __restrict__ sorted,
                                                                   const int32_t* __restrict__ padded_offsets, int E,
                                                                   int32_t P, int bmk, int32_t* __restrict__ work) {
  __shared__ int wsum[kListThreads / kWave];
  const int e = threadIdx.x;
  int cnt = 0, seg = 0;
  if (e < E) {
    // real rows are the prefix of the segment below the sentinel P
    seg = padded_offsets[e];
    int lo = seg, hi = padded_offsets[e + 1];
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sorted[mid] < P)
        lo = mid + 1;
      else
        hi = mid;
    }
    cnt = lo - seg;
  }
  const int tiles = (cnt + bmk - 1) / bmk;
  int total;
  const int off = list_exclusive_scan(tiles, wsum, total);
  for (int i = 0; i < tiles; ++i) {
    int32_t* t = work + 1 + kWorkFields * (off + i);
    t[0] = e;
    t[1] = seg + i * bmk;
    t[2] = min(bmk, cnt - i * bmk);
    t[3] = off;
    t[4] = tiles;
  }
  if (e == 0) work[0] = total;
}

// ---------------------------------------------------------------------------------------------
// Channel-wise requantization of the first GEMM's rows: one wavefront per row (grid stride), each
// lane with eight float4 loads of its row in flight before it quantizes them (one load round trip
// per 2048 columns instead of one per 256).
__global__ __launch_bounds__(kThreads) void requant_rows_kernel(const float* __restrict__ hf,
                                                                const float* __restrict__ part_amax,
                                                                const int32_t* __restrict__ sorted,
                                                                const int32_t* __restrict__ num_tiles, int64_t block_m,
                                                                int64_t P, int64_t I, int64_t n_tiles,
                                                                int8_t* __restrict__ h_q, float* __restrict__ h_s) {
  const int64_t used = (int64_t)num_tiles[0] * block_m;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / kWave);
  for (int64_t r = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave; r < used; r += stride) {
    if (sorted[r] >= P) continue;
    const int l = lane_id();
    float m = 0.0f;
    for (int64_t i = l; i < n_tiles; i += kWave) m = fmaxf(m, part_amax[r * n_tiles + i]);
    const float s = quant_scale(wave_max(m));
    if (l == 0) h_s[r] = s;
    const f32x4* src = reinterpret_cast<const f32x4*>(hf + r * I);
    uint32_t* dst = reinterpret_cast<uint32_t*>(h_q + r * I);
    constexpr int U = 8;  // float4 loads in flight per lane
    for (int64_t c0 = l; c0 < I / 4; c0 += kWave * U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + (int64_t)u * kWave;
        v[u] = c < I / 4 ? __builtin_nontemporal_load(src + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + (int64_t)u * kWave;
        if (c < I / 4)
          dst[c] = (uint32_t)(uint8_t)quant_value(v[u].x, s) | ((uint32_t)(uint8_t)quant_value(v[u].y, s) << 8) |
                   ((uint32_t)(uint8_t)quant_value(v[u].z, s) << 16) |
                   ((uint32_t)(uint8_t)quant_value(v[u].w, s) << 24);
      }
    }
  }
}

// out[t, n] = 0 + w[t,0] * y0 + w[t,1] * y1 + ... in slot order.  One token per workgroup row
// (its slot rows and weights are uniform, so they come through scalar loads); each thread sums
// kCombineVec float4 columns, all of a slot's loads in flight together.  pair_row is written by
// the second GEMM for this call's pairs only (a pair the align dropped keeps whatever an earlier
// call left): a slot counts when its row lies in this call's rows and holds that very pair.
// Tokens beyond the grid's kMaxGridBlocks rows of workgroups are taken with a grid stride.
constexpr int kCombineVec = 4;
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y,
                                                           const int32_t* __restrict__ pair_row,
                                                           const int32_t* __restrict__ sorted,
                                                           const int32_t* __restrict__ num_tiles, int64_t block_m,
                                                           const float* __restrict__ topk_w, int64_t T, int64_t k,
                                                           int64_t H, float* __restrict__ out) {
  const int64_t H4 = H / 4;
  const int64_t c0 = (int64_t)blockIdx.y * kThreads * kCombineVec + threadIdx.x;
  const int64_t used = (int64_t)num_tiles[0] * block_m;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    float4 o[kCombineVec];
#pragma unroll
    for (int i = 0; i < kCombineVec; ++i) o[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t j = 0; j < k; ++j) {
      const int32_t r = pair_row[t * k + j];
      if (r < 0 || r >= used || sorted[r] != t * k + j) continue;
      const float wj = topk_w[t * k + j];
      const float4* src = reinterpret_cast<const float4*>(y + (int64_t)r * H);
      float4 v[kCombineVec];
#pragma unroll
      for (int i = 0; i < kCombineVec; ++i) {
        const int64_t c = c0 + i * kThreads;
        if (c < H4) {
          const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + c);
          v[i] = make_float4(q.x, q.y, q.z, q.w);
        } else {
          v[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
#pragma unroll
      for (int i = 0; i < kCombineVec; ++i) {
        o[i].x = o[i].x + wj * v[i].x;
        o[i].y = o[i].y + wj * v[i].y;
        o[i].z = o[i].z + wj * v[i].z;
        o[i].w = o[i].w + wj * v[i].w;
      }
    }
    float4* dst = reinterpret_cast<float4*>(out + t * H);
#pragma unroll
    for (int i = 0; i < kCombineVec; ++i) {
      const int64_t c = c0 + i * kThreads;
      if (c < H4) dst[c] = o[i];
    }
  }
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Work list of the dense linear: one "expert", rows in their own order, tiles of bmk rows.
// ---------------------------------------------------------------------------------------------
// Engine choice and launches.

constexpr int kBNStaged = 128;   // staged engine: 64 gate + 64 up rows, or 128 output columns
constexpr int kBNBlock13 = 256;  // staged block-wise first GEMM: 128 gate + 128 up rows (one requant group)
constexpr int kDmaBM = 320;      // DMA engine: 320 x 256 tiles on 2 x 4 wavefronts of 160 x 64
constexpr int kDmaBN = 256;      // 128 gate + 128 up rows, or 256 output columns
constexpr int kDmaWM = 2, kDmaWN = 4;

int64_t dma_max_tiles(const GroupedShape& s, int64_t bm = kDmaBM) {
  const int64_t P = s.T * s.k;
  return (P + bm - 1) / bm + std::min<int64_t>(s.E, P);
}

// The work-list engines launch all (row tile, N-tile) items of a GEMM in one grid: they take only
// shapes whose items, for the wider N-tiling of the two GEMMs, stay within kMaxGridBlocks.
bool list_grid_fits(const GroupedShape& s, int64_t bm, int64_t bn) {
  return dma_max_tiles(s, bm) * std::max(s.I / (bn / 2), s.H / bn) <= kMaxGridBlocks;
}

// The DMA engine pays off once experts hold tens of rows (on average 64 or more here); its K steps
// go in pairs and its down GEMM's N-tiles are 256 wide, so hidden and intermediate sizes must be
// multiples of 256; other shapes run on the staged engine.
// Its DMA sources are 32-bit offsets into the activation or intermediate matrix and into one expert.
bool use_dma(const GroupedShape& s) {
  return s.T * s.k >= 64 * s.E && s.H % 256 == 0 && s.I % 256 == 0 && (uint64_t)s.T * s.H < (1ull << 32) &&
         (uint64_t)s.max_rows * s.I < (1ull << 32) && (uint64_t)2 * s.I * s.H < (1ull << 32) &&
         list_grid_fits(s, kDmaBM, kDmaBN);
}

// Ring engine: 128-row tiles, its K loops unrolled for the DeepSeek-V3 layer (hidden 7168,
// intermediate 2048).  Block-wise it takes every batch with 16 or more rows per expert on average;
// channel-wise the batches between that and kRingMaxAvgRows rows per expert, above which the
// 320-row tiles of the DMA engine feed the MFMAs with fewer bytes per operation.
constexpr int kRingBM = 128;
constexpr int kRingSmallBM = 64;  // FP8 / W4A8 at the DeepSeek-V3 shapes with fewer than 32 rows per expert
constexpr int kRingH = 7168, kRingI = 2048;
constexpr int64_t kRingMinAvgRows = 16, kRingMaxAvgRows = 192;
bool use_ring(const GroupedShape& s, int32_t scale_mode) {
  const int64_t P = s.T * s.k;
  return P >= kRingMinAvgRows * s.E && (scale_mode == 1 || P < kRingMaxAvgRows * s.E) && s.H == kRingH &&
         s.I == kRingI && (uint64_t)s.T * s.H < (1ull << 32) && (uint64_t)s.max_rows * s.I < (1ull << 32) &&
         list_grid_fits(s, kRingBM, kDmaBN);
}

// Tile lists of every work-list engine fit (the streaming engine's 16-row tiles are the most).
size_t work_bytes(const GroupedShape& s) {
  return round256(sizeof(int32_t) * (size_t)(1 + kWorkFields * dma_max_tiles(s, kStreamBM)));
}

// N-tiles of the first GEMM (one row maximum each per row).
int64_t w13_n_tiles(const GroupedShape& s, int32_t scale_mode) {
  if (scale_mode == 1) return s.I / (kBNBlock13 / 2);
  return use_ring(s, scale_mode) || use_dma(s) ? s.I / (kDmaBN / 2) : s.I / (kBNStaged / 2);
}

// One workgroup per (row tile, N-tile) item, in launches of at most kMaxGridBlocks items.
template <int BM, int BN, int WM, int WN, BMap MAP, Epi EPI>
hipError_t launch_staged(Params prm, int64_t max_rows, hipStream_t stream) {
  const int64_t items = (max_rows / BM) * prm.n_tiles;
  for (int64_t b0 = 0; b0 < items; b0 += kMaxGridBlocks) {
    prm.block0 = b0;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, MAP, EPI>),
                       dim3((uint32_t)std::min(items - b0, kMaxGridBlocks)), dim3(kThreads), 0, stream, prm);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Staged engine, tile height = block_m (64 for the block-wise first GEMM's 128-row tiles).
template <BMap MAP, Epi EPI, int BN>
hipError_t launch_bm(Params prm, int64_t max_rows, hipStream_t stream) {
  prm.n_tiles = MAP == BMap::Plain ? prm.N / BN : prm.I / (BN / 2);
  switch (prm.block_m) {
    case 16: return launch_staged<16, BN, 1, 4, MAP, EPI>(prm, max_rows, stream);
    case 32: return launch_staged<32, BN, 1, 4, MAP, EPI>(prm, max_rows, stream);
    case 64: return launch_staged<64, BN, 2, 2, MAP, EPI>(prm, max_rows, stream);
    default: return launch_staged<(EPI == Epi::W13Block ? 64 : 128), BN, 2, 2, MAP, EPI>(prm, max_rows, stream);
  }
}

template <BMap MAP, Epi EPI>
hipError_t launch_dma(Params prm, const GroupedShape& s, const int32_t* padded_offsets, int32_t* work,
                      hipStream_t stream) {
  prm.n_tiles = MAP == BMap::Plain ? prm.N / kDmaBN : prm.I / (kDmaBN / 2);
  prm.ksplit = 1;
  const int64_t grid = (dma_max_tiles(s) * prm.n_tiles + 7) / 8 * 8;
  if (grid > kMaxGridBlocks) return hipErrorInvalidConfiguration;  // shape gates keep it below
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kListThreads), 0, stream, prm.sorted, padded_offsets,
                     (int)s.E, (int32_t)prm.P, kDmaBM, work);
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<kDmaBM, kDmaBN, kDmaWM, kDmaWN, MAP, EPI>),
                     dim3((uint32_t)grid), dim3(kDmaWM * kDmaWN * kWave), 0, stream, prm, (const int32_t*)work);
  return hipGetLastError();
}

template <BMap MAP, Epi EPI, int KT, int BM = kRingBM>
hipError_t launch_ring(Params prm, const GroupedShape& s, const int32_t* padded_offsets, int32_t* work,
                            hipStream_t stream) {
  constexpr int NS = 3;
  prm.n_tiles = MAP == BMap::Plain ? prm.N / kDmaBN : prm.I / (kDmaBN / 2);
  prm.ksplit = 1;
  const int64_t grid = (dma_max_tiles(s, BM) * prm.n_tiles + 7) / 8 * 8;
  if (grid > kMaxGridBlocks) return hipErrorInvalidConfiguration;  // shape gates keep it below
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kListThreads), 0, stream, prm.sorted, padded_offsets,
                     (int)s.E, (int32_t)prm.P, BM, work);
  // 64-row tiles: all 8 wavefronts side by side along N (64 x 32 each), so at a handful of rows
  // per expert every wavefront has rows and the per-step widening and folding is split 8 ways
  constexpr int WM = BM == kRingSmallBM ? 1 : kDmaWM, WN = BM == kRingSmallBM ? 8 : kDmaWN;
  hipLaunchKernelGGL((grouped_gemm_ring_kernel<BM, kDmaBN, WM, WN, KT, MAP, EPI, NS>), dim3((uint32_t)grid),
                     dim3(WM * WN * kWave), 0, stream, prm, (const int32_t*)work);
  return hipGetLastError();
}

// FP8 and W4A8 operands take the ring engine, W4A8 with fewer than kStreamMaxAvgRows rows per
// expert on average the streaming engine; K sizes with an instantiated kernel (K / 128).
bool fp8_kt_ok(int64_t kt) { return kt == 1 || kt == 2 || kt == 4 || kt == 8 || kt == 16 || kt == 32 || kt == 56; }
constexpr int64_t kStreamMaxAvgRows = 16;

template <BMap MAP, Epi EPI, int KT>
hipError_t launch_w4_stream(Params prm, const GroupedShape& s, const int32_t* padded_offsets, int32_t* work,
                            hipStream_t stream) {
  prm.n_tiles = MAP == BMap::Plain ? prm.N / kStreamBN : prm.I / (kStreamBN / 2);
  prm.ksplit = 1;
  const int64_t grid = (dma_max_tiles(s, kStreamBM) * prm.n_tiles + 7) / 8 * 8;
  if (grid > kMaxGridBlocks) return hipErrorInvalidConfiguration;  // shape gates keep it below
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kListThreads), 0, stream, prm.sorted, padded_offsets,
                     (int)s.E, (int32_t)prm.P, kStreamBM, work);
  hipLaunchKernelGGL((grouped_gemm_w4_stream_kernel<KT, MAP, EPI>), dim3((uint32_t)grid), dim3(kStreamWN * kWave), 0,
                     stream, prm, (const int32_t*)work);
  return hipGetLastError();
}

template <BMap MAP, Epi EPI>
hipError_t launch_ring_kt(const Params& prm, const GroupedShape& s, const int32_t* padded_offsets, int32_t* work,
                          hipStream_t stream) {
  if constexpr (is_w4<EPI>()) {
    if (s.T * s.k < kStreamMaxAvgRows * s.E) {
      switch (prm.K / kDmaBK) {
        case 1: return launch_w4_stream<MAP, EPI, 1>(prm, s, padded_offsets, work, stream);
        case 2: return launch_w4_stream<MAP, EPI, 2>(prm, s, padded_offsets, work, stream);
        case 4: return launch_w4_stream<MAP, EPI, 4>(prm, s, padded_offsets, work, stream);
        case 8: return launch_w4_stream<MAP, EPI, 8>(prm, s, padded_offsets, work, stream);
        case 16: return launch_w4_stream<MAP, EPI, 16>(prm, s, padded_offsets, work, stream);
        case 32: return launch_w4_stream<MAP, EPI, 32>(prm, s, padded_offsets, work, stream);
        case 56: return launch_w4_stream<MAP, EPI, 56>(prm, s, padded_offsets, work, stream);
        default: return hipErrorInvalidValue;
      }
    }
  }
  // few rows per expert (decode) at the DeepSeek-V3 shapes: 64-row tiles halve the redundant A stream
  if (s.H == kRingH && s.I == kRingI && s.T * s.k < 32 * s.E) {
    if (prm.K / kDmaBK == kRingH / kDmaBK)
      return launch_ring<MAP, EPI, kRingH / kDmaBK, kRingSmallBM>(prm, s, padded_offsets, work, stream);
    return launch_ring<MAP, EPI, kRingI / kDmaBK, kRingSmallBM>(prm, s, padded_offsets, work, stream);
  }
  switch (prm.K / kDmaBK) {
    case 1: return launch_ring<MAP, EPI, 1>(prm, s, padded_offsets, work, stream);
    case 2: return launch_ring<MAP, EPI, 2>(prm, s, padded_offsets, work, stream);
    case 4: return launch_ring<MAP, EPI, 4>(prm, s, padded_offsets, work, stream);
    case 8: return launch_ring<MAP, EPI, 8>(prm, s, padded_offsets, work, stream);
    case 16: return launch_ring<MAP, EPI, 16>(prm, s, padded_offsets, work, stream);
    case 32: return launch_ring<MAP, EPI, 32>(prm, s, padded_offsets, work, stream);
    case 56: return launch_ring<MAP, EPI, 56>(prm, s, padded_offsets, work, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fp8_supported(const GroupedShape& s) {
  return s.H % kDmaBN == 0 && s.I % (kDmaBN / 2) == 0 && fp8_kt_ok(s.H / kDmaBK) && fp8_kt_ok(s.I / kDmaBK) &&
         (uint64_t)s.T * s.H < (1ull << 32) && (uint64_t)s.max_rows * s.I < (1ull << 32) &&
         (uint64_t)2 * s.I * s.H < (1ull << 32) && list_grid_fits(s, kRingBM, kDmaBN);
}

size_t w13_ws_bytes(const GroupedShape& s, int32_t scale_mode) {
  if (scale_mode == 2 || scale_mode == 3) return work_bytes(s);
  if (scale_mode == 1) return use_ring(s, 1) ? work_bytes(s) : 256;
  return round256(sizeof(float) * (size_t)(s.max_rows * s.I)) +
         round256(sizeof(float) * (size_t)(s.max_rows * w13_n_tiles(s, scale_mode))) + work_bytes(s);
}

size_t w2_ws_bytes(const GroupedShape& s, int32_t scale_mode) {
  (void)scale_mode;
  return round256(sizeof(float) * (size_t)(s.max_rows * s.H)) + round256(sizeof(int32_t) * (size_t)(s.T * s.k)) +
         work_bytes(s);
}

int32_t engine_of(const GroupedShape& s, int32_t scale_mode) {
  if (scale_mode == 2 || scale_mode == 3) {
    if (scale_mode == 3 && s.T * s.k < kStreamMaxAvgRows * s.E) return kEngineStream;
    return kEngineRing;
  }
  if (scale_mode == 1) return use_ring(s, 1) ? kEngineRing : kEngineStaged;
  return use_ring(s, 0) ? kEngineRing : use_dma(s) ? kEngineDma : kEngineStaged;
}

size_t i32_ws_bytes(const GroupedShape& s) { return work_bytes(s); }

// The raw accumulators through the engine, tile shape, gate/up pairing and work order of the
// channel-wise GEMM of the same shape (gather = 1: the first GEMM, gather = 0: the second), with
// an epilogue that stores the int32 sums instead of scaling them.
hipError_t gemm_i32(const GroupedShape& s, int32_t gather, const int8_t* a, const int8_t* w, const int32_t* sorted,
                    const int32_t* padded_offsets, const int32_t* tile_expert, const int32_t* num_tiles, int32_t* out,
                    void* ws, hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  Params prm{};
  prm.a = a;
  prm.gather = gather;
  prm.w = w;
  prm.N = gather ? 2 * s.I : s.H;
  prm.K = gather ? s.H : s.I;
  prm.sorted = sorted;
  prm.tile_expert = tile_expert;
  prm.num_tiles = num_tiles;
  prm.P = s.T * s.k;
  prm.k = s.k;
  prm.block_m = s.block_m;
  prm.I = s.I;
  prm.out_i32 = out;
  int32_t* work = static_cast<int32_t*>(ws);
  const int32_t engine = engine_of(s, 0);
  if (gather) {
    if (engine == kEngineRing)
      return launch_ring<BMap::Split, Epi::I32, kRingH / kDmaBK>(prm, s, padded_offsets, work, stream);
    if (engine == kEngineDma) return launch_dma<BMap::Split, Epi::I32>(prm, s, padded_offsets, work, stream);
    return launch_bm<BMap::Split, Epi::I32, kBNStaged>(prm, s.max_rows, stream);
  }
  if (engine == kEngineRing)
    return launch_ring<BMap::Plain, Epi::I32, kRingI / kDmaBK>(prm, s, padded_offsets, work, stream);
  if (engine == kEngineDma) return launch_dma<BMap::Plain, Epi::I32>(prm, s, padded_offsets, work, stream);
  return launch_bm<BMap::Plain, Epi::I32, kBNStaged>(prm, s.max_rows, stream);
}

hipError_t w13_silu(const GroupedShape& s, int32_t scale_mode, const int8_t* a_q, const float* a_s,
                    const int8_t* w13, const float* w13_s, const int32_t* sorted, const int32_t* padded_offsets,
                    const int32_t* tile_expert, const int32_t* num_tiles, int8_t* h_q, float* h_s, void* ws,
                    hipStream_t stream) {
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
  if (scale_mode == 2)
    return launch_ring_kt<BMap::Split, Epi::W13Fp8>(prm, s, padded_offsets, static_cast<int32_t*>(ws), stream);
  if (scale_mode == 3)
    return launch_ring_kt<BMap::Split, Epi::W13W4>(prm, s, padded_offsets, static_cast<int32_t*>(ws), stream);
  if (scale_mode == 1) {
    if (use_ring(s, 1))
      return launch_ring<BMap::Split, Epi::W13Block, kRingH / kDmaBK>(prm, s, padded_offsets,
                                                                      static_cast<int32_t*>(ws), stream);
    return launch_bm<BMap::Split, Epi::W13Block, kBNBlock13>(prm, s.max_rows, stream);
  }
  char* base = static_cast<char*>(ws);
  const int64_t n_tiles = w13_n_tiles(s, scale_mode);
  float* hf = reinterpret_cast<float*>(base);
  float* part = reinterpret_cast<float*>(base + round256(sizeof(float) * (size_t)(s.max_rows * s.I)));
  int32_t* work = reinterpret_cast<int32_t*>(base + round256(sizeof(float) * (size_t)(s.max_rows * s.I)) +
                                             round256(sizeof(float) * (size_t)(s.max_rows * n_tiles)));
  prm.out_f32 = hf;
  prm.part_amax = part;
  hipError_t err = use_ring(s, 0)
                       ? launch_ring<BMap::Split, Epi::W13Channel, kRingH / kDmaBK>(prm, s, padded_offsets, work, stream)
                   : use_dma(s) ? launch_dma<BMap::Split, Epi::W13Channel>(prm, s, padded_offsets, work, stream)
                                : launch_bm<BMap::Split, Epi::W13Channel, kBNStaged>(prm, s.max_rows, stream);
  if (err != hipSuccess) return err;
  const int64_t blocks = std::min((s.max_rows + kThreads / kWave - 1) / (kThreads / kWave), kMaxGridBlocks);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(requant_rows_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, hf, part, sorted,
                     num_tiles, s.block_m, s.T * s.k, s.I, n_tiles, h_q, h_s);
  return hipGetLastError();
}

hipError_t w2_combine(const GroupedShape& s, int32_t scale_mode, const int8_t* h_q, const float* h_s,
                      const int8_t* w2, const float* w2_s, const int32_t* sorted, const int32_t* padded_offsets,
                      const int32_t* tile_expert, const int32_t* num_tiles, const float* topk_w, float* out,
                      void* ws, hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  const int64_t P = s.T * s.k;
  char* base = static_cast<char*>(ws);
  float* y = reinterpret_cast<float*>(base);
  int32_t* pair_row = reinterpret_cast<int32_t*>(base + round256(sizeof(float) * (size_t)(s.max_rows * s.H)));
  int32_t* work = reinterpret_cast<int32_t*>(base + round256(sizeof(float) * (size_t)(s.max_rows * s.H)) +
                                             round256(sizeof(int32_t) * (size_t)P));
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
  prm.pair_row = pair_row;
  hipError_t err;
  if (scale_mode == 2)
    err = launch_ring_kt<BMap::Plain, Epi::W2Fp8>(prm, s, padded_offsets, work, stream);
  else if (scale_mode == 3)
    err = launch_ring_kt<BMap::Plain, Epi::W2W4>(prm, s, padded_offsets, work, stream);
  else if (scale_mode == 1)
    err = use_ring(s, 1) ? launch_ring<BMap::Plain, Epi::W2Block, kRingI / kDmaBK>(prm, s, padded_offsets, work, stream)
                         : launch_bm<BMap::Plain, Epi::W2Block, kBNStaged>(prm, s.max_rows, stream);
  else if (use_ring(s, 0))
    err = launch_ring<BMap::Plain, Epi::W2Channel, kRingI / kDmaBK>(prm, s, padded_offsets, work, stream);
  else if (use_dma(s))
    err = launch_dma<BMap::Plain, Epi::W2Channel>(prm, s, padded_offsets, work, stream);
  else
    err = launch_bm<BMap::Plain, Epi::W2Channel, kBNStaged>(prm, s.max_rows, stream);
  if (err != hipSuccess) return err;
  const int64_t col_blocks = (s.H / 4 + kThreads * kCombineVec - 1) / (kThreads * kCombineVec);
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)std::min(s.T, kMaxGridBlocks), (uint32_t)col_blocks), dim3(kThreads),
                     0, stream, y, pair_row, sorted, num_tiles, s.block_m, topk_w, s.T, s.k, s.H, out);
  return hipGetLastError();
}

// Dense W8A8 linear: the DMA engine on one weight matrix, rows in their own order.  When the
// (row tile, N-tile) items are fewer than the CUs (few rows), K is split into slices whose int32
// partial sums go to the workspace; a second pass adds them in slice order (exact: integers) and
// dequantizes once, so the result does not depend on the split.
__global__ __launch_bounds__(kThreads) void linear_reduce_kernel(const int32_t* __restrict__ part, int64_t ksplit,
                                                                 int64_t M, int64_t N, const float* __restrict__ a_s,
                                                                 const float* __restrict__ w_s,
                                                                 float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < M * N / 4; q += stride) {  // 4 outputs each
    const int64_t m = (4 * q) / N, n = (4 * q) % N;
    i32x4 acc = reinterpret_cast<const i32x4*>(part)[q];
    for (int64_t s = 1; s < ksplit; ++s) acc += reinterpret_cast<const i32x4*>(part + s * M * N)[q];
    const float as = a_s[m];
    float4 o;
    o.x = ((float)acc[0] * as) * w_s[n];
    o.y = ((float)acc[1] * as) * w_s[n + 1];
    o.z = ((float)acc[2] * as) * w_s[n + 2];
    o.w = ((float)acc[3] * as) * w_s[n + 3];
    reinterpret_cast<float4*>(out)[q] = o;
  }
}

static hipError_t linear_reduce(const int32_t* part, int64_t ksplit, int64_t M, int64_t N, const float* a_s,
                         const float* w_s, float* out, hipStream_t stream) {
  const int64_t blocks = std::min((M * N / 4 + kThreads - 1) / kThreads, kMaxGridBlocks);
  hipLaunchKernelGGL(linear_reduce_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, part, ksplit, M, N, a_s,
                     w_s, out);
  return hipGetLastError();
}

// Plan of a linear of this shape, for the MI355X's 256 CUs (a fixed count, so the workspace size is
// a function of the shape alone; the result does not depend on it).
//  - At most 128 rows and K a multiple of 2048: the ring engine's 128 x 256 tiles (three LDS stages,
//    two of them in flight, so a CU keeps twice the weight bytes of a two-stage tile in flight),
//    K split into 2048-byte slices (the 16-step K loop it is unrolled for).
//  - Else the DMA engine's tiles (320 x 256; 128 x 128 on 4 wavefronts, two per CU, for at most
//    128 rows) with K split only when the unsplit items leave CUs idle: the power of two s
//    minimising rounds / s, rounds = ceil(items * s / slots), every slice an even number of at least
//    8 K-steps; ties go to the smaller s (less int32 partial traffic).
constexpr int64_t kLinearCUs = 256;
constexpr int kLinSmallBM = 128, kLinSmallBN = 128, kLinSmallWM = 2, kLinSmallWN = 2;
constexpr int64_t kLinRingKT = kRingI / kDmaBK;  // 16 steps: 2048 K-bytes per slice
enum class LinEngine { Dma, DmaSmall, Ring };
struct LinearPlan {
  LinEngine engine;
  int64_t bm, ksplit;
};
LinearPlan linear_plan(int64_t M, int64_t N, int64_t K) {
  if (M <= kRingBM && N % kDmaBN == 0 && K % (kLinRingKT * kDmaBK) == 0)
    return {LinEngine::Ring, kRingBM, K / (kLinRingKT * kDmaBK)};
  const bool small = M <= kLinSmallBM && N % kLinSmallBN == 0;
  const int64_t slots = small ? 2 * kLinearCUs : kLinearCUs;
  const int64_t items = small ? N / kLinSmallBN : (M + kDmaBM - 1) / kDmaBM * (N / kDmaBN);
  const int64_t steps = K / kDmaBK;
  LinearPlan plan{small ? LinEngine::DmaSmall : LinEngine::Dma, small ? kLinSmallBM : kDmaBM, 1};
  if (items >= slots) return plan;
  double best_cost = (double)((items + slots - 1) / slots);
  for (int64_t s = 2; steps % (2 * s) == 0 && steps / s >= 8; s *= 2) {
    const double cost = (double)((items * s + slots - 1) / slots) / (double)s;
    if (cost < best_cost) {
      plan.ksplit = s;
      best_cost = cost;
    }
  }
  return plan;
}

// The int32 partial sums of a split K (at least 256 bytes, so that 0 stays the answer for an
// unsupported shape); the row tiles need no list (the kernels derive them from M).
size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const LinearPlan plan = linear_plan(M, N, K);
  return plan.ksplit > 1 ? round256(sizeof(int32_t) * (size_t)(plan.ksplit * M * N)) : 256;
}

bool linear_supported(int64_t M, int64_t N, int64_t K) {
  if (K % 256 != 0 || N % kDmaBN != 0 || (uint64_t)M * K >= (1ull << 32) || (uint64_t)N * K >= (1ull << 32))
    return false;
  const LinearPlan plan = linear_plan(M, N, K);
  const int64_t bn = plan.engine == LinEngine::DmaSmall ? kLinSmallBN : kDmaBN;
  return (M + plan.bm - 1) / plan.bm * (N / bn) * plan.ksplit <= kMaxGridBlocks;  // one grid of items
}

hipError_t linear(const int8_t* a_q, const float* a_s, const int8_t* w, const float* w_s, int64_t M, int64_t N,
                  int64_t K, float* out, void* ws, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const LinearPlan plan = linear_plan(M, N, K);
  const int64_t ksplit = plan.ksplit;
  Params prm{};
  prm.a = a_q;
  prm.gather = 0;
  prm.w = w;
  prm.N = N;
  prm.K = K;
  prm.sorted = nullptr;
  prm.P = M;
  prm.k = 1;
  prm.a_s = a_s;
  prm.w_s = w_s;
  prm.out_f32 = out;
  const bool small = plan.engine == LinEngine::DmaSmall;
  const int64_t bm = plan.bm;
  prm.n_tiles = N / (small ? kLinSmallBN : kDmaBN);
  prm.ksplit = ksplit;
  const int32_t* work = nullptr;  // row tiles of bm rows, derived in the kernels
  const int64_t tiles = (M + bm - 1) / bm;
  const int64_t grid = (tiles * prm.n_tiles * ksplit + 7) / 8 * 8;
  if (grid > kMaxGridBlocks) return hipErrorInvalidConfiguration;  // linear_supported keeps it below
  int32_t* part = static_cast<int32_t*>(ws);
  if (plan.engine == LinEngine::Ring) {
    constexpr int WM = 2, WN = 4;
    if (ksplit == 1) {
      hipLaunchKernelGGL((grouped_gemm_ring_kernel<kRingBM, kDmaBN, WM, WN, kLinRingKT, BMap::Plain, Epi::W2Channel>),
                         dim3((uint32_t)grid), dim3(WM * WN * kWave), 0, stream, prm, (const int32_t*)work);
      return hipGetLastError();
    }
    prm.out_i32 = part;
    hipLaunchKernelGGL((grouped_gemm_ring_kernel<kRingBM, kDmaBN, WM, WN, kLinRingKT, BMap::Plain, Epi::I32>),
                       dim3((uint32_t)grid), dim3(WM * WN * kWave), 0, stream, prm, (const int32_t*)work);
    return linear_reduce(part, ksplit, M, N, a_s, w_s, out, stream);
  }
  if (small) {
    constexpr int NT = kLinSmallWM * kLinSmallWN * kWave;
    if (ksplit == 1) {
      hipLaunchKernelGGL((grouped_gemm_dma_kernel<kLinSmallBM, kLinSmallBN, kLinSmallWM, kLinSmallWN, BMap::Plain,
                                                  Epi::W2Channel>),
                         dim3((uint32_t)grid), dim3(NT), 0, stream, prm, (const int32_t*)work);
      return hipGetLastError();
    }
    prm.out_i32 = part;
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<kLinSmallBM, kLinSmallBN, kLinSmallWM, kLinSmallWN, BMap::Plain,
                                                Epi::I32>),
                       dim3((uint32_t)grid), dim3(NT), 0, stream, prm, (const int32_t*)work);
    return linear_reduce(part, ksplit, M, N, a_s, w_s, out, stream);
  }
  if (ksplit == 1) {
    hipLaunchKernelGGL((grouped_gemm_dma_kernel<kDmaBM, kDmaBN, kDmaWM, kDmaWN, BMap::Plain, Epi::W2Channel>),
                       dim3((uint32_t)grid), dim3(kDmaWM * kDmaWN * kWave), 0, stream, prm, (const int32_t*)work);
    return hipGetLastError();
  }
  prm.out_i32 = part;
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<kDmaBM, kDmaBN, kDmaWM, kDmaWN, BMap::Plain, Epi::I32>),
                     dim3((uint32_t)grid), dim3(kDmaWM * kDmaWN * kWave), 0, stream, prm, (const int32_t*)work);
  return linear_reduce(part, ksplit, M, N, a_s, w_s, out, stream);
}

}  // namespace w8a8
