// route.hip -- top-k expert routing, one wavefront per token (gfx950).
//
// The pages only name the routing output (topk_idx, SGLang PR #8273).  Rules:
// softmax top-k with renormalised weights, or the DeepSeek-V3 rule -- sigmoid
// scores, node-limited grouped selection (group score = sum of the group's two
// best scores, keep topk_group groups), top-k, weights normalised and scaled.
// Order is a strict total order: larger score first, equal scores to the
// lower index, for groups and for experts.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kMaxE = 1024;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One step of a 16-lane reduction: the better of this lane's pair and the pair DPP control CTRL
// brings from another lane of the same 16-lane row.
template <int CTRL>
__device__ __forceinline__ void row_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide best (value, index) pair; every lane returns the winner (the whole wavefront must be
// active).  Within each 16-lane row: partner lanes l^1, l^2 (quad permutes), then the mirrored lane
// in the 8-lane half and in the row, so every lane of a row holds the row's best; the four rows'
// bests are then read as scalars and compared in row order.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  row_step<0xB1>(v, i);   // quad_perm [1, 0, 3, 2]
  row_step<0x4E>(v, i);   // quad_perm [2, 3, 0, 1]
  row_step<0x141>(v, i);  // row_half_mirror
  row_step<0x140>(v, i);  // row_mirror
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (better(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
}

template <int NPL>
__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                         int score_fn, int n_group, int topk_group, int renorm,
                                                         float scaling, const float* __restrict__ bias,
                                                         int32_t* __restrict__ ids, float* __restrict__ weights) {
  // Sized for this instantiation's E <= 64 NPL (12 KB a block at E = 256, not 48 KB for the 1024-expert
  // maximum), so that large batches keep many blocks per CU.
  constexpr int EP = NPL * kWave;
  static_assert(EP <= kMaxE, "experts per wavefront");
  __shared__ float sh_x[kWavesPerBlock][EP];  // logits (softmax) or sigmoid scores
  __shared__ float sh_c[kWavesPerBlock][EP];  // selection scores (sigmoid + bias)
  __shared__ int sh_sel[kWavesPerBlock][EP];
  const int w = threadIdx.x / kWave, l = lane_id();
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + w;
  const bool active = t < T;
  const bool sig = score_fn == 1;

  float key[NPL];
  uint32_t ok = 0;  // bit i: value i of this lane is eligible
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l + kWave * i;
    key[i] = -INFINITY;
    if (active && e < E) {
      const float lg = logits[t * E + e];
      if (sig) {
        const float s = 1.0f / (1.0f + expf(-lg));
        const float c = bias ? s + bias[e] : s;
        sh_x[w][e] = s;
        sh_c[w][e] = c;
        key[i] = c;
      } else {
        sh_x[w][e] = lg;
        key[i] = lg;
      }
      ok |= 1u << i;
    }
  }
  __syncthreads();

  if (sig && n_group > 1) {
    const int gs = E / n_group;
    float gscore = -INFINITY;
    int gidx = 0x7fffffff;
    if (gs <= kWave && (kWave % gs) == 0) {
      // A group is gs consecutive lanes of one 64-expert slot: a butterfly over the group's lanes
      // leaves the group's largest and second-largest selection score in each of them (only the
      // sum of the two counts, so ties need no index), then lane g fetches group g's sum.
      float part[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        float m1 = ((ok >> i) & 1u) ? key[i] : -INFINITY, m2 = -INFINITY;
        for (int o = 1; o < gs; o <<= 1) {
          const float p1 = __shfl_xor(m1, o, kWave), p2 = __shfl_xor(m2, o, kWave);
          const float n2 = fmaxf(fminf(m1, p1), fmaxf(m2, p2));
          m1 = fmaxf(m1, p1);
          m2 = n2;
        }
        part[i] = gs >= 2 ? m1 + m2 : m1;
      }
      const int first = (l < n_group ? l : 0) * gs;  // group l's first expert
      float got = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float v = __shfl(part[i], first % kWave, kWave);
        if (i == first / kWave) got = v;
      }
      if (active && l < n_group) {
        gscore = got;
        gidx = l;
      }
    } else if (active && l < n_group) {
      const float* c = sh_c[w] + l * gs;
      int b1 = 0;
      for (int i = 1; i < gs; ++i)
        if (c[i] > c[b1]) b1 = i;
      if (gs >= 2) {
        int b2 = b1 == 0 ? 1 : 0;
        for (int i = 0; i < gs; ++i)
          if (i != b1 && c[i] > c[b2]) b2 = i;
        gscore = c[b1] + c[b2];
      } else {
        gscore = c[b1];
      }
      gidx = l;
    }
    uint64_t kept = 0;
    for (int j = 0; j < topk_group; ++j) {
      float v = gscore;
      int i = gidx;
      wave_argmax(v, i);
      if (i >= 0 && i < 64) kept |= 1ull << i;
      if (l == i) gscore = -INFINITY, gidx = 0x7fffffff;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = l + kWave * i;
      if (e < E && !((kept >> (e / gs)) & 1ull)) ok &= ~(1u << i);
    }
  }

  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (((ok >> i) & 1u) && key[i] > bv) {  // ascending e per lane: strict > keeps the lower index
        bv = key[i];
        bi = l + kWave * i;
      }
    wave_argmax(bv, bi);
    if (bi == 0x7fffffff) bi = 0;  // no candidate left (only with NaN scores): keep indices in range
    else if ((bi % kWave) == l) ok &= ~(1u << (bi / kWave));
    if (l == 0) sh_sel[w][j] = bi;
  }
  __syncthreads();
  if (!active) return;

  // Normaliser: sequential sum in slot order (or expert order for the full softmax).
  float m = 0.0f, sum = 0.0f;
  if (!sig) m = sh_x[w][sh_sel[w][0]];
  if (l == 0) {
    if (!sig && !renorm) {
      for (int e = 0; e < E; ++e) sum = sum + expf(sh_x[w][e] - m);
    } else {
      for (int j = 0; j < k; ++j) {
        const float x = sh_x[w][sh_sel[w][j]];
        sum = sum + (sig ? x : expf(x - m));
      }
    }
  }
  sum = __shfl(sum, 0, kWave);
  for (int j = l; j < k; j += kWave) {
    const int e = sh_sel[w][j];
    const float x = sh_x[w][e];
    float v;
    if (sig)
      v = renorm ? x / sum : x;
    else
      v = expf(x - m) / sum;
    ids[t * k + j] = e;
    weights[t * k + j] = v * scaling;
  }
}

}  // namespace

hipError_t topk_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t score_fn, int64_t n_group,
                      int64_t topk_group, int32_t renormalize, float routed_scaling, const float* bias,
                      int32_t* ids, float* weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int npl = (int)((E + kWave - 1) / kWave);
  // Tokens go in pieces of at most kMaxGridBlocks workgroups (each token is routed on its own).
  const int64_t step = kMaxGridBlocks * kWavesPerBlock;
  for (int64_t t0 = 0; t0 < T; t0 += step) {
    const int64_t n = std::min(T - t0, step);
    const dim3 grid((uint32_t)((n + kWavesPerBlock - 1) / kWavesPerBlock)), block(kThreads);
    const float* lg = logits + t0 * E;
    int32_t* id = ids + t0 * k;
    float* wt = weights + t0 * k;
#define W8A8_ROUTE(N)                                                                                           \
  hipLaunchKernelGGL(route_kernel<N>, grid, block, 0, stream, lg, n, (int)E, (int)k, (int)score_fn, (int)n_group, \
                     (int)topk_group, (int)renormalize, routed_scaling, bias, id, wt)
    if (npl <= 1)
      W8A8_ROUTE(1);
    else if (npl <= 2)
      W8A8_ROUTE(2);
    else if (npl <= 4)
      W8A8_ROUTE(4);
    else if (npl <= 8)
      W8A8_ROUTE(8);
    else
      W8A8_ROUTE(16);
#undef W8A8_ROUTE
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w8a8
