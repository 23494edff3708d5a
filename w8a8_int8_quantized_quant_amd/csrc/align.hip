// align.hip -- stable grouping of (token, slot) pairs by expert (gfx950).
//
// Per-expert counts, expert offsets = zero-padded cumulative sum of the counts
// (SGLang PR #8273, review of the m_indices argument), the expert-sorted pair
// list with each expert's segment padded to a multiple of block_m, and the
// expert of every block_m-row tile (the "expert id per row" meaning of
// m_indices in the same review, at tile granularity).
//
// Deterministic, no atomics: pairs are cut into chunks of 1024; inside a chunk
// each wavefront ranks its pairs with ballots on the expert-id bits (the lanes
// holding the same expert form a mask; the rank is the popcount below the
// lane), wave histograms give the rank inside the chunk, one scan over chunks
// gives each chunk's base per expert, and a scatter writes every pair once.
// Up to kAlignSmallMax pairs (decode batches) one 1024-thread workgroup does all
// of it in a single launch, with the same ranks.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRounds = (int)(kAlignChunk / kThreads);  // 4 rounds of 64 pairs per wave
constexpr int kMaxE = 1024;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int64_t pair_of(int64_t chunk, int w, int round) {
  return chunk * kAlignChunk + (int64_t)w * (kWave * kRounds) + round * kWave + lane_id();
}

__global__ __launch_bounds__(kThreads) void align_hist_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                              int nbits, int32_t* __restrict__ hist,
                                                              int32_t* __restrict__ rank) {
  __shared__ int wh[kWaves][kMaxE];
  const int w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x;
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wh[i / E][i % E] = 0;
  __syncthreads();
  int my_rank[kRounds];
  int my_e[kRounds];
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    const int64_t p = pair_of(chunk, w, round);
    const int e = p < P ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t below = peers & lanemask_lt();
    int base = 0;
    if (valid) base = wh[w][e];
    my_rank[round] = base + __popcll(below);
    my_e[round] = valid ? e : -1;
    __syncthreads();
    if (valid && below == 0) wh[w][e] = base + __popcll(peers);
    __syncthreads();
  }
  // wave-exclusive bases per expert and the chunk total
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = wh[ww][e];
      wh[ww][e] = run;
      run += c;
    }
    hist[chunk * E + e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    if (my_e[round] >= 0) rank[pair_of(chunk, w, round)] = wh[w][my_e[round]] + my_rank[round];
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ int block_exclusive_scan(int v, int* wsum, int& total) {
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
  for (int i = 0; i < kScanThreads / kWave; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  __syncthreads();
  return before + x - v;
}

// Offsets from the per-expert counts (thread e of 1024 holds expert e's count): counts, offsets,
// padded offsets (also into po, E + 1 entries of LDS), the sentinel P in each segment's padding,
// num_tiles and the expert of every block_m-row tile.  Ends with po complete for every thread.
__device__ void write_offsets(int cnt, int E, int block_m, int32_t P, int* wsum, int* po, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ padded_offsets,
                              int32_t* __restrict__ sorted, int32_t* __restrict__ tile_expert,
                              int32_t* __restrict__ num_tiles) {
  const int e = threadIdx.x;
  const int pc = (cnt + block_m - 1) / block_m * block_m;
  int total_cnt, total_pc;
  const int off = block_exclusive_scan(cnt, wsum, total_cnt);
  const int poff = block_exclusive_scan(pc, wsum, total_pc);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    padded_offsets[e] = poff;
    po[e] = poff;
    for (int r = poff + cnt; r < poff + pc; ++r) sorted[r] = P;
  }
  if (e == 0) {
    offsets[E] = total_cnt;
    padded_offsets[E] = total_pc;
    po[E] = total_pc;
    num_tiles[0] = total_pc / block_m;
  }
  __syncthreads();
  const int ntiles = total_pc / block_m;
  for (int i = threadIdx.x; i < ntiles; i += kScanThreads) {
    const int row = i * block_m;
    int lo = 0, hi = E - 1;  // largest expert with po[expert] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (po[mid] <= row)
        lo = mid;
      else
        hi = mid - 1;
    }
    tile_expert[i] = lo;
  }
}

__global__ __launch_bounds__(kScanThreads) void align_scan_kernel(int32_t* __restrict__ hist, int64_t nchunks, int E,
                                                                  int block_m, int32_t P, int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ padded_offsets,
                                                                  int32_t* __restrict__ sorted,
                                                                  int32_t* __restrict__ tile_expert,
                                                                  int32_t* __restrict__ num_tiles) {
  __shared__ int wsum[kScanThreads / kWave];
  __shared__ int po[kMaxE + 1];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    int64_t c = 0;
    for (; c + 8 <= nchunks; c += 8) {
      int h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = hist[(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hist[(c + i) * E + e] = cnt;
        cnt += h[i];
      }
    }
    for (; c < nchunks; ++c) {
      const int h = hist[c * E + e];
      hist[c * E + e] = cnt;
      cnt += h;
    }
  }
  write_offsets(cnt, E, block_m, P, wsum, po, counts, offsets, padded_offsets, sorted, tile_expert, num_tiles);
}

// The whole align in one workgroup of kScanThreads threads, for P <= kAlignSmallMax: pair
// p = round * kScanThreads + thread.  A pair's rank in its expert's segment counts that expert's
// pairs in earlier rounds, in earlier wavefronts of its round, and on lower lanes of its wavefront
// (the ballot ranking of the chunked kernels), i.e. the pairs before it.
constexpr int kSmallWaves = kScanThreads / kWave;
constexpr int kSmallRounds = (int)(kAlignSmallMax / kScanThreads);
__global__ __launch_bounds__(kScanThreads) void align_small_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                                   int nbits, int block_m,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ padded_offsets,
                                                                   int32_t* __restrict__ sorted,
                                                                   int32_t* __restrict__ tile_expert,
                                                                   int32_t* __restrict__ num_tiles) {
  __shared__ int wh[kSmallWaves][kMaxE];  // per-wavefront counts of the round, then their bases
  __shared__ int seen[kMaxE];             // pairs of each expert in the rounds before
  __shared__ int wsum[kSmallWaves];
  __shared__ int po[kMaxE + 1];
  const int w = threadIdx.x / kWave;
  for (int e = threadIdx.x; e < E; e += kScanThreads) seen[e] = 0;
  int my_rank[kSmallRounds], my_e[kSmallRounds];
#pragma unroll
  for (int round = 0; round < kSmallRounds; ++round) {
    my_e[round] = -1;
    my_rank[round] = 0;
    if ((int64_t)round * kScanThreads >= P) continue;  // uniform
    for (int i = threadIdx.x; i < kSmallWaves * E; i += kScanThreads) wh[i / E][i % E] = 0;
    __syncthreads();
    const int64_t p = (int64_t)round * kScanThreads + threadIdx.x;
    const int e = p < P ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t below = peers & lanemask_lt();
    if (valid && below == 0) wh[w][e] = __popcll(peers);  // one writer per (wavefront, expert)
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kScanThreads) {
      int run = seen[x];
#pragma unroll
      for (int ww = 0; ww < kSmallWaves; ++ww) {
        const int c = wh[ww][x];
        wh[ww][x] = run;
        run += c;
      }
      seen[x] = run;
    }
    __syncthreads();
    if (valid) {
      my_e[round] = e;
      my_rank[round] = wh[w][e] + __popcll(below);
    }
    __syncthreads();  // the next round clears wh
  }
  const int cnt = (int)threadIdx.x < E ? seen[threadIdx.x] : 0;
  write_offsets(cnt, E, block_m, (int32_t)P, wsum, po, counts, offsets, padded_offsets, sorted, tile_expert,
                num_tiles);
#pragma unroll
  for (int round = 0; round < kSmallRounds; ++round)
    if (my_e[round] >= 0) sorted[po[my_e[round]] + my_rank[round]] = (int32_t)((int64_t)round * kScanThreads + threadIdx.x);
}

__global__ __launch_bounds__(kThreads) void align_scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                                 const int32_t* __restrict__ hist,
                                                                 const int32_t* __restrict__ rank,
                                                                 const int32_t* __restrict__ padded_offsets,
                                                                 int32_t* __restrict__ sorted) {
  const int w = threadIdx.x / kWave;
  const int64_t chunk = blockIdx.x;
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    const int64_t p = pair_of(chunk, w, round);
    if (p >= P) continue;
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    sorted[padded_offsets[e] + hist[chunk * E + e] + rank[p]] = (int32_t)p;
  }
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// Scratch of the allocation-free align entry point: the histogram and rank buffers live in this
// array instead of a caller's workspace.  Each device holds its own copy (at its own address) for
// the life of the process.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies get the address resolved per device below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of this device's `scratch`, resolved once per device (with that device current)
// and kept; later calls reuse it.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t align_ws_bytes(int64_t P, int64_t E) {
  const int64_t nchunks = (P + kAlignChunk - 1) / kAlignChunk;
  return round256(sizeof(int32_t) * (size_t)(nchunks * E)) + round256(sizeof(int32_t) * (size_t)P);
}

hipError_t align_by_expert(const int32_t* ids, int64_t P, int64_t E, int64_t block_m, int32_t* counts,
                           int32_t* offsets, int32_t* padded_offsets, int32_t* sorted, int32_t* tile_expert,
                           int32_t* num_tiles, int64_t max_tiles, void* ws, hipStream_t stream) {
  (void)max_tiles;
  const int64_t nchunks = (P + kAlignChunk - 1) / kAlignChunk;
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + round256(sizeof(int32_t) * nchunks * E));
  int nbits = 0;
  while ((1ll << nbits) < E) ++nbits;
  if (P <= kAlignSmallMax) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kScanThreads), 0, stream, ids, P, (int)E, nbits, (int)block_m,
                       counts, offsets, padded_offsets, sorted, tile_expert, num_tiles);
    return hipGetLastError();
  }
  if (nchunks > 0) {
    hipLaunchKernelGGL(align_hist_kernel, dim3((uint32_t)nchunks), dim3(kThreads), 0, stream, ids, P, (int)E,
                       nbits, hist, rank);
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist, nchunks, (int)E,
                     (int)block_m, (int32_t)P, counts, offsets, padded_offsets, sorted, tile_expert, num_tiles);
  if (nchunks > 0) {
    hipLaunchKernelGGL(align_scatter_kernel, dim3((uint32_t)nchunks), dim3(kThreads), 0, stream, ids, P, (int)E,
                       hist, rank, padded_offsets, sorted);
  }
  return hipGetLastError();
}

}  // namespace w8a8
