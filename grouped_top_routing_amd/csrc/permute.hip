// Token permutation and per-expert histogram on gfx950: a stable counting sort
// of the T*topk (token, slot) pairs by expert, with no atomics.
//
// The block runs only the chosen experts on each token ("Welcome Beam: a 501B
// open model you can own, customize, and scale", section "Mixture of Experts":
// only 8 experts run per token), so the pairs are regrouped expert-major before
// the expert GEMMs and scattered back after them.
//
// Up to 4096 pairs: one workgroup does all of it (permute_small_kernel).
// Larger batches: three kernels over fixed chunks of kChunk pairs (one
// workgroup per chunk, each wave owning a contiguous quarter):
//   hist     per-wave histograms in LDS; lanes holding the same expert are found
//            with eight ballots (one per id bit), and only the lowest such lane
//            adds the group's size, so no two lanes ever update one counter;
//            the chunk's 256-bin histogram goes to the workspace.
//   scan     one workgroup: per expert, the running total over chunks (chunk
//            base), then an LDS exclusive scan over experts (offsets).
//   scatter  recomputes the wave histograms, turns them into per-wave bases,
//            then walks the pairs in order: rank = base + (matching lanes
//            below this one); the group's lowest lane advances the base.
// Every pair's destination depends only on the pairs before it, so the result
// equals the sequential stable sort and is bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kBins = 256;

// Lanes of this wave whose id equals mine (valid lanes only), via 8 ballots.
__device__ __forceinline__ uint64_t match_peers(int e, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Per-wave histogram of this wave's quarter of the chunk into hist[wave][*].
__device__ __forceinline__ void wave_histogram(const int32_t* __restrict__ ids, int64_t n,
                                               int64_t begin, int64_t end, int E, int lane,
                                               int* __restrict__ hist_row) {
  for (int64_t i0 = begin; i0 < end; i0 += 64) {
    const int64_t i = i0 + lane;
    int e = -1;
    if (i < end && i < n) e = ids[i];
    const bool valid = e >= 0 && e < E;
    const uint64_t peers = match_peers(valid ? e : 0, valid);
    if (valid && (peers & lanemask_lt(lane)) == 0) hist_row[e] += __popcll(peers);
  }
}

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids,
                                                           int64_t n, int E,
                                                           int32_t* __restrict__ chunk_hist) {
  __shared__ int hist[4][kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * kBins; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t q = kChunk / 4;
  wave_histogram(ids, n, c0 + wave * q, c0 + (wave + 1) * q, E, lane, hist[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    chunk_hist[(size_t)blockIdx.x * E + e] = hist[0][e] + hist[1][e] + hist[2][e] + hist[3][e];
}

__global__ __launch_bounds__(256) void permute_scan_kernel(int32_t* __restrict__ chunk_hist,
                                                           int nchunks, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int sc[kBins];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    // running total over chunks, 32 chunks' loads in flight at a time
    for (int c0 = 0; c0 < nchunks; c0 += 32) {
      int v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = c0 + j < nchunks ? chunk_hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (c0 + j < nchunks) chunk_hist[(size_t)(c0 + j) * E + e] = total;
        total += v[j];
      }
    }
  }
  sc[e] = e < E ? total : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 bins
  for (int off = 1; off < kBins; off <<= 1) {
    const int v = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int excl = sc[e] - (e < E ? total : 0);
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    for (int c0 = 0; c0 < nchunks; c0 += 32) {
      int v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = c0 + j < nchunks ? chunk_hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (c0 + j < nchunks) chunk_hist[(size_t)(c0 + j) * E + e] = v[j] + excl;
    }
  }
  if (e == E - 1) offsets[E] = excl + total;
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, const int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ perm_dst) {
  __shared__ int hist[4][kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * kBins; i += 256) (&hist[0][0])[i] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t q = kChunk / 4;
  const int64_t begin = c0 + wave * q, end = c0 + (wave + 1) * q;
  wave_histogram(ids, n, begin, end, E, lane, hist[wave]);
  __syncthreads();
  // hist[w][e] <- first destination row of expert e for wave w
  for (int e = tid; e < E; e += 256) {
    int run = chunk_base[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = hist[w][e];
      hist[w][e] = run;
      run += v;
    }
  }
  __syncthreads();
  int* base = hist[wave];
  for (int64_t i0 = begin; i0 < end; i0 += 64) {
    const int64_t i = i0 + lane;
    const bool in = i < end && i < n;
    int e = -1;
    if (in) e = ids[i];
    const bool valid = e >= 0 && e < E;
    const uint64_t peers = match_peers(valid ? e : 0, valid);
    if (valid) {
      const uint64_t below = peers & lanemask_lt(lane);
      const int r = BEAM_CLAMP(base[e] + __popcll(below), 0, n - 1, kCheckPermuteRow);
      perm_dst[i] = r;
      perm_src[r] = (int32_t)i;
      if (below == 0) base[e] += __popcll(peers);
    } else if (in) {
      perm_dst[i] = -1;
    }
  }
}

// Small batches (up to kSmallPairs pairs, e.g. decode): the same stable sort
// in one workgroup of 16 waves, one launch instead of three.  Wave w owns the
// contiguous pairs [w q, (w + 1) q) (q a multiple of 64) and holds their ids
// in registers; its histogram, the scan over experts and the per-wave bases
// stay in LDS, so the ranks are those of the chunked kernels.
constexpr int kSmallWaves = 16;
constexpr int kSmallPerLane = 4;
constexpr int kSmallPairs = kSmallWaves * 64 * kSmallPerLane;

__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm_src,
                                                             int32_t* __restrict__ perm_dst) {
  __shared__ int hist[kSmallWaves][kBins];
  __shared__ int sc[kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kSmallWaves * kBins; i += 1024) (&hist[0][0])[i] = 0;
  // pairs per wave, a whole number of 64-pair steps (at most kSmallPerLane)
  const int q = (n + kSmallWaves * 64 - 1) / (kSmallWaves * 64) * 64;
  const int begin = wave * q, end = min(begin + q, n);
  int e[kSmallPerLane];
#pragma unroll
  for (int j = 0; j < kSmallPerLane; ++j) {
    const int i = begin + 64 * j + lane;
    e[j] = 64 * j < q && i < end ? ids[i] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSmallPerLane; ++j) {
    if (64 * j < q) {  // wave-uniform
      const bool valid = e[j] >= 0 && e[j] < E;
      const uint64_t peers = match_peers(valid ? e[j] : 0, valid);
      if (valid && (peers & lanemask_lt(lane)) == 0) hist[wave][e[j]] += __popcll(peers);
    }
  }
  __syncthreads();
  // totals per expert, exclusive scan over experts, per-wave first rows
  int total = 0;
  if (tid < E)
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) total += hist[w][tid];
  if (tid < kBins) sc[tid] = tid < E ? total : 0;
  __syncthreads();
  for (int off = 1; off < kBins; off <<= 1) {
    const int v = tid < kBins && tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    if (tid < kBins) sc[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = sc[tid] - total;
    counts[tid] = total;
    offsets[tid] = excl;
    if (tid == E - 1) offsets[E] = excl + total;
    int run = excl;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      const int v = hist[w][tid];
      hist[w][tid] = run;
      run += v;
    }
  }
  __syncthreads();
  int* base = hist[wave];
#pragma unroll
  for (int j = 0; j < kSmallPerLane; ++j) {
    if (64 * j < q) {  // wave-uniform
      const int i = begin + 64 * j + lane;
      const bool valid = e[j] >= 0 && e[j] < E;
      const uint64_t peers = match_peers(valid ? e[j] : 0, valid);
      if (valid) {
        const uint64_t below = peers & lanemask_lt(lane);
        const int r = BEAM_CLAMP(base[e[j]] + __popcll(below), 0, n - 1, kCheckPermuteRow);
        perm_dst[i] = r;
        perm_src[r] = i;
        if (below == 0) base[e[j]] += __popcll(peers);
      } else if (i < end) {
        perm_dst[i] = -1;
      }
    }
  }
}

BEAM_DEFINE_CHECK_READER(check_flags_permute)

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int32_t* counts, int32_t* offsets,
                          int32_t* perm_src, int32_t* perm_dst, int32_t* chunk_hist,
                          hipStream_t stream) {
  if (n > 0 && n <= kSmallPairs) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, stream, ids, (int)n, E,
                       counts, offsets, perm_src, perm_dst);
    return hipGetLastError();
  }
  const int nchunks = (int)((n + kChunk - 1) / kChunk);
  if (nchunks == 0) {
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, stream, chunk_hist, 0, E, counts,
                       offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nchunks), dim3(256), 0, stream, ids, n, E,
                     chunk_hist);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, stream, chunk_hist, nchunks, E,
                     counts, offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(256), 0, stream, ids, n, E,
                     chunk_hist, perm_src, perm_dst);
  return hipGetLastError();
}

}  // namespace beam
