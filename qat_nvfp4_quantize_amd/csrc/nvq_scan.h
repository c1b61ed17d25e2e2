// Workgroup-wide integer prefix sum for the small tables of the GEMM entry
// points (tile tables over at most 1024 experts).
#pragma once

#include <hip/hip_runtime.h>

namespace nvq {

// Inclusive prefix sum of v over the workgroup, in thread order.  blockDim.x
// is a multiple of 64 and at most 1024; every thread of the workgroup calls
// it; s_wave holds 16 ints of LDS.  Lane scans with __shfl_up, then wave 0
// scans the wave totals.
__device__ __forceinline__ int block_inclusive_scan(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nwaves ? s_wave[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int u = __shfl_up(w, off, 64);
      if (lane >= off) w += u;
    }
    if (lane < nwaves) s_wave[lane] = w;
  }
  __syncthreads();
  return wave > 0 ? v + s_wave[wave - 1] : v;
}

// Tile table of a row-tiled grouped GEMM: expert e's rows [off[e], off[e + 1])
// split into bm-row tiles, tile i = (expert, first row), experts in order.
// s_incl[e] holds the inclusive prefix of the experts' tile counts (set by
// the caller before calling).  Tile i is written by thread i % blockDim.x
// (its expert found by a binary search over the prefixes), so consecutive
// tiles go out together however the rows are spread over the experts.
__device__ __forceinline__ void write_tiles_from_prefix(const int32_t* __restrict__ off, int E, int bm,
                                                        const int* s_incl, int32_t* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles, int max_tiles) {
  __syncthreads();
  const int total = min(s_incl[E - 1], max_tiles);
  if (threadIdx.x == 0) *ntiles = total;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    int lo = 0, hi = E - 1;  // the first expert whose inclusive prefix exceeds i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_incl[mid] > i)
        hi = mid;
      else
        lo = mid + 1;
    }
    const int base = lo > 0 ? s_incl[lo - 1] : 0;
    tiles[2 * i] = lo;
    tiles[2 * i + 1] = off[lo] + (i - base) * bm;
  }
}

// The whole tile table from one workgroup of blockDim.x threads (a multiple
// of 64, at most 1024), E <= 4 blockDim.x: thread t owns experts 4t .. 4t + 3.
// s_wave: 16 ints of LDS; s_incl: E ints.
__device__ __forceinline__ void build_tile_table(const int32_t* __restrict__ off, int E, int bm,
                                                 int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                 int max_tiles, int* s_wave, int* s_incl) {
  const int t = threadIdx.x;
  int nt[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    nt[q] = e < E ? (off[e + 1] - off[e] + bm - 1) / bm : 0;
    sum += nt[q];
  }
  int run = block_inclusive_scan(sum, s_wave) - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    run += nt[q];
    if (e < E) s_incl[e] = run;
  }
  write_tiles_from_prefix(off, E, bm, s_incl, tiles, ntiles, max_tiles);
}

}  // namespace nvq
