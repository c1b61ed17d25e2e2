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

}  // namespace nvq
