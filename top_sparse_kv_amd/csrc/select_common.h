// Block-wide scan used by the select stage.
#pragma once

#include "skv_internal.h"

namespace skv {

// Block-wide exclusive prefix sum of one value per thread (blockDim.x <= 1024,
// a multiple of 64), in thread order.  `wsum` is LDS scratch of 16 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t s = wsum[w];
    if (w < wave) base += s;
    tot += s;
  }
  if (total) *total = tot;
  return base + incl - v;
}

}  // namespace skv
