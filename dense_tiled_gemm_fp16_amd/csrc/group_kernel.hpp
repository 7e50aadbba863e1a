// Set-up pass of a grouped launch (host translation unit only).
#pragma once

#include "tile_common.hpp"

namespace gemmf16 {

// One workgroup of 1024 threads.  For g = 0..G:
//   off_out[g] = off_in[g] clamped to [0, M]
//   tiles[g]   = sum over h < g of ceil(rows_h / BM),
//                rows_h = max(0, off_out[h+1] - off_out[h])
// so tiles[G] is the number of row tiles of the whole launch and every row
// that a later kernel touches lies inside [0, M), whatever the offsets.
// Each thread sums a contiguous chunk of groups; the chunk sums are scanned
// in LDS (Hillis-Steele, fixed order) and each thread then writes its chunk.
__global__ __launch_bounds__(1024) void group_setup(const int64_t* off_in, int32_t G, int64_t M,
                                                    int32_t BM, int64_t* off_out, int64_t* tiles) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int chunk = (G + 1023) / 1024;
  const int g0 = t * chunk < G ? t * chunk : G;
  const int g1 = g0 + chunk < G ? g0 + chunk : G;
  auto clampm = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > M ? M : v); };
  int64_t sum = 0;
  for (int g = g0; g < g1; ++g) {
    const int64_t r0 = clampm(off_in[g]), r1 = clampm(off_in[g + 1]);
    sum += r1 > r0 ? (r1 - r0 + BM - 1) / BM : 0;
  }
  part[t] = sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int64_t v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = t > 0 ? part[t - 1] : 0;
  for (int g = g0; g < g1; ++g) {
    const int64_t r0 = clampm(off_in[g]), r1 = clampm(off_in[g + 1]);
    off_out[g] = r0;
    tiles[g] = run;
    run += r1 > r0 ? (r1 - r0 + BM - 1) / BM : 0;
  }
  if (t == 1023) {
    off_out[G] = clampm(off_in[G]);
    tiles[G] = part[1023];
  }
}

}  // namespace gemmf16
