// Second pass of split K: the fixed-order reduction of fp32 partials.
// Included by the host translation unit only (a non-template kernel).
#pragma once

#include "tile_common.hpp"

namespace gemmf16 {

// C[m][n] = fp16_rne( sum_{s=0}^{S-1} W[s][m][n] ), ascending s.  Each thread
// owns 4 consecutive n of one row; grid-stride over the M x ceil(N/4) quads.
__global__ __launch_bounds__(256) void splitk_reduce(const float* W, int S, int64_t M, int64_t N,
                                                     uint16_t* C, int64_t ldc, int c_vec) {
  const int64_t NQ = (N + 3) / 4;
  const int64_t total = M * NQ;
  const int64_t MN = M * N;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = q / NQ, n = (q - m * NQ) * 4;
    const float* p = W + m * N + n;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    if ((N & 3) == 0) {
      for (int s = 0; s < S; ++s) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + s * MN);
        s0 += v[0]; s1 += v[1]; s2 += v[2]; s3 += v[3];
      }
    } else {
      for (int s = 0; s < S; ++s) {
        const float* ps = p + s * MN;
        s0 += ps[0];
        if (n + 1 < N) s1 += ps[1];
        if (n + 2 < N) s2 += ps[2];
        if (n + 3 < N) s3 += ps[3];
      }
    }
    uint16_t* c = C + m * ldc + n;
    const _Float16 h[4] = {(_Float16)s0, (_Float16)s1, (_Float16)s2, (_Float16)s3};
    if (c_vec && n + 4 <= N) {
      *reinterpret_cast<f16x4*>(c) = f16x4{h[0], h[1], h[2], h[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) reinterpret_cast<_Float16*>(c)[e] = h[e];
    }
  }
}

}  // namespace gemmf16
