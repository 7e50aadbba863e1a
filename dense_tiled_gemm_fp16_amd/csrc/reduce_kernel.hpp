// Second pass of split K: the fixed-order reduction of fp32 partials.
// Included by the host translation unit only (non-inline kernels).
#pragma once

#include "tile_common.hpp"

namespace gemmf16 {

// C[m][n] = rne( sum over s of W[s][m][n] ), s ascending from +0 (fp16 or
// bfloat16 output, by DT): the order is fixed, so results are
// bit-reproducible.  Two shapes of the same sum:
//   splitk_reduce_quad: a thread owns 4 consecutive n of one row and loads
//     16-byte vectors, eight K ranges at a time (large outputs);
//   splitk_reduce_elem: a thread owns one output and issues the loads of up
//     to 16 K ranges before adding them (small outputs, e.g. decode shapes,
//     where a second round trip or any cross-lane step would cost more than
//     the few bytes moved).
template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_quad(const float* W, int S, int64_t M, int64_t N,
                                                          uint16_t* C, int64_t ldc, int c_vec) {
  const int64_t NQ = (N + 3) / 4;
  const int64_t total = M * NQ;
  const int64_t MN = M * N;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += step) {
    const int64_t m = q / NQ, n = (q - m * NQ) * 4;
    const int nv = (N - n < 4) ? (int)(N - n) : 4;
    const float* p = W + m * N + n;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* ps = p + (int64_t)(s0 + j) * MN;
        if (s0 + j >= S) {
          v[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        } else if ((N & 3) == 0) {
          v[j] = *reinterpret_cast<const f32x4*>(ps);
        } else {
          v[j] = f32x4{ps[0], nv > 1 ? ps[1] : 0.0f, nv > 2 ? ps[2] : 0.0f, nv > 3 ? ps[3] : 0.0f};
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < S) {
          acc[0] += v[j][0];
          acc[1] += v[j][1];
          acc[2] += v[j][2];
          acc[3] += v[j][3];
        }
    }
    uint16_t* c = C + m * ldc + n;
    const uint16_t h[4] = {cvt_out<DT>(acc[0]), cvt_out<DT>(acc[1]), cvt_out<DT>(acc[2]),
                           cvt_out<DT>(acc[3])};
    if (c_vec && nv == 4) {
      *reinterpret_cast<u32x2*>(c) = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < nv) c[e] = h[e];
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_elem(const float* W, int S, int64_t M, int64_t N,
                                                          uint16_t* C, int64_t ldc, int c_vec) {
  (void)c_vec;
  const int64_t MN = M * N;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += step) {
    const float* p = W + e;
    float acc = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (s0 + j < S) ? p[(int64_t)(s0 + j) * MN] : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (s0 + j < S) acc += v[j];
    }
    const int64_t m = e / N, n = e - m * N;
    C[m * ldc + n] = cvt_out<DT>(acc);
  }
}

// Fix-up of a stream-K tail: tile i of the L split tiles (raster id
// sk_first + i) has S dense BM x BN fp32 partials at slots s * L + i of W;
// C = rne(sum over s, ascending).  One thread per 4 consecutive columns of a
// tile row; BN / 4 * BM / 256 workgroups per tile.
template <int DT>
__global__ __launch_bounds__(256) void sk_fixup(const float* W, int S, int64_t L, int64_t sk_first,
                                                int64_t GM, int64_t GN, int panel, int BM, int BN,
                                                int64_t M, int64_t N, uint16_t* C, int64_t ldc,
                                                int c_vec) {
  const int64_t per_tile = (int64_t)BM * BN / 4 / 256;
  const int64_t i = blockIdx.x / per_tile;
  const int64_t q = (blockIdx.x - i * per_tile) * 256 + threadIdx.x;
  const int64_t r = q / (BN / 4), c = (q - r * (BN / 4)) * 4;
  int64_t pm, pn;
  raster_tile(sk_first + i, GM, GN, panel, pm, pn);
  const int64_t m = pm * BM + r, n = pn * BN + c;
  if (m >= M || n >= N) return;
  const int64_t slot = (int64_t)BM * BN, stride = L * slot;
  const float* p = W + i * slot + r * BN + c;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = (s0 + j < S) ? *reinterpret_cast<const f32x4*>(p + (int64_t)(s0 + j) * stride)
                          : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        acc[0] += v[j][0];
        acc[1] += v[j][1];
        acc[2] += v[j][2];
        acc[3] += v[j][3];
      }
  }
  const int nv = (N - n < 4) ? (int)(N - n) : 4;
  uint16_t* o = C + m * ldc + n;
  const uint16_t h[4] = {cvt_out<DT>(acc[0]), cvt_out<DT>(acc[1]), cvt_out<DT>(acc[2]),
                         cvt_out<DT>(acc[3])};
  if (c_vec && nv == 4) {
    *reinterpret_cast<u32x2*>(o) = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < nv) o[e] = h[e];
  }
}

}  // namespace gemmf16
