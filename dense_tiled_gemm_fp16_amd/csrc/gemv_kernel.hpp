// Decode-shaped product (M <= 4) with N-contiguous B (gfx950).
//
// With a handful of rows of A the whole of B is streamed once to serve them,
// so the product is bound by HBM bandwidth, not by matrix throughput (the
// tiling tutorial, section 04: at M = 1 the whole weight serves one row; the
// TileLang tutorial ch. 14, pitfall 1: pipelining a memory-bound GEMM only
// takes on-chip space).  The kernel therefore uses plain VALU FMAs and spends
// its effort on keeping 16-byte loads of B in flight.
//
// Work split: workgroup (nb, s) owns columns [256 nb, 256 nb + 256) and the
// K range [s KR, (s+1) KR).  Thread (rg, cg) of the 8 x 32 thread grid owns 8
// consecutive columns (one 16-byte vector of a B row) and, per pass, RPT
// consecutive rows k; it issues all RPT loads before any arithmetic and
// accumulates in fp32 in ascending k.  The rows of A for the K range are
// staged once per chunk in LDS and read back as broadcasts.  The 8 row groups
// are summed through LDS in ascending rg order.
//
// With one K range the workgroup writes C (rounded to nearest even).  With
// several it writes fp32 partials P[s][m][n]; the fixed-order reduction
// kernel sums them in a second launch, which stream order makes see them.
// There is deliberately no in-kernel "last workgroup sums" step: that needs
// a device-scope release per workgroup, which on gfx950 writes back the
// XCD's L2 and serialises across the workgroups of an XCD (measured at tens
// of microseconds per call, several times the cost of the data stream).
#pragma once

#include "tile_common.hpp"

namespace gemmf16 {

struct GemvArgs {
  const uint16_t* A;
  int64_t lda_m, lda_k;
  const uint16_t* B;
  int64_t ldb_k;       // B is N-contiguous (ldb_n == 1), 16-byte aligned, ldb_k % 8 == 0
  uint16_t* C;
  int64_t ldc;
  float* P;            // partials [S][M][N] (S > 1 only)
  int64_t M, N, K;
  int64_t kr;          // rows per K range
  int32_t GN, S;
};

// k extent of one A staging chunk (a multiple of 8 * RPT for every RPT used).
constexpr int kGemvChunk = 1024;

template <int DT>
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = v[d];
    f[2 * d] = cvt_in<DT>((uint16_t)(w & 0xFFFFu));
    f[2 * d + 1] = cvt_in<DT>((uint16_t)(w >> 16));
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// acc[m][j] += sum over the RPT rows of A[m][k] * B[k][n + j], fp32.
//   fp16, MT >= 2: v_dot2_f32_f16 on pairs of consecutive rows (the fp16
//   products are exact in fp32; each instruction adds two of them), the
//   pairs of B assembled with one byte permute per two rows and column.
//   Otherwise (MT == 1, or bfloat16): one fused multiply-add per product.
template <int MT, int RPT, int DT>
__device__ __forceinline__ void fma_rows(float (&acc)[MT][8], const u32x4* v,
                                         const uint16_t (*As)[kGemvChunk], int j0) {
  u32x4 aw[MT][RPT / 8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < RPT / 8; ++q) aw[m][q] = *reinterpret_cast<const u32x4*>(&As[m][j0 + 8 * q]);
  if constexpr (MT >= 2 && DT == DT_F16) {
#pragma unroll
    for (int i = 0; i < RPT; i += 2) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = __builtin_amdgcn_perm(v[i + 1][d], v[i][d], 0x05040100u);  // column 2d
        const uint32_t hi = __builtin_amdgcn_perm(v[i + 1][d], v[i][d], 0x07060302u);  // column 2d+1
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint32_t ap = aw[m][i / 8][(i % 8) / 2];
          const f16x2 a2 = __builtin_bit_cast(f16x2, ap);
          acc[m][2 * d] = __builtin_amdgcn_fdot2(a2, __builtin_bit_cast(f16x2, lo), acc[m][2 * d], false);
          acc[m][2 * d + 1] = __builtin_amdgcn_fdot2(a2, __builtin_bit_cast(f16x2, hi), acc[m][2 * d + 1], false);
        }
      }
    }
  } else {
    float av[MT][RPT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < RPT / 8; ++q) unpack8<DT>(aw[m][q], &av[m][8 * q]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float b[8];
      unpack8<DT>(v[i], b);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_fmaf(av[m][i], b[j], acc[m][j]);
    }
  }
}

// Rows j0 .. j0+RPT-1 of the chunk for a thread that owns 8 full columns.
// Rows at or past cl are read from row cl-1 (inside the range) and replaced
// by zeros, so the loads need no branch.
template <int RPT>
__device__ __forceinline__ void load_rows(u32x4* v, const uint16_t* p0, int64_t ldb_k, int j0, int cl) {
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int j = (j0 + i < cl) ? j0 + i : cl - 1;
    const u32x4 x = *reinterpret_cast<const u32x4*>(p0 + j * ldb_k);
    v[i] = (j0 + i < cl) ? x : zero4();
  }
}

// MT: rows of A handled (>= M); RPT: rows of B per thread per pass; DT: the
// element format.
template <int MT, int RPT, int DT>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  static_assert(RPT % 8 == 0 && kGemvChunk % (8 * RPT) == 0, "pass shape");
  __shared__ __attribute__((aligned(16))) uint16_t As[MT][kGemvChunk];
  __shared__ __attribute__((aligned(16))) float red[8][256];
  const int tid = threadIdx.x;
  const int cg = tid & 31, rg = tid >> 5;
  const int64_t nb = blockIdx.x % a.GN, s = blockIdx.x / a.GN;
  const int64_t n = nb * 256 + cg * 8;
  const int64_t kb = s * a.kr;
  const int64_t ke = (kb + a.kr < a.K) ? kb + a.kr : a.K;
  // Columns this thread owns: 8, fewer at the ragged edge, or none.
  const int nvalid = (n + 8 <= a.N) ? 8 : (n < a.N ? (int)(a.N - n) : 0);
  const uint16_t* bcol = a.B + (nvalid > 0 ? n : 0);

  float acc[MT][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = 0.0f;

  for (int64_t c0 = kb; c0 < ke; c0 += kGemvChunk) {
    const int cl = (ke - c0 < kGemvChunk) ? (int)(ke - c0) : kGemvChunk;
    const uint16_t* p0 = bcol + c0 * a.ldb_k;
    // The chunk's first two passes of B are issued before A is staged, so
    // the round trip of the A loads hides under the B stream instead of
    // preceding it.
    u32x4 v0[RPT], v1[RPT];
    if (nvalid == 8) {
      load_rows<RPT>(v0, p0, a.ldb_k, rg * RPT, cl);
      load_rows<RPT>(v1, p0, a.ldb_k, rg * RPT + 8 * RPT, cl);
    }
    if (c0 != kb) __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int m = 0; m < MT; ++m)
      for (int j = tid; j < kGemvChunk; j += 256)
        As[m][j] = (m < a.M && j < cl) ? a.A[m * a.lda_m + (c0 + j) * a.lda_k] : (uint16_t)0;
    __syncthreads();
    if (nvalid == 8) {
      // Two passes in flight: the pass after next is issued before this
      // pass's arithmetic.  Rows are added in ascending order.
      for (int j0 = rg * RPT; j0 < cl; j0 += 16 * RPT) {
        fma_rows<MT, RPT, DT>(acc, v0, As, j0);
        if (j0 + 8 * RPT >= cl) break;
        if (j0 + 16 * RPT < cl) load_rows<RPT>(v0, p0, a.ldb_k, j0 + 16 * RPT, cl);
        fma_rows<MT, RPT, DT>(acc, v1, As, j0 + 8 * RPT);
        if (j0 + 24 * RPT < cl) load_rows<RPT>(v1, p0, a.ldb_k, j0 + 24 * RPT, cl);
      }
    } else if (nvalid > 0) {
      // The ragged last vector of a row: element loads, one pass at a time.
      for (int j0 = rg * RPT; j0 < cl; j0 += 8 * RPT) {
        u32x4 v[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          v[i] = (j0 + i < cl) ? load_partial8(p0 + (j0 + i) * a.ldb_k, 1, nvalid) : zero4();
        fma_rows<MT, RPT, DT>(acc, v, As, j0);
      }
    }
  }

  // Sum the 8 row groups in ascending order, one row of A at a time.
  const int64_t col = nb * 256 + tid;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= a.M) break;  // uniform across the workgroup
    __syncthreads();      // red is free
    *reinterpret_cast<f32x4*>(&red[rg][cg * 8]) = f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    *reinterpret_cast<f32x4*>(&red[rg][cg * 8 + 4]) = f32x4{acc[m][4], acc[m][5], acc[m][6], acc[m][7]};
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) t += red[r][tid];
    if (col < a.N) {
      if (a.S == 1)
        a.C[m * a.ldc + col] = cvt_out<DT>(t);
      else
        a.P[(s * a.M + m) * a.N + col] = t;
    }
  }
}

}  // namespace gemmf16
