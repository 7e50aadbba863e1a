// Pre-packing of a static B (the "interleave4" weight packing of the C500
// log, done once outside the timed region) into the layout the main
// kernel's K-major B stages have in LDS.  Included by the host translation
// unit only (non-inline kernel).
#pragma once

#include "dma_kernel.hpp"

namespace gemmf16 {

// Bp: ceil(N/256) panels x ceil(K/32) blocks of 16 KiB.  Byte o of block
// (p, s) holds, for row r = o / 64 (n = 256 p + r) and 16-byte slot
// q = (o % 64) / 16, the 8 elements k = 32 s + 8 (q ^ fa(r)) + e, e = 0..7
// (zero past N or K): the bytes a DMA of a K-major B stage writes to LDS.
// One thread per 16-byte slot; B is read through its element strides, or,
// with kvec (K-contiguous B whose rows start on 16-byte boundaries), with
// one 16-byte load where all 8 elements lie inside K.
__global__ __launch_bounds__(256) void pack_b_kernel(const uint16_t* B, int64_t ldb_k, int64_t ldb_n,
                                                     int64_t K, int64_t N, int64_t S, int64_t slots,
                                                     uint16_t* Bp, int kvec) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= slots) return;
  const int64_t blk = q / 1024, o = (q % 1024) * 16;
  const int64_t pnl = blk / S, s = blk - pnl * S;
  const int r = (int)(o / 64), c = (int)((o % 64) / 16) ^ fa(r);
  const int64_t n = 256 * pnl + r, k0 = 32 * s + 8 * c;
  if (kvec && n < N && k0 + 8 <= K) {
    *reinterpret_cast<u32x4*>(Bp + q * 8) = *reinterpret_cast<const u32x4*>(B + k0 + n * ldb_n);
    return;
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    h[e] = (n < N && k0 + e < K) ? (uint32_t)B[(k0 + e) * ldb_k + n * ldb_n] : 0u;
  *reinterpret_cast<u32x4*>(Bp + q * 8) =
      u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// The same blocks from a K-contiguous B with 16-byte aligned rows, a whole
// line at a time: thread q takes, in a pair of blocks (s = 2 s2 and 2 s2 + 1
// of a panel), n-row r and the 16-byte chunk c8 of its 64 k, so 8
// neighbouring threads read one 128-byte line of a row; the chunk goes to
// slot (c8 % 4) ^ fa(r) of block 2 s2 + c8 / 4.  Over single blocks each
// thread group read half lines, whose other halves went to workgroups on
// other XCDs (a 7168 x 2048 B: 14.1 us that way, 10.1 us this way).
__global__ __launch_bounds__(256) void pack_b_lines_kernel(const uint16_t* B, int64_t ldb_n, int64_t K,
                                                           int64_t N, int64_t S, int64_t threads, uint16_t* Bp) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= threads) return;
  const int64_t S2 = (S + 1) / 2;
  const int64_t pb = q / 2048;
  const int w = (int)(q % 2048), r = w / 8, c8 = w % 8;
  const int64_t pnl = pb / S2, s = 2 * (pb - pnl * S2) + c8 / 4;
  if (s >= S) return;
  const int c = c8 % 4;
  const int64_t n = 256 * pnl + r, k0 = 32 * s + 8 * c;
  uint16_t* dst = Bp + (pnl * S + s) * 8192 + r * 32 + ((c ^ fa(r)) * 8);
  if (n < N && k0 + 8 <= K) {
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(B + k0 + n * ldb_n);
    return;
  }
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (n < N && k0 + e < K) ? (uint32_t)B[k0 + e + n * ldb_n] : 0u;
  *reinterpret_cast<u32x4*>(dst) =
      u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// The same blocks from an N-contiguous B (ldb_n == 1) whose rows start off
// 16-byte boundaries, through LDS: workgroup b builds block b (panel
// b / S, k-block b % S).  Its 32 loads per thread (k-row i, column tid) are
// all in flight before the first LDS write, each instruction reading 128
// consecutive bytes of one k-row; then each thread gathers four 16-byte
// slots (8 k of one n) from LDS and stores them, the block's bytes in order.
__global__ __launch_bounds__(256) void pack_b_rows_kernel(const uint16_t* B, int64_t ldb_k, int64_t K,
                                                          int64_t N, int64_t S, uint16_t* Bp) {
  __shared__ uint16_t t[32][256 + 2];   // k-rows of 516 bytes: the column reads spread over the banks
  const int64_t blk = blockIdx.x;
  const int64_t pnl = blk / S, s = blk - pnl * S;
  const int64_t n0 = 256 * pnl, k0 = 32 * s;
  const int tid = threadIdx.x;
  const int64_t n = n0 + tid;
  uint32_t v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = (n < N && k0 + i < K) ? (uint32_t)B[(k0 + i) * ldb_k + n] : 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i][tid] = (uint16_t)v[i];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = j * 256 + tid;                   // 16-byte slot of the block
    const int r = q / 4, c = (q % 4) ^ fa(r);      // n-row r, k chunk c
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = t[8 * c + e][r];
    *reinterpret_cast<u32x4*>(Bp + blk * 8192 + q * 8) =
        u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
}

// FP8 B [K, N] (bytes, any strides) into the same 16 KiB blocks, one per
// 64 k: byte o of block (p, s) holds, for row r = o / 64 (n = 256 p + r) and
// 16-byte slot q = (o % 64) / 16, the bytes k = 64 s + 16 (q ^ fa(r)) + e,
// e = 0..15 (zero past N or K): the LDS image of the FP8 kernel's K-major
// B stage.  Thread w of a block takes row w % 256 and k chunk w / 256, so
// the 64 lanes of a wave read 64 consecutive columns of one k-row when B is
// N-contiguous.
__global__ __launch_bounds__(256) void pack_b8_kernel(const uint8_t* B, int64_t ldb_k, int64_t ldb_n,
                                                      int64_t K, int64_t N, int64_t S, int64_t slots,
                                                      uint8_t* Bp) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= slots) return;
  const int64_t blk = q / 1024;
  const int w = (int)(q % 1024), r = w % 256, c = w / 256;
  const int64_t pnl = blk / S, s = blk - pnl * S;
  const int64_t n = 256 * pnl + r, k0 = 64 * s + 16 * c;
  uint32_t h[4] = {0u, 0u, 0u, 0u};
  if (n < N) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (k0 + e < K) h[e / 4] |= (uint32_t)B[(k0 + e) * ldb_k + n * ldb_n] << (8 * (e % 4));
  }
  *reinterpret_cast<u32x4*>(Bp + blk * 16384 + r * 64 + ((c ^ fa(r)) * 16)) = u32x4{h[0], h[1], h[2], h[3]};
}

// A [M, K] (16-bit elements, any strides) realigned into Ap [M, ldp], K
// contiguous, ldp a multiple of 64 (rows on 128-byte boundaries), zero at
// k in [K, ldp): the layout the LDS-DMA tile's A stages read.  A workgroup
// moves a 64 x 128 block through LDS: all 32 of a thread's element loads
// are issued before the first LDS write, with consecutive lanes along k when
// A is K-contiguous (else along m, so an M-contiguous A is read in whole
// lines too); then each row leaves as 16-byte stores.  Workgroup ids are
// dealt so that the ids one XCD receives (the dispatcher sends id b to XCD
// b % 8) hold neighbouring blocks along k, which share the cache lines that
// a row not on a 128-byte boundary straddles.  Rows past M are neither read
// nor written.
__global__ __launch_bounds__(256) void realign_a_kernel(const uint16_t* A, int64_t lda_m, int64_t lda_k,
                                                        int64_t M, int64_t K, int64_t ldp, int64_t nbk,
                                                        uint16_t* Ap) {
  __shared__ __align__(16) uint16_t t[64][128 + 8];   // 272-byte rows: 16-byte reads stay aligned
  const int64_t T = (int64_t)gridDim.x, per = T / 8;
  int64_t b = blockIdx.x;
  if (b < per * 8) b = (b % 8) * per + b / 8;
  const int64_t m0 = (b / nbk) * 64, k0 = (b % nbk) * 128;
  const int tid = threadIdx.x;
  const bool k_fast = lda_k == 1 || lda_m != 1;
  uint32_t v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int e = i * 256 + tid;
    const int r = k_fast ? e >> 7 : e & 63, c = k_fast ? e & 127 : e >> 6;
    const int64_t m = m0 + r, k = k0 + c;
    v[i] = (m < M && k < K) ? (uint32_t)A[m * lda_m + k * lda_k] : 0u;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int e = i * 256 + tid;
    const int r = k_fast ? e >> 7 : e & 63, c = k_fast ? e & 127 : e >> 6;
    t[r][c] = (uint16_t)v[i];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = j * 256 + tid, r = q >> 4, c = (q & 15) * 8;
    if (m0 + r < M && k0 + c < ldp)
      *reinterpret_cast<u32x4*>(Ap + (m0 + r) * ldp + k0 + c) = *reinterpret_cast<const u32x4*>(&t[r][c]);
  }
}

// The same copy for an A with K-contiguous rows (lda_k == 1) that start
// off 16-byte boundaries: no transpose, so no LDS.  Each wave takes one
// (row, 1024-element segment) unit: its 16 loads per lane, 128 consecutive
// bytes per instruction, are all in flight before the 16 stores.  Units of
// one row sit in neighbouring waves, so the cache lines a misaligned row
// straddles are fetched once.
__global__ __launch_bounds__(256) void realign_a_rows_kernel(const uint16_t* A, int64_t lda_m, int64_t M,
                                                             int64_t K, int64_t ldp, int64_t nseg,
                                                             uint16_t* Ap) {
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= M * nseg) return;
  const int lane = threadIdx.x & 63;
  const int64_t m = u / nseg, k0 = (u - m * nseg) * 1024 + lane;
  const uint16_t* src = A + m * lda_m;
  uint16_t* dst = Ap + m * ldp;
  uint32_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t k = k0 + 64 * j;
    v[j] = k < K ? (uint32_t)src[k] : 0u;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t k = k0 + 64 * j;
    if (k < ldp) dst[k] = (uint16_t)v[j];
  }
}

}  // namespace gemmf16
