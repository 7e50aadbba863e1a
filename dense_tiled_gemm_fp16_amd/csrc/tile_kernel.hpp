// The tiled MFMA kernel and the split-K reduction (gfx950 / CDNA4).
//
// One workgroup owns one BM x BN output tile and one K range (the whole of K
// unless the launch is split).  It clears an fp32 accumulator, walks its K
// range in BK steps through a two-stage LDS ring, and stores once; every
// valid output has exactly one writer and after q steps the accumulator
// holds exactly the contributions of the valid k of those steps (the Triton
// article's sections "parallelise over outputs, keep K in the accumulator"
// and the ownership/loop-invariant paragraph; the tiling tutorial's section
// 03 and the double-buffering of section 06).
//
// Inner product: v_mfma_f32_32x32x16_f16 (MI = 32) or
// v_mfma_f32_16x16x32_f16 (MI = 16).  The MFMA is issued with the B tile as
// its first operand and the A tile as its second, i.e. it computes the
// transposed block C^T[n][m]; in that orientation each lane ends up holding
// 4 consecutive n of one output row m, which become one 8-byte store.
//
// Split K (TileLang tutorial ch. 14, section 4.1; Triton article, section
// "neighbouring programs share cache", last paragraph): with PARTIAL the
// workgroup writes its fp32 partial tile to W[split][M][N] instead of C, and
// splitk_reduce sums the partials in ascending split order, so the result is
// bit-identical from run to run (no atomics; the reduction kernel is in
// reduce_kernel.hpp).  fp32 partials, never fp16 (TileLang tutorial ch. 14,
// pitfall 4).
#pragma once

#include "tile_common.hpp"

namespace gemmf16 {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MI_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int MI = MI_;                     // MFMA output block edge
  static constexpr int KI = (MI == 32) ? 16 : 32;    // k per MFMA
  static constexpr int WTM = BM / WAVES_M;           // wave tile, rows (m)
  static constexpr int WTN = BN / WAVES_N;           // wave tile, cols (n)
  static constexpr int FM = WTM / MI, FN = WTN / MI; // MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert(MI == 32 || MI == 16, "MFMA shape");
  static_assert(WTM % MI == 0 && WTN % MI == 0 && BK % KI == 0, "tile shape");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

struct KArgs {
  const uint16_t* A;
  int64_t lda_m, lda_k;
  const uint16_t* B;
  int64_t ldb_k, ldb_n;
  uint16_t* C;
  int64_t ldc;
  float* W;          // split partials [S][M][N] (PARTIAL launches only)
  int64_t M, N, K;
  int64_t k_split;   // K elements per split, a multiple of BK
  int64_t GM, GN;    // tile grid
  int32_t panel;     // raster group height, <= 0 = plain order
  int32_t c_vec;     // C rows take 8-byte stores (ldc % 4 == 0, C 8-byte aligned)
  // Grouped launches only (see group_tile): per-group row offsets (G + 1,
  // clamped to [0, M]), prefix sums of per-group row tiles (G + 1), the
  // element distance between consecutive groups' B, and the group count.
  const int64_t* g_off;
  const int64_t* g_tiles;
  int64_t ldb_g;
  int32_t G;
  // Stream-K tail launches only (sk_tiles > 0, PARTIAL kernels of the
  // full-line-A tile): workgroup w takes K range w / sk_tiles of the tile
  // that raster id sk_first + w % sk_tiles maps to, and writes its partial
  // tile densely to W at slot w (BM x BN floats, row-major).
  int64_t sk_first;
  int64_t sk_tiles;
  // Split-K launches (PARTIAL, sk_tiles == 0): ids that share w mod 8 (one
  // XCD's share under the dispatcher's round-robin) hold all T tiles of the
  // same K ranges; needs a split count that is a multiple of 8.
  int32_t split_xcd;
};

// Workgroup id of a split-K launch -> (K range, tile index).  With
// split_xcd the T tiles of one K range read the same A rows and B columns
// at the same time on one XCD, so that XCD's L2 fetches them once instead of
// each tile's XCD fetching them again.
__device__ __forceinline__ void split_tile_of(int64_t w, int64_t T, int split_xcd, int64_t& split,
                                              int64_t& tile) {
  if (split_xcd) {
    const int64_t r = w >> 3;
    split = (w & 7) + 8 * (r / T);
    tile = r - (r / T) * T;
  } else {
    split = w / T;
    tile = w - split * T;
  }
}

// Grouped product (TileLang tutorial ch. 14, section 4.3: one launch over
// several GEMMs that share N and K, with per-group row counts; here group g
// owns rows [off[g], off[g+1]) of A and C and its own B).  The grid is an
// upper bound computed without the row counts: workgroups at or past the
// live count L = tiles[G] * GN return false.  Row tiles of the concatenated
// per-group tile lists are dealt to the XCDs in turn (the dispatcher sends
// id w to XCD w % 8; XCD x takes row tiles x, x + 8, ..., each with its GN
// column tiles in consecutive places, so they share the row tile's A in one
// L2).  All XCDs thus work through the groups together and only a few
// groups' B are live at a time, which the Infinity Cache holds; a contiguous
// run per XCD kept about eight groups' B live and ran 4-7% slower on the
// 32-expert MoE workload.  Row tiles past the last multiple of 8 keep plain
// order.  The group is the last g with tiles[g] <= t (binary search), and A,
// C, B and M are rebased on it.  ESZ: bytes per A and B element (2; 1 for
// FP8, whose strides count bytes).
template <int ESZ = 2>
__device__ __forceinline__ bool group_tile(KArgs& a, int64_t w, int64_t& pm, int64_t& pn) {
  const int64_t L = a.g_tiles[a.G] * a.GN;
  if (w >= L) return false;
  const int64_t R8 = a.g_tiles[a.G] / 8 * 8;
  int64_t t;
  if (w < R8 * a.GN) {
    const int64_t j = w / 8;   // place in XCD w % 8's run
    t = 8 * (j / a.GN) + w % 8;
    pn = j % a.GN;
  } else {
    t = w / a.GN;
    pn = w - t * a.GN;
  }
  int lo = 0, hi = a.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.g_tiles[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int64_t r0 = a.g_off[lo], r1 = a.g_off[lo + 1];
  pm = t - a.g_tiles[lo];
  a.A = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.A) + r0 * a.lda_m * ESZ);
  a.C += r0 * a.ldc;
  a.B = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.B) + (int64_t)lo * a.ldb_g * ESZ);
  a.M = r1 - r0;
  return true;
}

template <int MI>
struct Acc;
template <>
struct Acc<32> { typedef f32x16 type; static constexpr int N = 16; };
template <>
struct Acc<16> { typedef f32x4 type; static constexpr int N = 4; };

template <int MI, int DT>
__device__ __forceinline__ typename Acc<MI>::type mfma(f16x8 a, f16x8 b, typename Acc<MI>::type c) {
  if constexpr (DT == DT_F16) {
    if constexpr (MI == 32)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  } else {
    const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
    if constexpr (MI == 32)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
  }
}

// 4 consecutive outputs C[m][n..n+3] (round to nearest even).
template <int DT>
__device__ __forceinline__ void store4_out(const KArgs& a, int64_t m, int64_t n, float v0, float v1,
                                           float v2, float v3) {
  if (m >= a.M || n >= a.N) return;
  uint16_t* p = a.C + m * a.ldc + n;
  const uint16_t h[4] = {cvt_out<DT>(v0), cvt_out<DT>(v1), cvt_out<DT>(v2), cvt_out<DT>(v3)};
  if (a.c_vec && n + 4 <= a.N) {
    *reinterpret_cast<u32x2*>(p) = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) p[e] = h[e];
  }
}

// 4 consecutive fp32 partials W[split][m][n..n+3].
__device__ __forceinline__ void store4_f32(const KArgs& a, int64_t split, int64_t m, int64_t n,
                                           float v0, float v1, float v2, float v3) {
  if (m >= a.M || n >= a.N) return;
  float* p = a.W + (split * a.M + m) * a.N + n;
  if ((a.N & 3) == 0) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v0, v1, v2, v3};
  } else {
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) p[e] = v[e];
  }
}

// MFMAs of one BK step from one LDS stage.  Operand fragments are double
// buffered in registers: the reads for k-step ks+1 are issued before the
// MFMAs of k-step ks so LDS latency hides behind matrix work.
template <class CF, int DT>
__device__ __forceinline__ void compute_stage(const char* ta, const char* tb,
                                              typename Acc<CF::MI>::type (&acc)[CF::FN][CF::FM],
                                              int wm, int wn, int lane) {
  constexpr int MI = CF::MI, KI = CF::KI, KS = CF::BK / KI;
  const int lr = lane % MI, lc = lane / MI;
  f16x8 fa[2][CF::FN], fb[2][CF::FM];
  auto read = [&](int ks, int slot) {
    const int c = ks * (KI / 8) + lc;
#pragma unroll
    for (int i = 0; i < CF::FN; ++i)
      fa[slot][i] = *reinterpret_cast<const f16x8*>(tb + cell_off<CF::BN>(wn * CF::WTN + i * MI + lr, c));
#pragma unroll
    for (int j = 0; j < CF::FM; ++j)
      fb[slot][j] = *reinterpret_cast<const f16x8*>(ta + cell_off<CF::BM>(wm * CF::WTM + j * MI + lr, c));
  };
  read(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) read(ks + 1, (ks + 1) & 1);
#pragma unroll
    for (int i = 0; i < CF::FN; ++i)
#pragma unroll
      for (int j = 0; j < CF::FM; ++j) acc[i][j] = mfma<MI, DT>(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
  }
}

// The K loop over [kb, ke): full BK steps run branch-free; a ragged last step
// (K or the split end not a multiple of BK) is loaded with K masks.  Two LDS
// stages: while stage t is consumed, step t+1 is fetched into registers and
// then written to the other stage; one barrier per step.
template <class CF, int DT, bool ROWMASK, class SA, class SB>
__device__ __forceinline__ void main_loop(SA& sa, SB& sb, char* smem,
                                          typename Acc<CF::MI>::type (&acc)[CF::FN][CF::FM],
                                          int64_t kb, int64_t ke, int wm, int wn, int lane) {
  constexpr int BK = CF::BK;
  const int64_t nfull = (ke - kb) / BK;
  const bool tail = (ke - kb) % BK != 0;
  if (nfull > 0) {
    sa.template load<ROWMASK, false>(kb, ke);
    sb.template load<ROWMASK, false>(kb, ke);
  } else {
    sa.template load<ROWMASK, true>(kb, ke);
    sb.template load<ROWMASK, true>(kb, ke);
  }
  sa.store(smem);
  sb.store(smem + CF::A_BYTES);
  __syncthreads();
  int64_t t = 0;
  for (; t + 1 < nfull; ++t) {
    const int cur = (int)(t & 1);
    sa.template load<ROWMASK, false>(kb + (t + 1) * BK, ke);
    sb.template load<ROWMASK, false>(kb + (t + 1) * BK, ke);
    compute_stage<CF, DT>(smem + cur * CF::STAGE, smem + cur * CF::STAGE + CF::A_BYTES, acc, wm, wn, lane);
    sa.store(smem + (cur ^ 1) * CF::STAGE);
    sb.store(smem + (cur ^ 1) * CF::STAGE + CF::A_BYTES);
    __syncthreads();
  }
  if (tail && nfull > 0) {
    const int cur = (int)(t & 1);
    sa.template load<ROWMASK, true>(kb + nfull * BK, ke);
    sb.template load<ROWMASK, true>(kb + nfull * BK, ke);
    compute_stage<CF, DT>(smem + cur * CF::STAGE, smem + cur * CF::STAGE + CF::A_BYTES, acc, wm, wn, lane);
    sa.store(smem + (cur ^ 1) * CF::STAGE);
    sb.store(smem + (cur ^ 1) * CF::STAGE + CF::A_BYTES);
    __syncthreads();
    ++t;
  }
  const int cur = (int)(t & 1);
  compute_stage<CF, DT>(smem + cur * CF::STAGE, smem + cur * CF::STAGE + CF::A_BYTES, acc, wm, wn, lane);
}

template <class CF, int APATH, int BPATH, bool PARTIAL, bool GROUPED = false, int DT = DT_F16>
__global__ __launch_bounds__(CF::NT) void gemm_tile_kernel(KArgs a) {
  static_assert(!(PARTIAL && GROUPED), "grouped launches are never split");
  __shared__ __attribute__((aligned(16))) char smem[CF::LDS];
  constexpr int BK = CF::BK, MI = CF::MI;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

  const int64_t T = a.GM * a.GN;
  int64_t w = blockIdx.x;
  int64_t split = 0;
  if constexpr (PARTIAL) split_tile_of(blockIdx.x, T, a.split_xcd, split, w);
  int64_t pm, pn;
  if constexpr (GROUPED) {
    if (!group_tile(a, w, pm, pn)) return;   // uniform per workgroup, before any barrier
  } else {
    raster_tile(w, a.GM, a.GN, a.panel, pm, pn);
  }
  const int64_t m0 = pm * CF::BM, n0 = pn * CF::BN;
  const int64_t kb = split * a.k_split;
  const int64_t ke = (kb + a.k_split < a.K) ? kb + a.k_split : a.K;

  OperandStage<CF::BM, BK, CF::NT, APATH> sa;
  OperandStage<CF::BN, BK, CF::NT, BPATH> sb;
  sa.init(a.A, a.lda_m, a.lda_k, a.M, m0, tid);
  sb.init(a.B, a.ldb_n, a.ldb_k, a.N, n0, tid);

  typedef typename Acc<MI>::type acc_t;
  acc_t acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j)
#pragma unroll
      for (int e = 0; e < Acc<MI>::N; ++e) acc[i][j][e] = 0.0f;

  const bool interior = (m0 + CF::BM <= a.M) && (n0 + CF::BN <= a.N);
  if (interior)
    main_loop<CF, DT, false>(sa, sb, smem, acc, kb, ke, wm, wn, lane);
  else
    main_loop<CF, DT, true>(sa, sb, smem, acc, kb, ke, wm, wn, lane);

  // Epilogue.  MFMA output layout (C^T block, MI x MI): lane holds column
  // j = lane % MI (our m) and, for register group g, 4 consecutive rows
  // (our n) starting at 8g + 4*(lane/32) for MI = 32, 4*(lane/16) for MI = 16.
  constexpr int G = Acc<MI>::N / 4;
  const int lr = lane % MI;
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j) {
      const int64_t m = m0 + wm * CF::WTM + j * MI + lr;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int nl = (MI == 32) ? (8 * g + 4 * (lane >> 5)) : (4 * (lane >> 4));
        const int64_t n = n0 + wn * CF::WTN + i * MI + nl;
        const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if constexpr (PARTIAL)
          store4_f32(a, split, m, n, v0, v1, v2, v3);
        else
          store4_out<DT>(a, m, n, v0, v1, v2, v3);
      }
    }
}

}  // namespace gemmf16
