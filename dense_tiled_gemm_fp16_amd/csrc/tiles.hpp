// Tile configurations and the per-configuration kernel tables.  Each
// configuration is instantiated in its own translation unit (tile_<id>.hip)
// so the library builds in parallel; the host side only sees TileInfo.
#pragma once

#include "dma_a128_kernel.hpp"
#include "dma_kernel.hpp"
#include "f8_kernel.hpp"
#include "tile_kernel.hpp"

namespace gemmf16 {

// <BM, BN, BK, waves along m, waves along n, MFMA edge>
typedef TileCfg<128, 128, 64, 2, 2, 32> CfgT128;    // main / split-K, mid-size problems
typedef TileCfg<64, 32, 32, 2, 2, 16> CfgT64x32;    // the pages' 64x32x32 geometry
typedef TileCfg<16, 256, 64, 1, 4, 16> CfgS16;      // skinny, M <= 16
typedef TileCfg<32, 256, 64, 1, 4, 32> CfgS32;      // skinny, M <= 32
typedef TileCfg<64, 256, 64, 1, 4, 32> CfgS64;      // skinny, M <= 64
typedef TileCfg<256, 256, 64, 2, 2, 32> CfgT256;    // register path for layouts the DMA tiles skip
typedef DmaCfg<4, 4, 2> CfgDma256W8B;               // 256x256x32, 4-stage LDS-DMA ring, 8 waves of 64x128
typedef DmaCfg<4, 2, 2, 128, 128> CfgDma128;        // 128x128x32, 4-stage LDS-DMA ring, 4 waves of 64x64
typedef DmaCfg<4, 1, 2, 64, 128> CfgDma64x128;      // 64x128x32, the same ring, 2 waves of 64x64
typedef DmaA128Cfg<4, 2> CfgDmaA128;                // same tile, A staged in 128-byte rows

// Ids 9 to 12 belonged to superseded 256-wide tiles that no plan chose; they
// stay unused so that the other ids keep their meaning.
enum TileId {
  TILE_T128 = 1, TILE_T64X32 = 2, TILE_S16 = 3, TILE_S32 = 4, TILE_S64 = 5,
  TILE_T256 = 6, TILE_DMA128 = 7, TILE_DMA64X128 = 8, TILE_DMA256W8B = 13, TILE_DMA256A128 = 14, TILE_F8 = 15, TILE_MAX = 15
};

typedef void (*kfn_t)(KArgs);

struct TileInfo {
  int id, bm, bn, bk, nt;
  kfn_t final_fn[NDT][9];  // [format][a_path * 3 + b_path]; nullptr = not supported
  kfn_t partial_fn[NDT][9];
  kfn_t grouped_fn[NDT][9];  // grouped launches, per format (nullptr: not instantiated)
  kfn_t packed_fn[NDT];    // pre-packed B, K-contiguous A, per format (nullptr: none)
  kfn_t packed_partial_fn[NDT];  // the same writing fp32 partials (stream-K tails)
  int fallback;         // tile used for layouts this one does not support
  int n_mult;           // N-contiguous B needs N to be a multiple of this (0 = any)
  int64_t max_k;        // largest K the tile's 32-bit step counters cover (0 = any)
  int64_t max_ld;       // largest element stride its 32-bit lane offsets cover (0 = any)
};

template <class CF, bool P, bool G = false, int DT = DT_F16>
void fill_fns(kfn_t* f) {
  f[0] = gemm_tile_kernel<CF, PATH_GATHER, PATH_GATHER, P, G, DT>;
  f[1] = gemm_tile_kernel<CF, PATH_GATHER, PATH_KVEC, P, G, DT>;
  f[2] = gemm_tile_kernel<CF, PATH_GATHER, PATH_RVEC, P, G, DT>;
  f[3] = gemm_tile_kernel<CF, PATH_KVEC, PATH_GATHER, P, G, DT>;
  f[4] = gemm_tile_kernel<CF, PATH_KVEC, PATH_KVEC, P, G, DT>;
  f[5] = gemm_tile_kernel<CF, PATH_KVEC, PATH_RVEC, P, G, DT>;
  f[6] = gemm_tile_kernel<CF, PATH_RVEC, PATH_GATHER, P, G, DT>;
  f[7] = gemm_tile_kernel<CF, PATH_RVEC, PATH_KVEC, P, G, DT>;
  f[8] = gemm_tile_kernel<CF, PATH_RVEC, PATH_RVEC, P, G, DT>;
}

inline void clear_fns(TileInfo& t) {
  t.max_k = 0;
  t.max_ld = 0;
  for (int d = 0; d < NDT; ++d)
    for (int i = 0; i < 9; ++i) t.final_fn[d][i] = t.partial_fn[d][i] = nullptr;
  for (int d = 0; d < NDT; ++d)
    for (int i = 0; i < 9; ++i) t.grouped_fn[d][i] = nullptr;
  for (int d = 0; d < NDT; ++d) t.packed_fn[d] = t.packed_partial_fn[d] = nullptr;
}

// Register-path tiles: fp16 always; bfloat16 and grouped launches where asked.
template <class CF, bool WITH_GROUPED = false, bool WITH_BF16 = false>
TileInfo make_info(int id) {
  TileInfo t;
  t.id = id;
  t.bm = CF::BM;
  t.bn = CF::BN;
  t.bk = CF::BK;
  t.nt = CF::NT;
  clear_fns(t);
  fill_fns<CF, false>(t.final_fn[DT_F16]);
  fill_fns<CF, true>(t.partial_fn[DT_F16]);
  if constexpr (WITH_BF16) {
    fill_fns<CF, false, false, DT_BF16>(t.final_fn[DT_BF16]);
    fill_fns<CF, true, false, DT_BF16>(t.partial_fn[DT_BF16]);
  }
  if constexpr (WITH_GROUPED) {
    fill_fns<CF, false, true>(t.grouped_fn[DT_F16]);
    if constexpr (WITH_BF16) fill_fns<CF, false, true, DT_BF16>(t.grouped_fn[DT_BF16]);
  }
  t.fallback = 0;
  t.n_mult = 0;
  return t;
}

// The LDS-DMA kernel takes K-contiguous A with K- or N-contiguous B only;
// bfloat16, and FP8 with K-contiguous B, where asked.
template <int F8, class CF>
void fill_dma_f8(TileInfo& t) {
  t.final_fn[DT_F8 + F8][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, false, DT_F16, F8>;
  t.partial_fn[DT_F8 + F8][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, true, DT_F16, F8>;
}

template <class CF, bool WITH_BF16 = false>
TileInfo make_dma_info(int id, int fallback) {
  TileInfo t;
  t.id = id;
  t.bm = CF::BM;
  t.bn = CF::BN;
  t.bk = CF::BK;
  t.nt = CF::NT;
  clear_fns(t);
  t.final_fn[DT_F16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, false>;
  t.final_fn[DT_F16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_kernel<CF, false, false>;
  t.partial_fn[DT_F16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, true>;
  t.partial_fn[DT_F16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_kernel<CF, false, true>;
  if constexpr (WITH_BF16) {
    t.final_fn[DT_BF16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, false, DT_BF16>;
    t.final_fn[DT_BF16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_kernel<CF, false, false, DT_BF16>;
    t.partial_fn[DT_BF16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_kernel<CF, true, true, DT_BF16>;
    t.partial_fn[DT_BF16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_kernel<CF, false, true, DT_BF16>;
    fill_dma_f8<0, CF>(t);
    fill_dma_f8<1, CF>(t);
    fill_dma_f8<2, CF>(t);
    fill_dma_f8<3, CF>(t);
  }
  t.fallback = fallback;
  t.n_mult = 8;
  return t;
}

// The full-line-A LDS-DMA kernel takes K-contiguous A with K- or N-contiguous B.
template <class CF>
TileInfo make_dma_a128_info(int id, int fallback) {
  TileInfo t;
  t.id = id;
  t.bm = CF::BM;
  t.bn = CF::BN;
  t.bk = CF::BK;
  t.nt = CF::NT;
  clear_fns(t);
  t.final_fn[DT_F16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, false>;
  t.final_fn[DT_F16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, false>;
  t.partial_fn[DT_F16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, true>;
  t.partial_fn[DT_F16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, true>;
  t.final_fn[DT_BF16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, false, false, DT_BF16>;
  t.final_fn[DT_BF16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, false, false, DT_BF16>;
  t.partial_fn[DT_BF16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, true, false, DT_BF16>;
  t.partial_fn[DT_BF16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, true, false, DT_BF16>;
  t.grouped_fn[DT_F16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, false, true>;
  t.grouped_fn[DT_F16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, false, true>;
  t.grouped_fn[DT_BF16][PATH_KVEC * 3 + PATH_KVEC] = gemm_dma_a128_kernel<CF, true, false, true, DT_BF16>;
  t.grouped_fn[DT_BF16][PATH_KVEC * 3 + PATH_RVEC] = gemm_dma_a128_kernel<CF, false, false, true, DT_BF16>;
  t.packed_fn[DT_F16] = gemm_dma_a128_kernel<CF, true, false, false, DT_F16, true>;
  t.packed_fn[DT_BF16] = gemm_dma_a128_kernel<CF, true, false, false, DT_BF16, true>;
  t.packed_partial_fn[DT_F16] = gemm_dma_a128_kernel<CF, true, true, false, DT_F16, true>;
  t.packed_partial_fn[DT_BF16] = gemm_dma_a128_kernel<CF, true, true, false, DT_BF16, true>;
  t.fallback = fallback;
  t.n_mult = 8;
  t.max_k = INT64_C(1) << 36;   // 64-k super-steps counted in int
  t.max_ld = INT64_C(1) << 23;  // 255 rows * 2^23 * 2 bytes + bias < 2^32
  return t;
}

// The FP8 tile: K-contiguous A; B K-contiguous ([N, K] rows) or
// N-contiguous ([K, N] rows); the four format pairs; no other layout and no
// 16-bit format.
template <int FA, int FB>
void fill_f8(TileInfo& t) {
  t.final_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_KVEC] = gemm_f8_kernel<FA, FB, false>;
  t.partial_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_KVEC] = gemm_f8_kernel<FA, FB, true>;
  t.final_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_RVEC] = gemm_f8_kernel<FA, FB, false, true>;
  t.partial_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_RVEC] = gemm_f8_kernel<FA, FB, true, true>;
  t.packed_fn[DT_F8 + 2 * FA + FB] = gemm_f8_kernel<FA, FB, false, false, true>;
  t.packed_partial_fn[DT_F8 + 2 * FA + FB] = gemm_f8_kernel<FA, FB, true, false, true>;
  t.grouped_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_KVEC] = gemm_f8_kernel<FA, FB, false, false, false, true>;
  t.grouped_fn[DT_F8 + 2 * FA + FB][PATH_KVEC * 3 + PATH_RVEC] = gemm_f8_kernel<FA, FB, false, true, false, true>;
}

// Defined in tile_<id>.hip.
TileInfo tile_info_t128();
TileInfo tile_info_t64x32();
TileInfo tile_info_s16();
TileInfo tile_info_s32();
TileInfo tile_info_s64();
TileInfo tile_info_t256();
TileInfo tile_info_dma256w8b();
TileInfo tile_info_dma128();
TileInfo tile_info_dma64x128();
TileInfo tile_info_dma256a128();
TileInfo tile_info_f8();

}  // namespace gemmf16
