// Kernel instantiations for the 64x128 LDS-DMA tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_dma64x128() { return make_dma_info<CfgDma64x128, true>(TILE_DMA64X128, TILE_T128); }
}  // namespace gemmf16
