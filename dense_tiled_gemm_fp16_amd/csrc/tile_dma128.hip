// Kernel instantiations for the 128x128 LDS-DMA tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_dma128() { return make_dma_info<CfgDma128, true>(TILE_DMA128, TILE_T128); }
}  // namespace gemmf16
