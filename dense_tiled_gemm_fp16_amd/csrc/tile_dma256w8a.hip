// Kernel instantiations for an 8-wave LDS-DMA tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_dma256w8a() { return make_dma_info<CfgDma256W8A>(TILE_DMA256W8A, TILE_T256); }
}  // namespace gemmf16
