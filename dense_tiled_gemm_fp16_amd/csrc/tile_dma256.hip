// Kernel instantiations for the LDS-DMA tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_dma256() { return make_dma_info<CfgDma256>(TILE_DMA256, TILE_T256); }
}  // namespace gemmf16
