// Kernel instantiations for the full-line-A LDS-DMA tile (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_dma256a128() { return make_dma_a128_info<CfgDmaA128>(TILE_DMA256A128, TILE_DMA256W8B); }
}  // namespace gemmf16
