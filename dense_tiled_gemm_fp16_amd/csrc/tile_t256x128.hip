// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t256x128() { return make_info<CfgT256x128>(TILE_T256X128); }
}  // namespace gemmf16
