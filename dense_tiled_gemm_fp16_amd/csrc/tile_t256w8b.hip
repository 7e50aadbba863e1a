// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t256w8b() { return make_info<CfgT256W8B>(TILE_T256W8B); }
}  // namespace gemmf16
