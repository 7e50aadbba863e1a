// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t256w8a() { return make_info<CfgT256W8A>(TILE_T256W8A); }
}  // namespace gemmf16
