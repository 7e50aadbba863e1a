// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t64x32() { return make_info<CfgT64x32>(TILE_T64X32); }
}  // namespace gemmf16
