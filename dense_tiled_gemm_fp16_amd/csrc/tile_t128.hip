// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t128() { return make_info<CfgT128, true, true>(TILE_T128); }
}  // namespace gemmf16
