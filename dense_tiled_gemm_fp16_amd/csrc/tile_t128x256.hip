// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t128x256() { return make_info<CfgT128x256>(TILE_T128X256); }
}  // namespace gemmf16
