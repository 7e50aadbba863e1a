// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_t256() { return make_info<CfgT256>(TILE_T256); }
}  // namespace gemmf16
