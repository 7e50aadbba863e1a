// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_s64() { return make_info<CfgS64, false, true>(TILE_S64); }
}  // namespace gemmf16
