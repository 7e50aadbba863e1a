// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_s16() { return make_info<CfgS16, false, true>(TILE_S16); }
}  // namespace gemmf16
