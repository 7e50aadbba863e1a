// Kernel instantiations for one tile configuration (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_s32() { return make_info<CfgS32, false, true>(TILE_S32); }
}  // namespace gemmf16
