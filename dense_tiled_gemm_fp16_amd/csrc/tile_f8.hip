// Kernel instantiations for the FP8 tile (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
TileInfo tile_info_f8() { return make_f8_info(TILE_F8); }
}  // namespace gemmf16
