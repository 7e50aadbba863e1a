// Kernel instantiations for the FP8 tile (see tiles.hpp).
#include "tiles.hpp"

namespace gemmf16 {
// Kept in this unit: a non-template inline function in the shared header would
// instantiate (and emit) every FP8 kernel in each unit that includes it.
static TileInfo make_f8_info(int id) {
  TileInfo t;
  t.id = id;
  t.bm = F8Cfg::BM;
  t.bn = F8Cfg::BN;
  t.bk = F8Cfg::BK;
  t.nt = F8Cfg::NT;
  clear_fns(t);
  fill_f8<F8_E4M3, F8_E4M3>(t);
  fill_f8<F8_E4M3, F8_E5M2>(t);
  fill_f8<F8_E5M2, F8_E4M3>(t);
  fill_f8<F8_E5M2, F8_E5M2>(t);
  t.fallback = id;
  t.n_mult = 0;
  return t;
}

TileInfo tile_info_f8() { return make_f8_info(TILE_F8); }
}  // namespace gemmf16
