// Static facts of the kernel instances (host code: used by validation, plan creation and the
// tile query of the C-ABI).
#include "ge_tiles.h"

namespace ge {

TileInfo tile_info(TileKind kind) {
  switch (kind) {
    case TILE_256x256: return info_of<T256>();
    case TILE_256x128_PAIR: return info_of<T256P>();
    case TILE_128x128: return info_of<T128>();
    case TILE_64x64: return info_of<T64>();
    case TILE_128x128_PAIR: return info_of<T128P>();
    case TILE_256x256_2W: return info_of<T256W8>();
    case TILE_256x128_PAIR_2W: return info_of<T256PW8>();
    default: return TileInfo{0, 0, 0, 0, false, 0};
  }
}

}  // namespace ge
