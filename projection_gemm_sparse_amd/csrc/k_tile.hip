// k_tile.hip -- LDS tile kernel instantiations (tile.hpp).
#include "kernels.h"
#include "tile.hpp"

namespace {

template <int MT16, int NW>
const void* tile_per(int per) {
  switch (per) {
    case 8: return reinterpret_cast<const void*>(&fp::tile_kernel<MT16, NW, 4, 2>);
    case 10: return reinterpret_cast<const void*>(&fp::tile_kernel<MT16, NW, 5, 2>);
    case 16: return reinterpret_cast<const void*>(&fp::tile_kernel<MT16, NW, 4, 4>);
    case 20: return reinterpret_cast<const void*>(&fp::tile_kernel<MT16, NW, 5, 4>);
    case 40: return reinterpret_cast<const void*>(&fp::tile_kernel<MT16, NW, 5, 8>);
    default: return nullptr;
  }
}

template <int MT16>
const void* tile_nw(int nw, int per) {
  switch (nw) {
    case 2: return tile_per<MT16, 2>(per);
    case 4: return tile_per<MT16, 4>(per);
    case 8: return tile_per<MT16, 8>(per);
    default: return nullptr;
  }
}

}  // namespace

namespace fpk {

const void* tile(int mt16, int nw, int per) {
  switch (mt16) {
    case 1: return tile_nw<1>(nw, per);
    case 2: return tile_nw<2>(nw, per);
    case 4: return tile_nw<4>(nw, per);
    case 8: return tile_nw<8>(nw, per);
    case 16: return tile_nw<16>(nw, per);
    default: return nullptr;
  }
}

}  // namespace fpk
