// k_ring.hip -- ring tile and weight-resident tile kernel instantiations
// (tile_ring.hpp, tile_wres.hpp).
#include "kernels.h"
#include "tile_ring.hpp"
#include "tile_wres.hpp"

namespace {

template <int WR, int A, int WM, int B>
const void* ring_st(int stages) {
  switch (stages) {
    case 3: return reinterpret_cast<const void*>(&fp::ring_tile_kernel<WR, A, WM, B, 3>);
    case 4:
      if constexpr (B <= 4)
        return reinterpret_cast<const void*>(&fp::ring_tile_kernel<WR, A, WM, B, 4>);
      return nullptr;
    case 6:
      if constexpr (B <= 4)
        return reinterpret_cast<const void*>(&fp::ring_tile_kernel<WR, A, WM, B, 6>);
      return nullptr;
    default: return nullptr;
  }
}

}  // namespace

namespace fpk {

// Wave grids of the ring kernel per token block (16 * mt16 slots).
const void* ring(int mt16, int stages) {
  switch (mt16) {
    case 1: return ring_st<4, 1, 1, 1>(stages);
    case 2: return ring_st<4, 1, 1, 2>(stages);
    case 4: return ring_st<2, 2, 2, 2>(stages);
    case 8: return ring_st<2, 2, 2, 4>(stages);
    case 16: return ring_st<2, 2, 2, 8>(stages);
    default: return nullptr;
  }
}

const void* wres(int mt16) {
  switch (mt16) {
    case 2: return reinterpret_cast<const void*>(&fp::wres_tile_kernel<1>);
    case 4: return reinterpret_cast<const void*>(&fp::wres_tile_kernel<2>);
    case 8: return reinterpret_cast<const void*>(&fp::wres_tile_kernel<4>);
    case 16: return reinterpret_cast<const void*>(&fp::wres_tile_kernel<8>);
    default: return nullptr;
  }
}

}  // namespace fpk
