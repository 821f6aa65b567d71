// k_skinny_bf16.hip -- vector-ALU kernel instantiations: bf16 projections
// and the gate/up (SwiGLU) form.
#include "kernels.h"
#include "skinny_table.hpp"

namespace fpk {

const void* skinny_pairs(int mt, int cj, int rw) {
  using namespace fpk_detail;
  switch (mt) {
    case 1: return skinny_pairs_cj<1>(cj, rw);
    case 2: return skinny_pairs_cj<2>(cj, rw);
    case 4: return skinny_pairs_cj<4>(cj, rw);
    case 8: return skinny_pairs_cj<8>(cj, rw);
    default: return nullptr;
  }
}

}  // namespace fpk

// bf16 half of fpk::skinny (the fp32 half is in k_skinny_f32.hip)
const void* fpk_skinny_bf16(int mt, int cj, int rw) {
  return fpk_detail::skinny_plain<true>(mt, cj, rw);
}
