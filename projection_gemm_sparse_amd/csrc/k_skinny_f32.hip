// k_skinny_f32.hip -- vector-ALU kernel instantiations: fp32 projections and
// fp32 outputs from bf16 operands (router logits); also the fpk::skinny
// getter over both operand types.
#include "kernels.h"
#include "skinny_table.hpp"

const void* fpk_skinny_bf16(int mt, int cj, int rw);

namespace fpk {

const void* skinny(bool bf16, int mt, int cj, int rw) {
  return bf16 ? fpk_skinny_bf16(mt, cj, rw) : fpk_detail::skinny_plain<false>(mt, cj, rw);
}

const void* skinny_f32out(int mt, int cj, int rw) {
  using namespace fpk_detail;
  switch (mt) {
    case 1: return skinny_f32out_cj<1>(cj, rw);
    case 2: return skinny_f32out_cj<2>(cj, rw);
    case 4: return skinny_f32out_cj<4>(cj, rw);
    case 8: return skinny_f32out_cj<8>(cj, rw);
    case 16: return skinny_f32out_cj<16>(cj, rw);
    default: return nullptr;
  }
}

}  // namespace fpk
