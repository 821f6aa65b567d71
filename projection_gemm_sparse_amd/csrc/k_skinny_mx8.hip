// k_skinny_mx8.hip -- vector-ALU kernel instantiations for MXFP8 weights;
// also the fpk::skinny_mx getter over the block-scaled formats.
#include "kernels.h"
#include "skinny_table.hpp"

const void* fpk_skinny_fp4(int var, int mt, int cj, int rw);

namespace fpk {

const void* skinny_mx(int var, int mt, int cj, int rw) {
  if (var == fp::kVarMx8) return fpk_detail::skinny_mx<fp::kVarMx8>(mt, cj, rw);
  return fpk_skinny_fp4(var, mt, cj, rw);
}

}  // namespace fpk
