// k_skinny_fp4.hip -- vector-ALU kernel instantiations for 4-bit weights
// (MXFP4 and NVFP4).
#include "kernels.h"
#include "skinny_table.hpp"

const void* fpk_skinny_fp4(int var, int mt, int cj, int rw) {
  if (var == fp::kVarMx4) return fpk_detail::skinny_mx<fp::kVarMx4>(mt, cj, rw);
  if (var == fp::kVarNv4) return fpk_detail::skinny_mx<fp::kVarNv4>(mt, cj, rw);
  return nullptr;
}
