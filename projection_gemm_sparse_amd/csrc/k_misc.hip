// k_misc.hip -- the non-template kernels: the second-launch split-K finish,
// the epilogues, the block-scaled weight decoders, the streaming ceiling
// and the counter fill.  Their definitions are compiled in this unit only.
#define FP_DEFINE_MISC_KERNELS 1
#include "kernels.h"
#include "tile.hpp"
#include "epilogue.hpp"
#include "mxfp8.hpp"
#include "stream.hpp"

namespace fp {

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace fp

namespace fpk {

const void* splitk_reduce() { return reinterpret_cast<const void*>(&fp::splitk_reduce_kernel); }
const void* rmsnorm() { return reinterpret_cast<const void*>(&fp::rmsnorm_kernel); }
const void* swiglu() { return reinterpret_cast<const void*>(&fp::swiglu_kernel); }
const void* mxfp8_to_bf16() { return reinterpret_cast<const void*>(&fp::mxfp8_to_bf16_kernel); }
const void* mxfp4_to_bf16() { return reinterpret_cast<const void*>(&fp::mxfp4_to_bf16_kernel); }
const void* nvfp4_to_bf16() { return reinterpret_cast<const void*>(&fp::nvfp4_to_bf16_kernel); }
const void* stream_read() { return reinterpret_cast<const void*>(&fp::stream_read_kernel); }
const void* fill_u32() { return reinterpret_cast<const void*>(&fp::fill_u32_kernel); }
const void* stream_read_shaped(int batch) {
  switch (batch) {
    case 8: return reinterpret_cast<const void*>(&fp::stream_read_shaped_kernel<8>);
    case 16: return reinterpret_cast<const void*>(&fp::stream_read_shaped_kernel<16>);
    case 32: return reinterpret_cast<const void*>(&fp::stream_read_shaped_kernel<32>);
    default: return nullptr;
  }
}

}  // namespace fpk
