// kernels.h -- the kernel instantiations of libfusedproj, one getter per
// kernel family.  Each family is compiled in its own translation unit
// (k_*.hip), so that every instantiation is emitted exactly once and the
// units build in parallel; the host code (api.hip) only takes the kernel
// addresses these return and launches them.  A getter returns nullptr for a
// configuration that has no compiled instantiation.
#pragma once

#include <stdint.h>

namespace fpk {

// Weight-streaming vector-ALU kernel (skinny.hpp): bf16 or fp32 operands and
// outputs, MT-token bucket (1, 2, 4, 8), CJ chunks per lane, RW rows per wave.
const void* skinny(bool bf16, int mt, int cj, int rw);
// The same kernel over gate/up row pairs with the SwiGLU epilogue (bf16).
const void* skinny_pairs(int mt, int cj, int rw);
// bf16 operands, fp32 outputs (router logits), MT up to 16.
const void* skinny_f32out(int mt, int cj, int rw);
// Block-scaled weights: var = fp::kVarMx8, kVarMx4 or kVarNv4.
const void* skinny_mx(int var, int mt, int cj, int rw);

// Small-M matrix-core kernel (smfma.hpp): KT steps per wave; mt 8, 16 or
// 24 (one to three token halves); pairs = gate/up SwiGLU form; M picks the
// load order of the two-half forms; tt row tiles per wave (2: not gate/up,
// at most two halves).
const void* smfma(int kt, bool pairs, int mt, int64_t M, int tt = 1);
// Block-scaled weights on the small-M matrix-core kernel: dtype FP_MXFP8,
// FP_MXFP4 or FP_NVFP4; mh token halves (1 or 2).
const void* smfma_mx(int32_t dtype, int mh, int kt);

// LDS tile kernel (tile.hpp): 16 * mt16 token slots, nw row tiles, compiled
// slice bound `per` (8, 10, 16, 20, 40 k steps).
const void* tile(int mt16, int nw, int per);
// Ring tile kernel (tile_ring.hpp): 16 * mt16 token slots, `stages` buffers.
const void* ring(int mt16, int stages);
// Weight-resident tile kernel (tile_wres.hpp): 16 * mt16 token slots
// (mt16 2, 4, 8 or 16).
const void* wres(int mt16);
// Second-launch finish of a split tile launch.
const void* splitk_reduce();

// Epilogue, decode and measurement kernels.
const void* rmsnorm();
const void* swiglu();
const void* mxfp8_to_bf16();
const void* mxfp4_to_bf16();
const void* nvfp4_to_bf16();
const void* stream_read();
const void* fill_u32();
// The streaming kernel with its launch shape as a parameter: BATCH loads in
// flight per lane (8, 16 or 32).
const void* stream_read_shaped(int batch);

}  // namespace fpk
