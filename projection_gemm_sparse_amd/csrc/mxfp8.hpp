// mxfp8.hpp -- dequantisation of MXFP8, MXFP4 and NVFP4 weight rows to bf16.
//
// The pages name MXFP8 projections for the DeepSeek-V4.1 wq_a / wkv weights
// ("tinygemm2 for the DeepSeek-V4.1 hidden-state projections", TensorRT-LLM
// PR #20636, Description) without defining the encoding; the reading is the
// open microscaling format: E4M3 codes, one E8M0 scale per 32 consecutive
// elements along K.  Storage (this library's layout): a row is its K codes
// followed by its K/32 scales.  The projection kernels decode on the fly
// (kVarMx8); this kernel writes the decoded weights out, for a caller that
// needs them as bf16 (a fallback linear layer) and to check the decode.
#pragma once

#include "common.hpp"

namespace fp {

// The decode kernels: defined only in the unit that compiles the non-template
// kernels (k_misc.hip), so each is emitted once.
#ifdef FP_DEFINE_MISC_KERNELS
// Thread t decodes code chunk t (16 codes) of the rows: row t / kc, chunk
// t % kc (kc = K / 16), to 32 bytes of bf16 at out[row, 16 * chunk ...].
__global__ void __launch_bounds__(256)
mxfp8_to_bf16_kernel(const unsigned char* __restrict__ w, unsigned char* __restrict__ out,
                     int32_t kc, int64_t n_chunks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_chunks) return;
  const int64_t row = t / kc;
  const int c = (int)(t - row * kc);
  const uint64_t row_bytes = (uint64_t)kc * 16u + ((uint32_t)kc >> 1);
  const unsigned char* wrow = w + (uint64_t)row * row_bytes;
  const u32x4 q = *reinterpret_cast<const u32x4*>(wrow + (uint64_t)c * 16u);
  const uint32_t sb = wrow[(uint64_t)kc * 16u + (uint32_t)(c >> 1)];
  const float sc = u2f(sb != 0u ? sb << 23 : 0x00400000u);
  u32x4 o0, o1;
  o0.x = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.x, sc, false));
  o0.y = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.x, sc, true));
  o0.z = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.y, sc, false));
  o0.w = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.y, sc, true));
  o1.x = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.z, sc, false));
  o1.y = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.z, sc, true));
  o1.z = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.w, sc, false));
  o1.w = __builtin_bit_cast(unsigned, decode_e4m3_pair(q.w, sc, true));
  u32x4* orow = reinterpret_cast<u32x4*>(out + ((uint64_t)row * kc * 16u + (uint64_t)c * 16u) * 2u);
  orow[0] = o0;
  orow[1] = o1;
}

// MXFP4 rows (K/2 code bytes, low nibble first, then K/32 scales): thread t
// decodes code chunk t (16 bytes = 32 codes, one block) of row t / kc, kc =
// K / 32, to 64 bytes of bf16.
__global__ void __launch_bounds__(256)
mxfp4_to_bf16_kernel(const unsigned char* __restrict__ w, unsigned char* __restrict__ out,
                     int32_t kc, int64_t n_chunks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_chunks) return;
  const int64_t row = t / kc;
  const int c = (int)(t - row * kc);
  const uint64_t row_bytes = (uint64_t)kc * 16u + (uint32_t)kc;
  const unsigned char* wrow = w + (uint64_t)row * row_bytes;
  const u32x4 q = *reinterpret_cast<const u32x4*>(wrow + (uint64_t)c * 16u);
  const uint32_t sb = wrow[(uint64_t)kc * 16u + (uint32_t)c];
  const float sc = u2f(sb != 0u ? sb << 23 : 0x00400000u);
  u32x4* orow = reinterpret_cast<u32x4*>(out + ((uint64_t)row * kc * 32u + (uint64_t)c * 32u) * 2u);
  const unsigned qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 o;
    o.x = __builtin_bit_cast(unsigned, decode_e2m1_pair<0>(qs[i], sc));
    o.y = __builtin_bit_cast(unsigned, decode_e2m1_pair<1>(qs[i], sc));
    o.z = __builtin_bit_cast(unsigned, decode_e2m1_pair<2>(qs[i], sc));
    o.w = __builtin_bit_cast(unsigned, decode_e2m1_pair<3>(qs[i], sc));
    orow[i] = o;
  }
}

// NVFP4 rows (K/2 code bytes, low nibble first, then K/16 E4M3 scales):
// thread t decodes code chunk t (16 bytes, 32 codes, two 16-element
// blocks) of the rows to 64 bytes of bf16: each element e2m1 * e4m3 (exact
// in fp32) times the tensor scale g in fp32, rounded once to bf16.
__global__ void __launch_bounds__(256)
nvfp4_to_bf16_kernel(const unsigned char* __restrict__ w, unsigned char* __restrict__ out,
                     int32_t kc, int64_t n_chunks, float g) {
#pragma clang fp contract(off)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_chunks) return;
  const int64_t row = t / kc;
  const int c = (int)(t - row * kc);
  const uint64_t row_bytes = (uint64_t)kc * 16u + (uint32_t)kc * 2u;
  const unsigned char* wrow = w + (uint64_t)row * row_bytes;
  const u32x4 q = *reinterpret_cast<const u32x4*>(wrow + (uint64_t)c * 16u);
  const unsigned sb = *reinterpret_cast<const uint16_t*>(wrow + (uint64_t)kc * 16u + 2u * c);
  const float sc[2] = {e4m3_to_f32(sb & 0xffu), e4m3_to_f32(sb >> 8)};
  u32x4* orow = reinterpret_cast<u32x4*>(out + ((uint64_t)row * kc * 32u + (uint64_t)c * 32u) * 2u);
  const unsigned qs[4] = {q.x, q.y, q.z, q.w};
  auto scaled = [&](bf16x2 d) {
    const unsigned u = __builtin_bit_cast(unsigned, d);
    const float lo = u2f(u << 16) * g, hi = u2f(u & 0xffff0000u) * g;
    return (unsigned)f32_to_bf16_rne(lo) | ((unsigned)f32_to_bf16_rne(hi) << 16);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = sc[i >> 1];  // 8 codes per word: words 0, 1 in block 0
    u32x4 o;
    o.x = scaled(decode_e2m1_pair_nv<0>(qs[i], s));
    o.y = scaled(decode_e2m1_pair_nv<1>(qs[i], s));
    o.z = scaled(decode_e2m1_pair_nv<2>(qs[i], s));
    o.w = scaled(decode_e2m1_pair_nv<3>(qs[i], s));
    orow[i] = o;
  }
}

#endif  // FP_DEFINE_MISC_KERNELS

}  // namespace fp
