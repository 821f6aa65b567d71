// epilogue.hpp -- the steps that consume the fused projection: RMSNorm of a
// projection's output with a per-column gain (q_norm over the q_a columns
// and kv_norm over the kv columns in "tinygemm2 for the DeepSeek-V4.1
// hidden-state projections", TensorRT-LLM PR #20636, Description) and
// SwiGLU of a row-concatenated gate/up pair (dense-MLP commit of "Staircase:
// GLM-5.2 NVFP4 low-latency decode target for Rubin (TP16)", PR #20502: gate
// and up rounded to bf16 before the SwiGLU).
//
// Both read the projection as bf16, i.e. after its single rounding, so a
// fused form rounds exactly where the unfused chain (one projection launch
// per projection, then a normalisation or activation launch) does, and the
// two give bitwise equal results.
//
// SwiGLU needs only the gate and up value of the same column: a gate/up
// launch takes its rows in pairs (gate row j, up row j; the PAIRS variant of
// the projection kernels), so one row group computes both sums and writes h
// directly -- no second launch, no cross-workgroup step.
//
// RMSNorm needs every column of a token's row, and those columns are spread
// over all workgroups of the projection launch.  Finishing it inside that
// launch (the last workgroup to arrive on a counter re-reads the rows) was
// measured on MI355X to cost more than a second launch: an agent-scope
// atomic round trip alone takes ~1.5 us there, against ~1.75 us for a whole
// kernel boundary in a graph.  The fused RMSNorm is therefore the projection
// launch (all projections) followed by ONE normalisation launch over every
// normalised (projection, token) row, one wave per row.
//
// Fixed arithmetic, shared by every path:
//   RMSNorm of a row v[0..N) (N = 8 * nch, 16-byte chunks c < nch, lane l of
//   the row's wave holds chunks l, l + 64, ...):
//     q_c   = sum of squares of chunk c's 8 elements, in element order (fma)
//     a_l   = q_l + q_{l+64} + ... (ascending, c < nch)
//     total = 64-lane butterfly of a_l (transpose_reduce with one value)
//     rinv  = 1 / sqrt(total / N + eps)   (correctly rounded fp32 ops)
//     out_j = bf16_rne((v_j * rinv) * gamma_j)
//   SwiGLU: h = bf16_rne((g / (1 + exp(-g))) * u)
#pragma once

#include "common.hpp"

namespace fp {

constexpr int kNormMaxChunks = 4;   // 16-byte chunks per lane in a row
constexpr int kNormMaxN = 64 * 8 * kNormMaxChunks;  // widest normalised row

__device__ __forceinline__ float bf16_lo(unsigned u) { return u2f(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return u2f(u & 0xffff0000u); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  return (unsigned)f32_to_bf16_rne(lo) | ((unsigned)f32_to_bf16_rne(hi) << 16);
}

// Sum of squares of the 8 bf16 values of one chunk, in element order.
__device__ __forceinline__ float chunk_sumsq(const u32x4& v) {
#pragma clang fp contract(off)
  const unsigned a = v.x, b = v.y, c = v.z, d = v.w;
  float q = bf16_lo(a) * bf16_lo(a);
  q = __builtin_fmaf(bf16_hi(a), bf16_hi(a), q);
  q = __builtin_fmaf(bf16_lo(b), bf16_lo(b), q);
  q = __builtin_fmaf(bf16_hi(b), bf16_hi(b), q);
  q = __builtin_fmaf(bf16_lo(c), bf16_lo(c), q);
  q = __builtin_fmaf(bf16_hi(c), bf16_hi(c), q);
  q = __builtin_fmaf(bf16_lo(d), bf16_lo(d), q);
  q = __builtin_fmaf(bf16_hi(d), bf16_hi(d), q);
  return q;
}

// 1 / sqrt(total / N + eps) from a row's sum of squares.
__device__ __forceinline__ float rms_inv(float total, int N, float eps) {
#pragma clang fp contract(off)
  const float ms = total / (float)N;
  return 1.0f / __builtin_sqrtf(ms + eps);
}

__device__ __forceinline__ float norm_one(float v, float r, float g) {
#pragma clang fp contract(off)
  return (v * r) * g;
}

__device__ __forceinline__ u32x4 norm_chunk(const u32x4& v, const u32x4& g, float r) {
  u32x4 o;
  const unsigned v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
  const unsigned g0 = g.x, g1 = g.y, g2 = g.z, g3 = g.w;
  o.x = pack_bf16(norm_one(bf16_lo(v0), r, bf16_lo(g0)), norm_one(bf16_hi(v0), r, bf16_hi(g0)));
  o.y = pack_bf16(norm_one(bf16_lo(v1), r, bf16_lo(g1)), norm_one(bf16_hi(v1), r, bf16_hi(g1)));
  o.z = pack_bf16(norm_one(bf16_lo(v2), r, bf16_lo(g2)), norm_one(bf16_hi(v2), r, bf16_hi(g2)));
  o.w = pack_bf16(norm_one(bf16_lo(v3), r, bf16_lo(g3)), norm_one(bf16_hi(v3), r, bf16_hi(g3)));
  return o;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
#pragma clang fp contract(off)
  return (g / (1.0f + expf(-g))) * u;
}

__device__ __forceinline__ u32x4 swiglu_chunk(const u32x4& g, const u32x4& u) {
  u32x4 o;
  const unsigned g0 = g.x, g1 = g.y, g2 = g.z, g3 = g.w;
  const unsigned u0 = u.x, u1 = u.y, u2 = u.z, u3 = u.w;
  o.x = pack_bf16(silu_mul(bf16_lo(g0), bf16_lo(u0)), silu_mul(bf16_hi(g0), bf16_hi(u0)));
  o.y = pack_bf16(silu_mul(bf16_lo(g1), bf16_lo(u1)), silu_mul(bf16_hi(g1), bf16_hi(u1)));
  o.z = pack_bf16(silu_mul(bf16_lo(g2), bf16_lo(u2)), silu_mul(bf16_hi(g2), bf16_hi(u2)));
  o.w = pack_bf16(silu_mul(bf16_lo(g3), bf16_lo(u3)), silu_mul(bf16_hi(g3), bf16_hi(u3)));
  return o;
}

// Stores h[m, j] of a gate/up pair (logical row `row` = 2j, see pair_row)
// from the fp32 sums of its gate and up rows, each rounded to bf16 first, as
// the unfused chain's projection outputs are.
__device__ __forceinline__ void store_pair(unsigned char* h, int half, int row, int m,
                                           float g_sum, float u_sum) {
  typedef __attribute__((address_space(1))) uint16_t g_u16p;
  const float g = u2f((unsigned)f32_to_bf16_rne(g_sum) << 16);
  const float u = u2f((unsigned)f32_to_bf16_rne(u_sum) << 16);
  const int idx = m * half + (row >> 1);
  __hip_atomic_store((g_u16p*)(reinterpret_cast<uint16_t*>(h) + idx),
                     f32_to_bf16_rne(silu_mul(g, u)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// RMSNorm launch over the rows of up to kMaxSeg tensors: block b normalises
// row m = b % M of tensor t = b / M (y[t], gamma[t], out[t], N[t]; out[t]
// may equal y[t]: every lane reads its chunks before writing them).
struct NormTable {
  const unsigned char* y[kMaxSeg];
  const unsigned char* gamma[kMaxSeg];
  unsigned char* out[kMaxSeg];
  int32_t N[kMaxSeg];
  int32_t M;
  float eps;
};

// The epilogue kernels: defined only in the unit that compiles the non-template
// kernels (k_misc.hip), so each is emitted once.
#ifdef FP_DEFINE_MISC_KERNELS
__global__ void __launch_bounds__(64) rmsnorm_kernel(const NormTable t) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x;
  const int ti = (int)blockIdx.x / t.M;
  const int m = (int)blockIdx.x - ti * t.M;
  const int N = t.N[ti];
  const int nch = N >> 3;
  const u32x4* yr = reinterpret_cast<const u32x4*>(t.y[ti] + (size_t)m * N * 2);
  const u32x4* gr = reinterpret_cast<const u32x4*>(t.gamma[ti]);
  u32x4* orow = reinterpret_cast<u32x4*>(t.out[ti] + (size_t)m * N * 2);
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  u32x4 v[kNormMaxChunks], g[kNormMaxChunks];
#pragma unroll
  for (int j = 0; j < kNormMaxChunks; ++j) {
    const int c = lane + 64 * j;
    v[j] = c < nch ? yr[c] : zero4;
    g[j] = c < nch ? gr[c] : zero4;
  }
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormMaxChunks; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) acc += chunk_sumsq(v[j]);
  }
  float tot[1] = {acc};
  transpose_reduce<1>(tot, lane);
  const float r = rms_inv(tot[0], N, t.eps);
#pragma unroll
  for (int j = 0; j < kNormMaxChunks; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) orow[c] = norm_chunk(v[j], g[j], r);
  }
}

// h = silu(g) * u over n_chunks 16-byte chunks (bf16, dense).
__global__ void __launch_bounds__(256)
swiglu_kernel(const unsigned char* __restrict__ g, const unsigned char* __restrict__ u,
              unsigned char* __restrict__ h, int32_t n_chunks) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= n_chunks) return;
  reinterpret_cast<u32x4*>(h)[f] = swiglu_chunk(reinterpret_cast<const u32x4*>(g)[f],
                                                reinterpret_cast<const u32x4*>(u)[f]);
}

#endif  // FP_DEFINE_MISC_KERNELS

}  // namespace fp
