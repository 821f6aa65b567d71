// epilogue.hpp -- the steps that consume the fused projection, applied in
// the same launch: RMSNorm of a projection's output with a per-column gain
// (q_norm over the q_a columns and kv_norm over the kv columns in "tinygemm2
// for the DeepSeek-V4.1 hidden-state projections", TensorRT-LLM PR #20636,
// Description) and SwiGLU of a row-concatenated gate/up pair (dense-MLP
// commit of "Staircase: GLM-5.2 NVFP4 low-latency decode target for Rubin
// (TP16)", PR #20502: gate and up rounded to bf16 before the SwiGLU).
//
// Both read the projection as bf16, i.e. after its single rounding, so the
// fused chain rounds exactly where the unfused one (projection kernel, then
// a normalisation or activation kernel) does.
//
// In-launch finish.  A normalisation needs every column of a token's row,
// and those rows are spread over all workgroups of the projection launch.
// Each workgroup therefore stages its bf16 outputs in the workspace with
// agent-coherent stores, waits for their acknowledgement and arrives on a
// counter; the workgroup that arrives last reads the staged outputs back
// (agent-coherent 16-byte loads straight into LDS), applies the epilogue,
// writes the final tensors and resets the counter to zero for the next call
// (graph replays need no host action).  The gate/up pair of SwiGLU lives in
// two segments of the same launch and is finished the same way.
//
// Fixed arithmetic, shared with the standalone kernels below so that the
// fused call and the unfused chain give bitwise equal results:
//   RMSNorm of a row v[0..N) (N = 8 * nch, 16-byte chunks c < nch):
//     q_c   = sum of squares of chunk c's 8 elements, in element order (fma)
//     lane l of a wave: a_l = q_l + q_{l+64} + ... (ascending, c < nch)
//     total = 64-lane butterfly of a_l (transpose_reduce with one value)
//     rinv  = 1 / sqrt(total / N + eps)   (correctly rounded fp32 ops)
//     out_j = bf16_rne((v_j * rinv) * gamma_j)
//   SwiGLU: h = bf16_rne((g / (1 + exp(-g))) * u)
#pragma once

#include "common.hpp"

namespace fp {

constexpr int kEpiMaxM = 8;         // token counts the epilogues serve
constexpr int kNormMaxChunks = 4;   // 16-byte chunks per lane in a row
constexpr int kNormMaxN = 64 * 8 * kNormMaxChunks;  // widest normalised row
constexpr int kAuxSc1 = 16;         // buffer cache policy: agent-coherent

typedef __attribute__((address_space(3))) void epi_lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t epi_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           0x00020000);
}

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

// ---------------------------------------------------------------------------
// Row sum of a wave: lane l adds q[l], q[l + 64], ... (c < nch) in ascending
// order, then the 64 lanes are combined by the fixed butterfly; every lane
// returns the same total.
__device__ __forceinline__ float wave_row_total(const float* q, int nch, int lane) {
#pragma clang fp contract(off)
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kNormMaxChunks; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) acc += q[c];
  }
  float v[1] = {acc};
  transpose_reduce<1>(v, lane);
  return v[0];
}


__host__ __device__ constexpr uint32_t round64_slots(uint32_t n) { return (n + 63u) & ~63u; }

// LDS bytes of the in-launch finish (host and device agree on this layout):
//   [0, 16)   arrival flag
//   RMSNorm:  per normalised segment i (in segment order) the staged rows,
//             round64(M * nch_i) 16-byte slots; then per segment the gain,
//             round64(nch_i) slots; then the M * nch_i chunk sums (fp32);
//             then one row factor per (segment, token)
//   SwiGLU:   the staged gate rows, round64(M * nch) slots, then the up rows
__host__ __device__ inline uint32_t epi_lds_bytes(int mode, int M, int n_seg,
                                                  const int32_t* begin,
                                                  const bool* normed) {
  uint32_t b = 16;
  if (mode == kEpiSwiglu) {
    const uint32_t nch = (uint32_t)(begin[1] - begin[0]) >> 3;
    return b + 2u * round64_slots((uint32_t)M * nch) * 16u;
  }
  uint32_t ys = 0, gs = 0, qs = 0, rows = 0;
  for (int i = 0; i < n_seg; ++i) {
    if (!normed[i]) continue;
    const uint32_t nch = (uint32_t)(begin[i + 1] - begin[i]) >> 3;
    ys += round64_slots((uint32_t)M * nch) * 16u;
    gs += round64_slots(nch) * 16u;
    qs += (uint32_t)M * nch * 4u;
    rows += (uint32_t)M;
  }
  return b + ys + gs + ((qs + 15u) & ~15u) + rows * 4u;
}

// The in-launch finish.  Called by every thread of every workgroup after its
// output stores (it has barriers).  counter / n_blocks come from the Epi
// argument, read by the caller at its start.
__device__ __forceinline__ void epi_finish(const OutTable& tab, const Epi& e, uint32_t* counter,
                                        int n_blocks, int M, int nthreads,
                                        unsigned char* lds) {
  typedef __attribute__((address_space(1))) uint32_t gu32e;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = nthreads >> 6;
  int* flag = reinterpret_cast<int*>(lds);
  // this thread's staged stores are acknowledged before the workgroup arrives
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add((gu32e*)counter, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (unsigned)(n_blocks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  const int mode = e.mode;
  const int n_seg = tab.n_seg;

  if (mode == kEpiSwiglu) {
    const int nch = (tab.begin[1] - tab.begin[0]) >> 3;
    const int cnt = M * nch;
    const uint32_t greg = 16;
    const uint32_t ureg = greg + round64_slots((uint32_t)cnt) * 16u;
    const __amdgpu_buffer_rsrc_t rg = epi_rsrc(tab.y[0], (uint32_t)cnt * 16u);
    const __amdgpu_buffer_rsrc_t ru = epi_rsrc(tab.y[1], (uint32_t)cnt * 16u);
    for (int base = wave * 64; base < cnt; base += nthreads) {
      const int f = base + lane;
      const uint32_t off = f < cnt ? (uint32_t)f * 16u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rg, (epi_lds_void*)(lds + greg + (uint32_t)base * 16u), 16, off, 0, 0, kAuxSc1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ru, (epi_lds_void*)(lds + ureg + (uint32_t)base * 16u), 16, off, 0, 0, kAuxSc1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    const u32x4* gl = reinterpret_cast<const u32x4*>(lds + greg);
    const u32x4* ul = reinterpret_cast<const u32x4*>(lds + ureg);
    u32x4* h = reinterpret_cast<u32x4*>(e.out[0]);
    for (int f = tid; f < cnt; f += nthreads) h[f] = swiglu_chunk(gl[f], ul[f]);
  } else {
    // 1. staged rows and gains of every normalised segment -> LDS
    uint32_t yo = 16;
    for (int i = 0; i < n_seg; ++i) {
      if (e.gamma[i] == nullptr) continue;
      const int nch = (tab.begin[i + 1] - tab.begin[i]) >> 3;
      const int cnt = M * nch;
      const __amdgpu_buffer_rsrc_t ry = epi_rsrc(tab.y[i], (uint32_t)cnt * 16u);
      for (int base = wave * 64; base < cnt; base += nthreads) {
        const int f = base + lane;
        const uint32_t off = f < cnt ? (uint32_t)f * 16u : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ry, (epi_lds_void*)(lds + yo + (uint32_t)base * 16u), 16, off, 0, 0, kAuxSc1);
      }
      yo += round64_slots((uint32_t)cnt) * 16u;
    }
    const uint32_t gstart = yo;
    uint32_t go = gstart;
    for (int i = 0; i < n_seg; ++i) {
      if (e.gamma[i] == nullptr) continue;
      const int nch = (tab.begin[i + 1] - tab.begin[i]) >> 3;
      const __amdgpu_buffer_rsrc_t rgm = epi_rsrc(e.gamma[i], (uint32_t)nch * 16u);
      for (int base = wave * 64; base < nch; base += nthreads) {
        const int f = base + lane;
        const uint32_t off = f < nch ? (uint32_t)f * 16u : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rgm, (epi_lds_void*)(lds + go + (uint32_t)base * 16u), 16, off, 0, 0, 0);
      }
      go += round64_slots((uint32_t)nch) * 16u;
    }
    const uint32_t qstart = go;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // 2. chunk sums of squares
    float* ql = reinterpret_cast<float*>(lds + qstart);
    yo = 16;
    uint32_t qo = 0;
    for (int i = 0; i < n_seg; ++i) {
      if (e.gamma[i] == nullptr) continue;
      const int nch = (tab.begin[i + 1] - tab.begin[i]) >> 3;
      const int cnt = M * nch;
      const u32x4* yl = reinterpret_cast<const u32x4*>(lds + yo);
      for (int f = tid; f < cnt; f += nthreads) ql[qo + f] = chunk_sumsq(yl[f]);
      yo += round64_slots((uint32_t)cnt) * 16u;
      qo += (uint32_t)cnt;
    }
    const uint32_t rstart = qstart + ((qo * 4u + 15u) & ~15u);
    float* rl = reinterpret_cast<float*>(lds + rstart);
    __syncthreads();
    // 3. one row factor per (segment, token), one wave per row
    qo = 0;
    uint32_t ro = 0;
    for (int i = 0; i < n_seg; ++i) {
      if (e.gamma[i] == nullptr) continue;
      const int N = tab.begin[i + 1] - tab.begin[i];
      const int nch = N >> 3;
      for (int m = wave; m < M; m += nw) {
        const float total = wave_row_total(ql + qo + (uint32_t)(m * nch), nch, lane);
        const float r = rms_inv(total, N, e.eps);
        if (lane == 0) rl[ro + m] = r;
      }
      qo += (uint32_t)(M * nch);
      ro += (uint32_t)M;
    }
    __syncthreads();
    // 4. normalised rows out
    yo = 16;
    go = gstart;
    ro = 0;
    for (int i = 0; i < n_seg; ++i) {
      if (e.gamma[i] == nullptr) continue;
      const int nch = (tab.begin[i + 1] - tab.begin[i]) >> 3;
      const int cnt = M * nch;
      const u32x4* yl = reinterpret_cast<const u32x4*>(lds + yo);
      const u32x4* gl = reinterpret_cast<const u32x4*>(lds + go);
      u32x4* o = reinterpret_cast<u32x4*>(e.out[i]);
      for (int f = tid; f < cnt; f += nthreads) {
        const int m = f / nch;
        const int c = f - m * nch;
        o[f] = norm_chunk(yl[f], gl[c], rl[ro + m]);
      }
      yo += round64_slots((uint32_t)cnt) * 16u;
      go += round64_slots((uint32_t)nch) * 16u;
      ro += (uint32_t)M;
    }
  }
  if (tid == 0) {
    __hip_atomic_store((gu32e*)counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Standalone kernels: the unfused chain's second step, with the arithmetic
// above (bitwise equal to the in-launch finish).

// RMSNorm of y[M, N] (bf16, dense) with gain gamma[N]: one wave per row.
__global__ void __launch_bounds__(64)
rmsnorm_kernel(const unsigned char* __restrict__ y, const unsigned char* __restrict__ gamma,
               unsigned char* __restrict__ out, int32_t N, float eps) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x;
  const int m = blockIdx.x;
  const int nch = N >> 3;
  const u32x4* yr = reinterpret_cast<const u32x4*>(y + (size_t)m * N * 2);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4* orow = reinterpret_cast<u32x4*>(out + (size_t)m * N * 2);
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
  float t[1] = {acc};
  transpose_reduce<1>(t, lane);
  const float r = rms_inv(t[0], N, eps);
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

}  // namespace fp
