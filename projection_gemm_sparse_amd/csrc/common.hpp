// common.hpp -- device-side helpers shared by the projection kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Reinterpretation of one 32-bit lane value.  These take the value as a
// by-value argument on purpose: __builtin_bit_cast applied directly to an
// ext_vector element expression (v.y, v[1]) reads element 0 with this
// compiler, so every element is first copied into a scalar parameter.
__device__ __forceinline__ float u2f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f2u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ bf16x2 u2bf2(unsigned u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ bf16x8 u4bf8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

constexpr int kMaxSeg = 16;

// One projection's slice of a launch's row space: rows
// [row_begin, row_begin + rows) of the launch write output column
// (row - row_begin) of the dense [M, rows] tensor y.
struct Seg {
  unsigned char* y;
  int64_t rows;
  int64_t row_begin;
};

// The rows one launch computes.  Their weights are contiguous rows of w
// (row r at w + r * row_bytes): the fused call covers the whole
// concatenated buffer with one segment per projection, a separate call one
// projection's rows with a single segment.
struct RowSpace {
  const unsigned char* w;
  int64_t n_rows;
  int32_t n_seg;
  Seg seg[kMaxSeg];
};

constexpr int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

constexpr int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Largest workgroup a kernel is compiled for, from an estimate of the
// registers one lane needs: at most 512 VGPRs per lane and SIMD are shared by
// the waves resident on a SIMD, four SIMDs per CU.
constexpr int max_threads_for_regs(int regs) {
  int waves_per_simd = 512 / regs;
  if (waves_per_simd > 4) waves_per_simd = 4;
  if (waves_per_simd < 1) waves_per_simd = 1;
  return 256 * waves_per_simd;
}

constexpr int skinny_max_threads(int mt, int rw, int cj) {
  return max_threads_for_regs(pow2ceil(rw * mt) + 4 * rw * cj + 4 * mt * cj + 32);
}

constexpr int mfma_max_threads(int mt16, int ktw, bool xlds) {
  return max_threads_for_regs(16 * ktw + 4 * mt16 + (xlds ? 8 : 16 * ktw * mt16) + 24);
}

__device__ __forceinline__ const unsigned char* row_pointer(
    const RowSpace& rs, int64_t row, int64_t row_bytes) {
  if (row < 0 || row >= rs.n_rows) return nullptr;
  return rs.w + row * row_bytes;
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Output segments of one workgroup.  A workgroup's rows span at most a few
// segments; the two that hold its first rows are looked up once, early in
// the kernel, so the kernel-argument reads are not on the epilogue's
// critical path.  Rows in later segments (workgroups straddling several
// tiny projections) fall back to a scan of the table.
struct OutSegs {
  unsigned char* y0;
  int64_t b0, n0;
  unsigned char* y1;
  int64_t b1, n1;
};

__device__ __forceinline__ OutSegs find_out_segs(const RowSpace& rs, int64_t first_row) {
  OutSegs o;
  o.y0 = nullptr; o.b0 = 0; o.n0 = 0;
  o.y1 = nullptr; o.b1 = 0; o.n1 = 0;
  int i = 0;
  while (i < rs.n_seg && first_row >= rs.seg[i].row_begin + rs.seg[i].rows) ++i;
  if (i < rs.n_seg) {
    o.y0 = rs.seg[i].y; o.b0 = rs.seg[i].row_begin; o.n0 = rs.seg[i].rows;
  }
  if (i + 1 < rs.n_seg) {
    o.y1 = rs.seg[i + 1].y; o.b1 = rs.seg[i + 1].row_begin; o.n1 = rs.seg[i + 1].rows;
  }
  return o;
}

// Stores output element (launch row `row`, token m): y_i[m, row - row_begin]
// of the dense [M, rows] tensor of the segment that holds the row.
template <bool BF16>
__device__ __forceinline__ void store_out(const RowSpace& rs, const OutSegs& os,
                                          int64_t row, int m, float v) {
  unsigned char* y = nullptr;
  int64_t idx = 0;
  if (row >= os.b0 && row < os.b0 + os.n0) {
    y = os.y0;
    idx = (int64_t)m * os.n0 + (row - os.b0);
  } else if (row >= os.b1 && row < os.b1 + os.n1) {
    y = os.y1;
    idx = (int64_t)m * os.n1 + (row - os.b1);
  } else {
    for (int i = 0; i < rs.n_seg; ++i) {
      const int64_t b = rs.seg[i].row_begin;
      const int64_t n = rs.seg[i].rows;
      if (row >= b && row < b + n) {
        y = rs.seg[i].y;
        idx = (int64_t)m * n + (row - b);
      }
    }
  }
  if (y == nullptr) return;
  // agent-coherent (sc1) stores: the line is written through instead of
  // left dirty in this XCD's L2, which shortens the end-of-kernel writeback
  if constexpr (BF16) {
    __hip_atomic_store(reinterpret_cast<uint16_t*>(y) + idx, f32_to_bf16_rne(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store(reinterpret_cast<float*>(y) + idx, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Multiply-accumulate of one 16-byte chunk of a weight row with the same
// chunk of an activation row, into one fp32 partial sum, in element order.
// bf16: four v_dot2 (pairs of exact bf16 products added into fp32);
// fp32: four fused multiply-adds.
template <bool BF16>
__device__ __forceinline__ float dot_chunk(const u32x4& w, const u32x4& x,
                                           float acc) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(u2bf2(w.x), u2bf2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(u2bf2(w.y), u2bf2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(u2bf2(w.z), u2bf2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(u2bf2(w.w), u2bf2(x.w), acc, false);
  } else {
    acc = __builtin_fmaf(u2f(w.x), u2f(x.x), acc);
    acc = __builtin_fmaf(u2f(w.y), u2f(x.y), acc);
    acc = __builtin_fmaf(u2f(w.z), u2f(x.z), acc);
    acc = __builtin_fmaf(u2f(w.w), u2f(x.w), acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Deterministic wave reduction ("transpose reduce").
//
// Each of the 64 lanes holds C partial sums v[0..C) of C different outputs;
// the wave must produce, for every output, the sum over all 64 lanes.  Six
// pairing steps combine lane l with a partner that differs in one lane-index
// bit (bit 5: lanes l and l^32 via v_permlane32_swap; bit 4: l and l^16 via
// v_permlane16_swap; bit 3: l and 15-l inside a 16-lane row via DPP
// row_mirror; bit 2: l and 7-l via row_half_mirror; bits 1 and 0: quad
// permutations).  While two or more values remain, a step pairs value i
// with value i + C/2: lanes whose bit is 0 keep the sum of value i, lanes
// whose bit is 1 the sum of value i + C/2, so the number of values per lane
// halves and no lane does redundant work.  With one value left the step is
// an ordinary butterfly.  Every output is therefore summed by the same
// binary tree over lanes, whatever C is: the result of an output does not
// depend on how many other outputs share the wave.
//
// Final placement, for C = 2^p values: if C >= 64 lane l holds
// values q + (C/64) * l for q < C/64; otherwise lane l holds value
// l >> (6 - p) (replicated over 2^(6-p) consecutive lanes).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return u2f((unsigned)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xF, 0xF, false));
}

// v_permlane32_swap / v_permlane16_swap of (a, b) followed by the sum of the
// two swapped registers.
__device__ __forceinline__ float swap32_add(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(a), f2u(b), false, false);
  const unsigned r0 = r[0];
  const unsigned r1 = r[1];
  return u2f(r0) + u2f(r1);
}

__device__ __forceinline__ float swap16_add(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(f2u(a), f2u(b), false, false);
  const unsigned r0 = r[0];
  const unsigned r1 = r[1];
  return u2f(r0) + u2f(r1);
}

constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]

template <int C>
__device__ __forceinline__ void tr_step_swap32(float* v) {
  if constexpr (C >= 2) {
#pragma unroll
    for (int i = 0; i < C / 2; ++i) v[i] = swap32_add(v[i], v[i + C / 2]);
  } else {
    v[0] = swap32_add(v[0], v[0]);
  }
}

template <int C>
__device__ __forceinline__ void tr_step_swap16(float* v) {
  if constexpr (C >= 2) {
#pragma unroll
    for (int i = 0; i < C / 2; ++i) v[i] = swap16_add(v[i], v[i + C / 2]);
  } else {
    v[0] = swap16_add(v[0], v[0]);
  }
}

template <int C, int CTRL, int BIT>
__device__ __forceinline__ void tr_step_dpp(float* v, int lane) {
  if constexpr (C >= 2) {
    const bool up = (lane >> BIT) & 1;
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      const float a = v[i], b = v[i + C / 2];
      const float send = up ? a : b;
      const float keep = up ? b : a;
      v[i] = keep + dpp_f32<CTRL>(send);
    }
  } else {
    v[0] = v[0] + dpp_f32<CTRL>(v[0]);
  }
}

template <int C>
__device__ __forceinline__ void transpose_reduce(float* v, int lane) {
  static_assert((C & (C - 1)) == 0, "power-of-two value count");
  constexpr int C0 = C;
  constexpr int C1 = C0 > 1 ? C0 / 2 : 1;
  constexpr int C2 = C1 > 1 ? C1 / 2 : 1;
  constexpr int C3 = C2 > 1 ? C2 / 2 : 1;
  constexpr int C4 = C3 > 1 ? C3 / 2 : 1;
  constexpr int C5 = C4 > 1 ? C4 / 2 : 1;
  tr_step_swap32<C0>(v);
  tr_step_swap16<C1>(v);
  tr_step_dpp<C2, kDppRowMirror, 3>(v, lane);
  tr_step_dpp<C3, kDppRowHalfMirror, 2>(v, lane);
  tr_step_dpp<C4, kDppQuadXor2, 1>(v, lane);
  tr_step_dpp<C5, kDppQuadXor1, 0>(v, lane);
}

// ---------------------------------------------------------------------------
// Split-K partial sums and their finish inside the same launch.
//
// Each of the S workgroups of row block rb writes its fp32 partial sums to
// partial[s][row][m] with agent-coherent stores (sc1: written through to the
// point of coherence shared by all XCDs instead of staying dirty in this
// XCD's L2), waits until they are acknowledged, and then arrives on
// counters[rb].  The workgroup that arrives last reads the S partials with
// agent-coherent loads, adds them in slice order s = 0, 1, ..., S-1, stores
// the outputs and resets the counter to zero, so the next call (or graph
// replay) needs no host action.  Because every partial store and load is
// agent-coherent, no L2 writeback or invalidation (what an agent-scope
// fence would cost per workgroup) is needed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Must be called by every thread of the workgroup (it has barriers).
template <bool BF16>
__device__ __forceinline__ void splitk_finish(const RowSpace& rs,
                                              const float* partial,
                                              uint32_t* counters, int rb,
                                              int S, int64_t row_base,
                                              int64_t R, int M, int* flag) {
  // this thread's partial stores are complete (vmcnt = 0; expcnt and
  // lgkmcnt left at their maximum) before the workgroup arrives
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counters + rb, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (unsigned)(S - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  const int64_t n_rows = rs.n_rows;
  const int64_t rows_here = (n_rows - row_base) < R ? (n_rows - row_base) : R;
  const int64_t n_fin = rows_here * M;
  const int64_t sstride = n_rows * M;
  const OutSegs os = find_out_segs(rs, row_base);
  for (int64_t t = threadIdx.x; t < n_fin; t += blockDim.x) {
    const int64_t rr = t / M;
    const int m = (int)(t - rr * M);
    const int64_t row = row_base + rr;
    const float* pp = partial + row * M + m;
    float sum = load_partial(pp);
    for (int ss = 1; ss < S; ++ss) sum += load_partial(pp + ss * sstride);
    store_out<BF16>(rs, os, row, m, sum);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(counters + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace fp
