// common.hpp -- device-side helpers shared by the projection kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
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
// Most waves that split one row's K range inside a workgroup.
constexpr int kMaxWaveParts = 16;

// Output table of a launch.  The launch covers rows [0, n_rows) of its
// weight buffer; projection (segment) i owns rows [begin[i], begin[i+1])
// and row r of it writes column r - begin[i] of the dense [M, N_i] tensor
// y[i] (N_i = begin[i+1] - begin[i]).  Unused entries repeat n_rows.
struct OutTable {
  unsigned char* y[kMaxSeg];
  int32_t begin[kMaxSeg + 1];
  int32_t n_seg;
  float tscale[kMaxSeg];  // NVFP4: each segment's fp32 tensor scale
};

// Trailing kernel argument (not preloaded): the output table for launches
// with more than two segments, and the split-K workspace.
struct Tail {
  OutTable out;
  float* partial;      // S > 1: [S][n_rows][M] (vector-ALU), [S][M][n_rows rounded to 4] (tile kernels)
  uint32_t* counters;  // one per row block when S > 1, zero between calls
};

// Kernel variants (a compile-time parameter of the small-M kernels).
constexpr int kVarPlain = 0;
constexpr int kVarPairs = 1;
constexpr int kVarF32Out = 2;
constexpr int kVarMx8 = 3;
constexpr int kVarMx4 = 4;
constexpr int kVarNv4 = 5;

// Gate/up launches (the PAIRS variant of the kernels): the launch's n_rows =
// 2N logical rows interleave the two halves of the weight buffer -- logical
// row 2j is gate row j, 2j + 1 is up row j (buffer row N + j, N = split) --
// so one row group holds both rows of a pair and writes
// h[m, j] = silu(g) * u (g and u rounded to bf16 first) to y0, a dense
// [M, N] tensor.  Buffer row of a logical row:
__device__ __forceinline__ int pair_row(int row, int half) {
  return (row >> 1) + (row & 1) * half;
}

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

// MXFP8 / MXFP4 weights (kVarMx8, kVarMx4) hold 8- or 4-byte code units, a
// scale per unit and four decoded pairs.
constexpr int skinny_max_threads(int mt, int rw, int cj, int var = kVarPlain) {
  return var == kVarMx8 || var == kVarMx4 || var == kVarNv4
             ? max_threads_for_regs(pow2ceil(rw * mt) + 3 * rw * cj + 4 * mt * cj + 36)
             : max_threads_for_regs(pow2ceil(rw * mt) + 4 * rw * cj + 4 * mt * cj + 32);
}


// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Where a workgroup's outputs go.  Two segments are resolved per workgroup
// before its weights land: rows [b0, b1) write y0 (width b1 - b0) and rows
// [b1, e1) write y1 (width e1 - b1).  A launch of one or two projections
// passes y0, y1 and the split row as preloaded kernel arguments (no memory
// read at all).  A launch of more projections passes split < 0; the
// workgroup then reads the row boundaries from the output table, picks the
// segment of its first row and the next one, and reads their pointers --
// all at its start, pinned there so that the scalar loads are not sunk
// towards the end of the kernel, where a kernel-argument read would put a
// memory round trip on the critical path.  Rows past those two segments (a
// workgroup straddling a projection shorter than itself) are resolved from
// the table when stored.
struct OutMap {
  unsigned char* y0;
  unsigned char* y1;
  int b0, b1, e1;
  // segments to search for a row past e1 (0 with two segments: there is
  // none; read here, while the loads are in flight, so that no
  // kernel-argument load is left for the stores)
  int n_seg;
  // tensor scales of y0's and y1's segments (SCALED: NVFP4 weights; 1
  // otherwise), read and pinned at the start for the same reason
  float ts0, ts1;
};

template <bool SCALED = false>
__device__ __forceinline__ OutMap make_out_map(unsigned char* y0, unsigned char* y1, int split,
                                               int n_rows, const OutTable& tab, int first_row) {
  OutMap o;
  o.ts0 = 1.0f;
  o.ts1 = 1.0f;
  if (split >= 0) {
    o.y0 = y0;
    o.y1 = y1;
    o.b0 = 0;
    o.b1 = split;
    o.e1 = n_rows;
    o.n_seg = 0;
    if constexpr (SCALED) {
      o.ts0 = tab.tscale[0];
      o.ts1 = tab.tscale[1];
      asm volatile("" : "+s"(o.ts0), "+s"(o.ts1));
    }
    return o;
  }
  const int n_seg = tab.n_seg;
  o.n_seg = n_seg;
  int i0 = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i) i0 = (i < n_seg && first_row >= tab.begin[i]) ? i : i0;
  const int i1 = i0 + 1 < kMaxSeg ? i0 + 1 : kMaxSeg - 1;
  const int i2 = i0 + 2 < kMaxSeg ? i0 + 2 : kMaxSeg;
  o.y0 = tab.y[i0];
  o.y1 = tab.y[i1];
  o.b0 = tab.begin[i0];
  o.b1 = tab.begin[i0 + 1];
  o.e1 = tab.begin[i2];
  if constexpr (SCALED) {
    o.ts0 = tab.tscale[i0];
    o.ts1 = tab.tscale[i1];
    asm volatile("" : "+s"(o.ts0), "+s"(o.ts1));
  }
  asm volatile("" : "+s"(o.y0), "+s"(o.y1), "+s"(o.b0), "+s"(o.b1), "+s"(o.e1), "+s"(o.n_seg));
  return o;
}

// Stores output element (launch row `row`, token m) rounded once to the
// output type (bf16: round to nearest even).  Agent-coherent (sc1) stores:
// the line is written through instead of left dirty in this XCD's L2.
// SCALED (NVFP4): the fp32 sum is first multiplied by its segment's tensor
// scale (one fp32 multiply, then the single rounding).
template <bool BF16, bool SCALED = false>
__device__ __forceinline__ void store_y(const OutMap& o, const OutTable& tab, int row, int m,
                                        float v) {
  unsigned char* y;
  int idx;
  float ts = 1.0f;
  if (row < o.e1) {
    // the workgroup's first two segments: selects, no branch
    const bool first = row < o.b1;
    y = first ? o.y0 : o.y1;
    const int b = first ? o.b0 : o.b1;
    const int n = first ? o.b1 - o.b0 : o.e1 - o.b1;
    idx = m * n + (row - b);
    ts = first ? o.ts0 : o.ts1;
  } else {
    // a third segment inside the workgroup (more than two projections only)
    y = nullptr;
    idx = 0;
    for (int i = 0; i < o.n_seg; ++i) {
      if (row >= tab.begin[i] && row < tab.begin[i + 1]) {
        y = tab.y[i];
        idx = m * (tab.begin[i + 1] - tab.begin[i]) + (row - tab.begin[i]);
        ts = tab.tscale[i];
      }
    }
    if (y == nullptr) return;
  }
  if constexpr (SCALED) {
#pragma clang fp contract(off)
    v = v * ts;
  }
  // global (not generic) address space: a global_store, no aperture check
  typedef __attribute__((address_space(1))) uint16_t g_u16;
  typedef __attribute__((address_space(1))) float g_f32;
  if constexpr (BF16) {
    __hip_atomic_store((g_u16*)(reinterpret_cast<uint16_t*>(y) + idx), f32_to_bf16_rne(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store((g_f32*)(reinterpret_cast<float*>(y) + idx), v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// bf16 outputs of four consecutive rows row .. row + 3 of token m (each
// rounded once, as store_y): one 8-byte store where the four rows lie below
// n_rows in one of the map's first two segments at an 8-byte aligned
// address -- the outputs of one token are contiguous in its projection's
// [M, N_i] tensor, so a wave's quads of consecutive rows write whole lines --
// else one store_y per row below n_rows.
__device__ __forceinline__ void store_y4(const OutMap& o, const OutTable& tab, int row, int m,
                                         f32x4 v, int n_rows) {
  typedef __attribute__((address_space(1))) uint64_t g_u64;
  if (row + 3 < n_rows && row + 3 < o.e1 && (row + 3 < o.b1 || row >= o.b1)) {
    const bool first = row < o.b1;
    const int b = first ? o.b0 : o.b1;
    const int n = first ? o.b1 - o.b0 : o.e1 - o.b1;
    uint16_t* y = reinterpret_cast<uint16_t*>(first ? o.y0 : o.y1) + (m * n + (row - b));
    if ((reinterpret_cast<uintptr_t>(y) & 7) == 0) {
      const uint64_t q = (uint64_t)f32_to_bf16_rne(v[0]) |
                         ((uint64_t)f32_to_bf16_rne(v[1]) << 16) |
                         ((uint64_t)f32_to_bf16_rne(v[2]) << 32) |
                         ((uint64_t)f32_to_bf16_rne(v[3]) << 48);
      __hip_atomic_store((g_u64*)y, q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (row + j < n_rows) store_y<true>(o, tab, row + j, m, v[j]);
}

// Cross-wave sums in LDS.  A kernel whose waves split K writes the partial
// sums of wave part p (p < P <= kMaxWaveParts) of a block of `per` outputs
// to smem[(block * kMaxWaveParts + p) * per + output]: the outputs of one
// part side by side, so that the threads of consecutive outputs read
// consecutive words.  The slots of parts P .. kMaxWaveParts - 1 hold -0.0f,
// which leaves every fp32 sum bitwise unchanged: the reader adds all
// kMaxWaveParts slots in part order, one chain of adds with no selects.

// -0.0f into the slots of parts P .. kMaxWaveParts - 1 of `blocks` blocks
// (every thread of the workgroup takes part; before the barrier that
// precedes the reads).
__device__ __forceinline__ void fill_unused_parts(float* smem, int blocks, int P, int per,
                                                  int tid, int n_threads) {
  const int per_block = (kMaxWaveParts - P) * per;
  for (int i = tid; i < blocks * per_block; i += n_threads) {
    const int b = i / per_block;
    smem[(b * kMaxWaveParts + P) * per + (i - b * per_block)] = -0.0f;
  }
}

// The sum over the wave parts of one output, slot p at q[p * stride], in
// part order.
__device__ __forceinline__ float sum_wave_parts(const float* q, int stride) {
  float v[kMaxWaveParts];
#pragma unroll
  for (int i = 0; i < kMaxWaveParts; ++i) v[i] = q[i * stride];
  float sum = v[0];
#pragma unroll
  for (int i = 1; i < kMaxWaveParts; ++i) sum += v[i];
  return sum;
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

// Two E4M3 codes (bytes 0-1 of `u`, or bytes 2-3 with `hi`) times an fp32
// power-of-two scale, as a bf16 pair (element 0 from the lower byte):
// v_cvt_scalef32_pk_bf16_fp8.  Exact whenever the scaled value lies in bf16's
// normal range (an E4M3 value has at most 4 significant bits).
__device__ __forceinline__ bf16x2 decode_e4m3_pair(unsigned u, float scale, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u, scale, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u, scale, false);
}

// Two E2M1 codes (the low and high nibble of byte `b` of `u`; the low nibble
// is element 0) times an fp32 power-of-two scale, as a bf16 pair:
// v_cvt_scalef32_pk_bf16_fp4.  Exact whenever the scaled value lies in
// bf16's normal range (an E2M1 value has at most 2 significant bits).
template <int B>
__device__ __forceinline__ bf16x2 decode_e2m1_pair(unsigned u, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u, scale, B);
}

// Two E2M1 codes (byte B of u) times an NVFP4 block scale `s` (an E4M3
// value as fp32: at most 4 significant bits), as a bf16 pair.
// v_cvt_scalef32_pk_bf16_fp4 applies only the exponent of its fp32 scale
// operand (measured on MI355X: code 0.5 at scale 1.5 gives 0.5), which is
// all an E8M0 scale has; here the codes are decoded to fp32 at scale 1
// (v_cvt_scalef32_pk_f32_fp4), multiplied by s in fp32 (exact: at most
// 2 + 4 significant bits) and converted to bf16 (v_cvt_pk_bf16_f32, exact
// for the same reason).
template <int B>
__device__ __forceinline__ bf16x2 decode_e2m1_pair_nv(unsigned u, float s) {
#pragma clang fp contract(off)
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(u, 1.0f, B);
  const float lo = d[0] * s;
  const float hi = d[1] * s;
  return bf16x2{(__bf16)lo, (__bf16)hi};
}

// Two E4M3 codes (bytes 0 and 1 of u) as fp32 values (exact; OCP E4M3:
// bias 7, subnormals m * 2^-9): v_cvt_scalef32_pk_f32_fp8 at scale 1.
__device__ __forceinline__ void e4m3x2_to_f32(unsigned u, float* lo, float* hi) {
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u, 1.0f, false);
  *lo = d[0];
  *hi = d[1];
}

// An E4M3 code as an fp32 value (exact: 4 significant bits; sign, 4
// exponent bits of bias 7, 3 mantissa bits, subnormals m * 2^-9).  The NaN
// codes (0x7F, 0xFF) are outside the served domain and decode to a large
// finite value.
__device__ __forceinline__ float e4m3_to_f32(unsigned b) {
  const unsigned e = (b >> 3) & 0xFu, m = b & 7u, s = (b & 0x80u) << 24;
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  return e != 0u ? u2f(s | ((e + 120u) << 23) | (m << 20)) : (s ? -sub : sub);
}

// Dot product of 8 decoded weights (four bf16 pairs, element order) with
// the 8 activations of one chunk, added into `acc` pair by pair in order
// (the order of dot_chunk).
__device__ __forceinline__ float dot_decoded(const bf16x2* d, const u32x4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(d[0], u2bf2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(d[1], u2bf2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(d[2], u2bf2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(d[3], u2bf2(x.w), acc, false);
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
// partial[s][row][m] (the tile kernels: partial[s][m][row], see
// splitk_finish_vec) with agent-coherent stores (sc1: written through to the
// point of coherence shared by all XCDs instead of staying dirty in this
// XCD's L2), waits until they are acknowledged, and then arrives on
// counters[rb].  The workgroup that arrives last reads the S partials with
// agent-coherent loads, adds them in slice order s = 0, 1, ..., S-1, stores
// the outputs and resets the counter to zero, so the next call (or graph
// replay) needs no host action.  Because every partial store and load is
// agent-coherent, no L2 writeback or invalidation (what an agent-scope
// fence would cost per workgroup) is needed.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(1))) float gf32;
typedef __attribute__((address_space(1))) uint32_t gu32;

__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store((gf32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_partial(const float* p) {
  return __hip_atomic_load((gf32*)const_cast<float*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Must be called by every thread of the workgroup (it has barriers).
template <bool BF16, bool SCALED = false>
__device__ __forceinline__ void splitk_finish(int n_rows_i,
                                              const float* partial,
                                              uint32_t* counters, int rb,
                                              int S, int64_t row_base,
                                              int64_t R, int M, int nthreads,
                                              const OutMap& os, const OutTable& tab,
                                              int* flag) {
  // this thread's partial stores are complete (vmcnt = 0; expcnt and
  // lgkmcnt left at their maximum) before the workgroup arrives
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add((gu32*)(counters + rb), 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (unsigned)(S - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  const int64_t n_rows = n_rows_i;
  const int64_t rows_here = (n_rows - row_base) < R ? (n_rows - row_base) : R;
  const int64_t n_fin = rows_here * M;
  const int64_t sstride = n_rows * M;
  for (int64_t t = threadIdx.x; t < n_fin; t += nthreads) {
    const int64_t rr = t / M;
    const int m = (int)(t - rr * M);
    const int64_t row = row_base + rr;
    const float* pp = partial + row * M + m;
    float sum = load_partial(pp);
    for (int ss = 1; ss < S; ++ss) sum += load_partial(pp + ss * sstride);
    store_y<BF16, SCALED>(os, tab, (int)row, m, sum);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store((gu32*)(counters + rb), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace fp
