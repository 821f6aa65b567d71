// skinny.hpp -- weight-streaming vector-ALU kernel for y = x . W^T with few
// token rows (M <= 8), bf16 (v_dot2, fp32 sums) or fp32 (fp32 FMA).
//
// Work split.  A launch covers n_rows weight rows (one or more projection
// segments).  A workgroup owns R = G * RW consecutive rows and one of S
// slices of the K contraction.  Its G * P waves form G row groups of RW rows
// each; the P waves of a row group split the slice into P parts of
// 64 * CJ sixteen-byte chunks, and lane l of part p reads chunks
// p*64*CJ + j*64 + l (j < CJ) of each of its RW rows -- consecutive lanes
// read consecutive 16-byte chunks, so every wave-wide load is one 1 KiB
// contiguous run of a weight row.  Every weight byte is loaded exactly once
// per call, non-temporally, and all of a lane's RW*CJ weight loads are
// issued before the first multiply so the whole workgroup's share of
// W is in flight at once.
//
// Activations.  Lane l needs x[m, chunk] only for its own chunks; each of
// them is used by the RW rows of the lane, so x is held in registers (no
// element of x is needed twice by one row group).
//
// Reduction, in a fixed order that depends only on (K, dtype, P, CJ, S):
//   1. in each lane, sequentially over its CJ chunks and, inside a chunk,
//      in element order;
//   2. across the 64 lanes of the wave by the transpose reduce of
//      common.hpp (one fixed tree of lane pairings);
//   3. across the P waves of the row group in LDS, in wave order;
//   4. with S > 1, across the S workgroups of the row block: each writes its
//      partial sums to the workspace, and the last workgroup to arrive
//      (arrival counter) adds the S partials in slice order, stores the
//      outputs and resets the counter to zero for the next call.
// The order does not depend on RW, G, the number of rows of the launch or
// the position of a row, so the fused launch and the one-launch-per-
// projection path give bitwise equal outputs, and repeats and graph
// replays are bitwise equal.  The fp32 sum is rounded once to bf16
// (round to nearest even) when stored.
#pragma once

#include "common.hpp"

namespace fp {

struct SkinnyArgs {
  const unsigned char* x;  // activations, M rows
  int64_t ldx_bytes;       // row stride of x in bytes (multiple of 16)
  int64_t row_bytes;       // K * element size (multiple of 16)
  int32_t M;               // token rows, <= MT
  int32_t kc;              // 16-byte chunks per row
  int32_t P;               // waves per row group (K parts of a slice)
  int32_t G;               // row groups per workgroup
  int32_t S;               // K slices (workgroups per row block)
  int32_t cps;             // chunks per slice = P * 64 * CJ
  int32_t R;               // rows per workgroup = G * RW
  RowSpace rs;             // rows of this launch
  float* partial;          // [S][n_rows][M] when S > 1
  uint32_t* counters;      // one per row block when S > 1, zero between calls
};

template <int MT, int RW, int CJ, bool BF16>
__global__ void __launch_bounds__(skinny_max_threads(MT, RW, CJ))
skinny_kernel(const SkinnyArgs a) {
  constexpr int V = RW * MT;        // outputs per lane
  constexpr int VP = pow2ceil(V);   // padded to a power of two
  constexpr int QV = VP >= 64 ? VP / 64 : 1;
  constexpr int LSTRIDE = VP >= 64 ? 1 : 64 / VP;

  extern __shared__ float smem[];   // [G][P][VP] wave sums, then one flag
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index made scalar so that row and slice arithmetic stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = wave % a.P;
  const int gq = wave / a.P;
  const int rb = blockIdx.x / a.S;
  const int s = blockIdx.x - rb * a.S;
  const int64_t row_base = (int64_t)rb * a.R;
  const int64_t wrow0 = row_base + (int64_t)gq * RW;
  const int cbase = s * a.cps + p * (64 * CJ) + lane;

  // 1. weight stream: every load of the lane issued up front
  u32x4 wv[RW][CJ];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const unsigned char* wrow = row_pointer(a.rs, wrow0 + r, a.row_bytes);
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      const int c = cbase + j * 64;
      if (wrow != nullptr && c < a.kc) {
        wv[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow) + c);
      } else {
        wv[r][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // 2. the lane's activation chunks
  u32x4 xv[MT][CJ];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      const int c = cbase + j * 64;
      if (m < a.M && c < a.kc) {
        xv[m][j] = reinterpret_cast<const u32x4*>(a.x + (int64_t)m * a.ldx_bytes)[c];
      } else {
        xv[m][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // 3. per-lane partial sums, chunk by chunk
  float v[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) v[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < CJ; ++j) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        v[r * MT + m] = dot_chunk<BF16>(wv[r][j], xv[m][j], v[r * MT + m]);
      }
    }
  }
  // 4. across the wave
  transpose_reduce<VP>(v, lane);
  float* red = smem + (gq * a.P + p) * VP;
  if (lane % LSTRIDE == 0) {
#pragma unroll
    for (int q = 0; q < QV; ++q) red[q + QV * (lane / LSTRIDE)] = v[q];
  }
  __syncthreads();

  // 5. across the P waves of each row group, in wave order
  const int64_t n_rows = a.rs.n_rows;
  const int n_out = a.G * V;
  for (int t = tid; t < n_out; t += blockDim.x) {
    const int g2 = t / V;
    const int idx = t - g2 * V;
    const int r = idx / MT;
    const int m = idx - r * MT;
    const int64_t row = row_base + (int64_t)g2 * RW + r;
    if (m >= a.M || row >= n_rows) continue;
    const float* rp = smem + g2 * a.P * VP + idx;
    float sum = rp[0];
    for (int pp = 1; pp < a.P; ++pp) sum += rp[pp * VP];
    if (a.S == 1) {
      store_out<BF16>(a.rs, row, m, sum);
    } else {
      a.partial[((int64_t)s * n_rows + row) * a.M + m] = sum;
    }
  }
  if (a.S == 1) return;

  // 6. split-K: the last workgroup of the row block adds the S partials
  splitk_finish<BF16>(a.rs, a.partial, a.counters, rb, a.S, row_base, a.R, a.M,
                      reinterpret_cast<int*>(smem + a.G * a.P * VP));
}

}  // namespace fp
