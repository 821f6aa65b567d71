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
// element of x is needed twice by one row group).  They are loaded before
// the weights, so the rows can be multiplied as their loads land.
//
// Reduction, in a fixed order that depends only on (K, dtype, P, CJ, S):
//   1. in each lane, sequentially over its CJ chunks and, inside a chunk,
//      in element order;
//   2. across the 64 lanes of the wave by the transpose reduce of
//      common.hpp (one fixed tree of lane pairings);
//   3. across the P waves of the row group in LDS, in wave order (the
//      sums of one wave part side by side, so that the threads of
//      consecutive outputs read consecutive words);
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
#include "epilogue.hpp"

namespace fp {

// Kernel arguments.  The leading scalars are preloaded into SGPRs at wave
// launch (-amdgpu-kernarg-preload-count), so nothing the kernel needs before
// its stores is read from kernel-argument memory after the loads are issued:
//   w, x       weights (row stride kc * 16 bytes) and activations (M rows,
//              row stride ldx bytes)
//   y0, y1     outputs of the first two segments, split = first row of the
//              second (split < 0: more than two segments, see OutMap)
//   kc         16-byte chunks per row (K * element size / 16)
//   geo        P | G << 8 | S << 16: waves per row group (K parts of a
//              slice), row groups per workgroup, K slices
// A K slice holds P * 64 * CJ chunks; a workgroup owns G * RW rows.  The
// hardware preloads at most 14 argument dwords, exactly these; one more
// would be read from memory before the first load could issue.
// VAR selects a variant, each compiled only where it is used:
//   kVarPlain   the projections, stored as the input type;
//   kVarPairs   a gate/up launch (rows taken in pairs, see pair_row; RW
//               even, S = 1, bf16) that writes silu(gate) * up;
//   kVarF32Out  bf16 operands with fp32 outputs (router logits), up to 16
//               tokens (MT = 16);
//   kVarMx8     MXFP8 weights, bf16 activations and outputs.  A weight row
//               is its K E4M3 codes followed by the K/32 E8M0 scales of its
//               32-element blocks (row stride K + K/32 bytes).  The unit of
//               work is 8 elements, as in the bf16 kernel: kc counts them
//               (K/8); a lane loads the unit's 8 codes (8 bytes) and its
//               block's scale, decodes them to four bf16 pairs
//               (v_cvt_scalef32_pk_bf16_fp8: exact, an E4M3 value times a
//               power of two has at most 4 significant bits) and multiplies
//               them with the unit's activation chunk by v_dot2 in element
//               order -- the bf16 kernel's arithmetic on half the weight
//               bytes;
//   kVarMx4     MXFP4 weights: the same with E2M1 codes, two per byte (the
//               low nibble first): a unit is 4 code bytes, a row K/2 code
//               bytes followed by its K/32 scales, and each code byte
//               decodes to one bf16 pair (v_cvt_scalef32_pk_bf16_fp4).
//   kVarNv4     NVFP4 weights: E2M1 codes as kVarMx4, one E4M3 scale per
//               16 elements (a row: K/2 code bytes, then K/16 scales), so
//               two units share a scale; writing the scale as 2^E * f,
//               the unit decodes exactly at 2^E and its 8-term sum (from
//               0, in element order) is added into the output's sum with
//               one fused multiply-add by f; each finished sum is
//               multiplied by its projection's fp32 tensor scale before the
//               single rounding.
template <int MT, int RW, int CJ, bool BF16, int VAR = kVarPlain>
__global__ void __launch_bounds__(skinny_max_threads(MT, RW, CJ, VAR))
skinny_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
              unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows,
              int32_t kc, int32_t M, int32_t split, int32_t geo, const Tail a) {
  constexpr int V = RW * MT;        // outputs per lane
  constexpr int VP = pow2ceil(V);   // padded to a power of two
  constexpr int QV = VP >= 64 ? VP / 64 : 1;
  constexpr int LSTRIDE = VP >= 64 ? 1 : 64 / VP;
  constexpr bool PAIRS = VAR == kVarPairs;
  constexpr bool OUT_BF16 = BF16 && VAR != kVarF32Out;
  constexpr bool MX8 = VAR == kVarMx8;
  constexpr bool NV4 = VAR == kVarNv4;
  constexpr bool MX4 = VAR == kVarMx4 || NV4;  // 4-bit codes, 4 bytes per unit
  constexpr bool MX = MX8 || MX4;
  constexpr uint32_t UB = MX8 ? 8u : 4u;  // code bytes per 8-element unit

  extern __shared__ float smem[];   // [G][VP][16] wave sums, then one flag
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index made scalar so that row and slice arithmetic stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the common single-group, unsplit case avoids the integer divisions
  const int P = geo & 0xff;
  const int Gv = (geo >> 8) & 0xff;
  const int Sv = geo >> 16;
  const bool simple = (geo >> 8) == (1 | (1 << 8));
  const int p = simple ? wave : wave % P;
  const int gq = simple ? 0 : wave / P;
  const int rb = simple ? (int)blockIdx.x : (int)blockIdx.x / Sv;
  const int s = simple ? 0 : (int)blockIdx.x - rb * Sv;
  const int row_base = rb * (Gv * RW);
  const int wrow0 = row_base + gq * RW;
  const int cbase = s * (P * 64 * CJ) + p * (64 * CJ) + lane;
  // MXFP8 / MXFP4: UB code bytes per unit, then one scale byte per 4 units
  // (NVFP4: one scale per 2 units)
  const uint32_t row_bytes = NV4  ? (uint32_t)kc * UB + ((uint32_t)kc >> 1)
                             : MX ? (uint32_t)kc * UB + ((uint32_t)kc >> 2)
                                  : (uint32_t)kc * 16u;

  // Loads are branch-free: an out-of-range chunk or row loads a clamped,
  // always-valid address, and out-of-range chunks are replaced by zero only
  // when they are consumed (rows past the end are computed and dropped).  The
  // loads thus form one straight-line sequence, and each row can be consumed
  // as soon as its own loads have landed.
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  bool c_ok[CJ];
#pragma unroll
  for (int j = 0; j < CJ; ++j) c_ok[j] = cbase + j * 64 < kc;

  // 1. the lane's activation chunks first: they come from L2/MALL and are
  //    needed by every row, so loading them ahead of the weights keeps them
  //    off the tail of the weight stream
  u32x4 xv[MT][CJ];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mc = m < M ? m : M - 1;
    const u32x4* xrow = reinterpret_cast<const u32x4*>(x + (uint64_t)(uint32_t)mc * ldx);
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      const int c = cbase + j * 64;
      xv[m][j] = xrow[c < kc ? c : kc - 1];
    }
  }
  // 2. weight stream: every load of the lane issued up front, row by row
  u32x4 wv[MX ? 1 : RW][CJ];
  u32x2 qv[MX8 ? RW : 1][CJ];     // MXFP8: the unit's 8 codes
  uint32_t q4[MX4 ? RW : 1][CJ];  // MXFP4: the unit's 8 codes (4 bytes)
  uint32_t sv[MX ? RW : 1][CJ];   // MXFP8 / MXFP4: the block's E8M0 scale
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int lrow = wrow0 + r < n_rows ? wrow0 + r : n_rows - 1;
    const int row = PAIRS ? pair_row(lrow, split) : lrow;
    const unsigned char* wrow_b = w + (uint64_t)(uint32_t)row * row_bytes;
    if constexpr (MX8) {
      const u32x2* wrow = reinterpret_cast<const u32x2*>(wrow_b);
#pragma unroll
      for (int j = 0; j < CJ; ++j) {
        const int c = cbase + j * 64;
        qv[r][j] = __builtin_nontemporal_load(wrow + (c < kc ? c : kc - 1));
      }
      const unsigned char* srow = wrow_b + (uint32_t)kc * 8u;
#pragma unroll
      for (int j = 0; j < CJ; ++j) {
        const int c = cbase + j * 64;
        sv[r][j] = srow[(c < kc ? c : kc - 1) >> 2];
      }
    } else if constexpr (MX4) {
      const uint32_t* wrow = reinterpret_cast<const uint32_t*>(wrow_b);
#pragma unroll
      for (int j = 0; j < CJ; ++j) {
        const int c = cbase + j * 64;
        q4[r][j] = __builtin_nontemporal_load(wrow + (c < kc ? c : kc - 1));
      }
      const unsigned char* srow = wrow_b + (uint32_t)kc * 4u;
#pragma unroll
      for (int j = 0; j < CJ; ++j) {
        const int c = cbase + j * 64;
        sv[r][j] = srow[(c < kc ? c : kc - 1) >> (NV4 ? 1 : 2)];
      }
    } else {
      const u32x4* wrow = reinterpret_cast<const u32x4*>(wrow_b);
#pragma unroll
      for (int j = 0; j < CJ; ++j) {
        const int c = cbase + j * 64;
        wv[r][j] = __builtin_nontemporal_load(wrow + (c < kc ? c : kc - 1));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // where this workgroup's outputs go, and the split-K workspace, resolved
  // while the loads are in flight
  const OutMap om = make_out_map<NV4>(y0, y1, split, n_rows, a.out, row_base);
  float* partial = a.partial;
  uint32_t* counters = a.counters;
  if (Sv > 1) asm volatile("" : "+s"(partial), "+s"(counters));
  // the cross-wave slots of absent wave parts read as -0.0f
  if (P > 1 || Sv > 1 || PAIRS) fill_unused_parts(smem, Gv, P, VP, tid, Gv * P * 64);
  __builtin_amdgcn_sched_barrier(0);
  // activations past M or past K count as zero
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < CJ; ++j) xv[m][j] = (m < M && c_ok[j]) ? xv[m][j] : zero4;
  }

  // 3. per-lane partial sums in load order (row by row), so each row is
  //    consumed as soon as its loads have landed; each output still adds its
  //    chunks in order j = 0 .. CJ-1
  float v[VP];
#pragma unroll
  for (int i = 0; i < VP; ++i) v[i] = 0.0f;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    // keep the rows in load order: the compiler then waits only for the
    // loads of row r (vmcnt counts loads in issue order)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      if constexpr (MX8) {
        // codes past K read as zero; scale 2^(s - 127) as an fp32 (s = 0:
        // the subnormal 2^-127)
        const u32x2 q = c_ok[j] ? qv[r][j] : u32x2{0u, 0u};
        const uint32_t sb = sv[r][j];
        const float sc = u2f(sb != 0u ? sb << 23 : 0x00400000u);
        const unsigned q0 = q.x, q1 = q.y;
        const bf16x2 d[4] = {decode_e4m3_pair(q0, sc, false), decode_e4m3_pair(q0, sc, true),
                             decode_e4m3_pair(q1, sc, false), decode_e4m3_pair(q1, sc, true)};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          v[r * MT + m] = dot_decoded(d, xv[m][j], v[r * MT + m]);
        }
      } else if constexpr (MX4) {
        const unsigned q = c_ok[j] ? q4[r][j] : 0u;
        const uint32_t sb = sv[r][j];
        // MXFP4: E8M0 scale 2^(s - 127); NVFP4: the E4M3 block scale (the
        // tensor scale is applied to the finished sum)
        if constexpr (NV4) {
          // the E4M3 scale as 2^E * f: the codes decode at the power of
          // two (the decode instruction applies only a scale's exponent;
          // exact), the unit's 8-term sum is formed from 0 and added in
          // with one fused multiply-add by f (f = 1 + m/8, or m for the
          // subnormal scales m * 2^-9)
          const unsigned e = (sb >> 3) & 0xFu, mb = sb & 7u;
          const float p2 = u2f(e != 0u ? (e + 120u) << 23 : 0x3B000000u);  // 2^(e-7) or 2^-9
          const float fm = (sb & 0x80u) ? -1.0f : 1.0f;
          const float f = e != 0u ? fm * (1.0f + 0.125f * (float)mb) : fm * (float)mb;
          const bf16x2 d[4] = {decode_e2m1_pair<0>(q, p2), decode_e2m1_pair<1>(q, p2),
                               decode_e2m1_pair<2>(q, p2), decode_e2m1_pair<3>(q, p2)};
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float t = dot_decoded(d, xv[m][j], 0.0f);
            v[r * MT + m] = __builtin_fmaf(t, f, v[r * MT + m]);
          }
        } else {
          const float sc = u2f(sb != 0u ? sb << 23 : 0x00400000u);
          const bf16x2 d[4] = {decode_e2m1_pair<0>(q, sc), decode_e2m1_pair<1>(q, sc),
                               decode_e2m1_pair<2>(q, sc), decode_e2m1_pair<3>(q, sc)};
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            v[r * MT + m] = dot_decoded(d, xv[m][j], v[r * MT + m]);
          }
        }
      } else {
        const u32x4 wj = c_ok[j] ? wv[r][j] : zero4;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          v[r * MT + m] = dot_chunk<BF16>(wj, xv[m][j], v[r * MT + m]);
        }
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. across the wave
  transpose_reduce<VP>(v, lane);
  if (P == 1 && Sv == 1 && !PAIRS) {
    // the wave holds whole rows: its lanes store the finished sums, no
    // workgroup barrier
    if (lane % LSTRIDE == 0) {
#pragma unroll
      for (int q = 0; q < QV; ++q) {
        const int idx = q + QV * (lane / LSTRIDE);
        const int r = idx / MT;
        const int m = idx - r * MT;
        const int row = wrow0 + r;
        if (idx < V && m < M && row < n_rows) store_y<OUT_BF16, NV4>(om, a.out, row, m, v[q]);
      }
    }
    return;
  }
  // wave sums to LDS, [row group][wave part][output]: the VP outputs of one
  // wave part side by side
  float* red = smem + (gq * kMaxWaveParts + p) * VP;
  if (lane % LSTRIDE == 0) {
#pragma unroll
    for (int q = 0; q < QV; ++q) red[q + QV * (lane / LSTRIDE)] = v[q];
  }
  __syncthreads();

  // 5. across the P waves of each row group, in wave order.  There are at
  //    most G * V <= G * P * 64 outputs, one per thread.
  const int n_out = Gv * V;
  if (tid < n_out) {
    const int g2 = tid / V;
    const int idx = tid - g2 * V;
    const int r = idx / MT;
    const int m = idx - r * MT;
    const int row = row_base + g2 * RW + r;
    if (m < M && row < n_rows) {
      const float* q0 = smem + g2 * kMaxWaveParts * VP + idx;
      const float sum = sum_wave_parts(q0, VP);
      if constexpr (PAIRS) {
        // even logical rows: gate row j, its up row in the next slot
        if ((r & 1) == 0) {
          const float u_sum = sum_wave_parts(q0 + MT, VP);
          store_pair(y0, split, row, m, sum, u_sum);
        }
      } else if (Sv == 1) {
        store_y<OUT_BF16, NV4>(om, a.out, row, m, sum);
      } else {
        store_partial(partial + ((int64_t)s * n_rows + row) * M + m, sum);
      }
    }
  }
  if (Sv == 1) return;

  // 6. split-K: the last workgroup of the row block adds the S partials
  splitk_finish<OUT_BF16, NV4>(n_rows, partial, counters, rb, Sv, row_base, (int64_t)Gv * RW, M,
                      Gv * P * 64, om, a.out,
                      reinterpret_cast<int*>(smem + Gv * VP * kMaxWaveParts));
}

}  // namespace fp
