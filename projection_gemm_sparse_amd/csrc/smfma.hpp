// smfma.hpp -- matrix-core kernel for y = x . W^T with few tokens (M <= 16),
// bf16 in, fp32 accumulate, bf16 out.
//
// Why matrix cores at M <= 8.  The weight stream is the cost, but once the
// weights have landed a vector-ALU kernel still has to do 2 * M * K
// multiply-adds per row and then add the partial sums of its 64 lanes; at
// M = 8 that arithmetic (v_dot2 plus the cross-lane reduction) takes longer
// than a microsecond per CU and it all happens after the last weights
// arrive.  One v_mfma_f32_16x16x32_bf16 does the multiply-adds of a
// 16 x 32 x 16 block and the reduction over its 32 k-slots in the matrix
// unit, so the work left after the stream is a handful of instructions.
//
// Instruction layout (gfx950): D[16 x 16] += A[16 x 32] . B[32 x 16].  Lane
// l supplies A's row l%16 and B's column l%16 with eight bf16 values of
// k-slot group g = l/16 (k-slots 8g .. 8g+7); lane l receives D[4g + v][l%16]
// for v = 0..3.  The product sums over the 32 k-slots, so any element of K
// may sit in a k-slot as long as A and B carry the same one there.
//
// K-slice packing (two sub-slices).  With at most 8 tokens, half of the 16
// B columns would be idle, so the tile is 8 weight rows x 2 sub-slices of
// K: A row s*8 + r is weight row r on sub-slice s, B column s*8 + m is
// token m on sub-slice s.  The useful outputs are the two diagonal 8 x 8
// blocks D[s*8 + r][s*8 + m]; their sum over s is row r, token m.  At one
// MFMA step t of a wave, the lane of k-slot group g on sub-slice s carries
// the 16-byte chunk
//     c = c0 + 8t + 2g + s
// of its row (c0 = first chunk of the wave's K range), so one step covers
// 8 rows x 128 contiguous bytes; every weight byte is loaded once,
// non-temporally, as stored (no re-laid-out copy: writes through the
// projection views stay valid).  The loads themselves keep each
// quarter-wave on two rows (2 x 128 contiguous bytes) and a four-dword
// lane shuffle (ds_bpermute) moves each chunk to its MFMA lane.
//
// Nine to sixteen tokens (MH = 2 token halves; 17..24: MH = 3): every step
// multiplies the same A operand with the B operands of tokens 0..7, 8..15
// (and 16..23) -- one MFMA and one accumulator per half; the weights are
// still loaded once.  Per token the arithmetic, hence the result, is the
// same as with one half.
//
// Work split.  A workgroup owns G row groups of TT tiles of RT <= 8 rows (a
// tile with RT < 8 leaves its last A rows unused; the 1792-row fused launch
// uses one tile of 7 rows per workgroup so that its 256 workgroups cover
// the 256 CUs once).  With TT = 2 tiles every wave multiplies the same
// activation operand (each token half's) with the weights of two tiles:
// a launch of more rows than 8 per CU then keeps one workgroup per CU,
// and each CU loads the activations once instead of once per workgroup
// (at M = 8 and K = 6144 the activations are 98 KB per workgroup, more
// than the 74 KB of six weight rows).
// The PK waves of a row group split K into PK parts of KT steps (8 chunks
// each).  All of a wave's weight and activation loads are issued before its
// first MFMA, and the steps consume them in issue order.
//
// Reduction order, fixed by (K, PK, KT): MFMA steps in order inside a wave
// (the matrix unit's own order inside a step); then per output, through
// LDS, each sub-slice over the PK waves in wave order, then the two
// sub-slice sums added.  It does
// not depend on the row's position in the tile, on RT, G or the rows of
// the launch, so the fused launch and the one-launch-per-projection path are
// bitwise equal, as are repeats and graph replays.
#pragma once

#include "common.hpp"
#include "epilogue.hpp"

namespace fp {

constexpr int kFmtNv4 = 5;  // the NVFP4 form of smfma_mx_kernel

// Per-lane register estimate: the KT steps' 16-byte chunks of every tile's
// weights and every half's activations, plus addresses and accumulators.
// Forms of four or more operand sets (two tiles with two halves, three
// halves) are counted as compiled (144-152 VGPRs on gfx950 at KT = 8, so
// that 12 waves fit a CU); the others keep the estimate they were tuned
// with.
constexpr int smfma_regs(int kt, int mh, int tt) {
  return mh + tt >= 4 ? 4 * kt * (mh + tt) + 24
                      : 4 * kt * (mh + tt) + 24 + 16 * (mh - 1) + 4 * (tt - 1);
}

constexpr int smfma_max_threads(int kt, int mh = 1, int tt = 1) {
  return max_threads_for_regs(smfma_regs(kt, mh, tt));
}

// Output stage of both small-M kernels (not gate/up).  The cross-wave
// slots hold, per block gh = g2 * MH + h (row group g2, token half h) and
// wave part, the 2 x 64 sums [sub-slice][row][token]; the outputs of a block
// go in chunks of 32, four tokens x the eight rows (chunk c & 1 of block
// c / 2: tokens 8 h + 4 (c & 1) .. + 3), one chunk per wave at a time, so
// that one store instruction writes each token's rows of the tile.  Lanes
// 0..31 add sub-slice 0 of their output over the wave parts, lanes 32..63
// sub-slice 1, and one lane swap (v_permlane32_swap) brings the two
// together: sub-slice 0 + sub-slice 1.
template <int MH, bool SCALED>
__device__ __forceinline__ void smfma_store_outputs(const float* smem, int Gv, int n_waves,
                                                    int wave, int lane, int RT, int row_base,
                                                    int M, int n_rows, const OutMap& om,
                                                    const OutTable& tab) {
  const int n_chunks = Gv * MH * 2;
  for (int c = wave; c < n_chunks; c += n_waves) {
    const int gh = c >> 1;
    const int r = lane & 7;
    const int mt = 4 * (c & 1) + ((lane >> 3) & 3);  // token in the half
    const float* q = smem + gh * kMaxWaveParts * 128 + (lane >> 5) * 64 + r * 8 + mt;
    const float part = sum_wave_parts(q, 128);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                     __float_as_uint(part), false, false);
    const int g2 = gh / MH;
    const int m = 8 * (gh - g2 * MH) + mt;
    const int row = row_base + g2 * RT + r;
    if (lane < 32 && r < RT && m < M && row < n_rows)
      store_y<true, SCALED>(om, tab, row, m, __uint_as_float(sw[0]) + __uint_as_float(sw[1]));
  }
}

// Leading scalars preloaded into SGPRs (see skinny_kernel for w, x, y0,
// y1, ldx, n_rows, kc, M, split); geo = RT | PK << 8 | G << 16.
// PAIRS: a gate/up launch (rows taken in pairs, see pair_row; RT even)
// that writes silu(gate) * up instead of the projections.  MH: token halves
// (1: M <= 8, 2: M <= 16, 3: M <= 24).  XFIRST (two or more halves): every
// activation load before the weights (the fuller later halves) instead of
// each step's first-half, weight and later-half chunks in turn.  TT: row tiles per
// wave (2: not gate/up); tile j of row group g2 holds rows
// row_base + (g2 TT + j) RT ...
template <int KT, bool PAIRS = false, int MH = 1, bool XFIRST = true, int TT = 1>
__global__ void __launch_bounds__(smfma_max_threads(KT, MH, TT))
smfma_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
             unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows,
             int32_t kc, int32_t M, int32_t split, int32_t geo, const Tail a) {
  static_assert(MH == 1 || ((MH == 2 || MH == 3) && !PAIRS), "token halves");
  static_assert(TT == 1 || (TT == 2 && !PAIRS), "two tiles: not gate/up");
  extern __shared__ float smem[];  // [G][TT][MH][16 wave parts][2][8][8]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RT = geo & 0xff;
  const int PK = (geo >> 8) & 0xff;
  const int Gv = geo >> 16;
  const int p = Gv == 1 ? wave : wave % PK;
  const int g2 = Gv == 1 ? 0 : wave / PK;
  const int row_base = (int)blockIdx.x * (Gv * TT * RT);
  const int row0 = row_base + g2 * TT * RT;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int sub = i16 >> 3;   // sub-slice of this lane's A row and B column
  const int r8 = i16 & 7;     // A: weight row in the tile; B: token
  const int cw = p * (8 * KT);        // first chunk of the wave's K range
  const int c0 = cw + 2 * g + sub;    // chunk of this lane's operands at step 0
  const uint32_t row_bytes = (uint32_t)kc * 16u;
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  // Loads use the layout that keeps each quarter-wave on two rows: lane L
  // reads row (token) rl = 2 (L / 16) + (L / 8) % 2, chunk cl = L % 8 of
  // the step's eight chunks, so a quarter-wave covers 2 x 128 contiguous
  // bytes (as the vector-ALU kernel's 1 KiB runs do).  The operand of MFMA
  // lane (i16, g) -- row i16 % 8, chunk 2g + i16 / 8 -- then sits in lane
  // 8 (i16 % 8) + 2g + i16 / 8 and is fetched with four ds_bpermute_b32.
  const int rl = 2 * (lane >> 4) + ((lane >> 3) & 1);
  const int cl = lane & 7;
  const int src4 = (8 * (lane & 7) + 2 * (lane >> 4) + ((lane >> 3) & 1)) * 4;
  auto shuffle = [&](const u32x4& v) {
    u32x4 o;
    o.x = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.x);
    o.y = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.y);
    o.z = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.z);
    o.w = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.w);
    return o;
  };

  // 1. activations (token rl, clamped to a valid row; tokens past M are
  //    zeroed after the shuffle) and the weights (row rl of the tile,
  //    clamped to the launch): all loads issued before the first MFMA.
  //    Measured on MI355X at [1792, 5120]: with one token half, issuing each
  //    step's activation and weight chunks in turn beats all activations
  //    first (M = 8: 5.9 vs 6.15 us; M = 4: 5.5 vs 5.95); with two halves
  //    that order pays only while the second half is at most half full
  //    (XFIRST picks; a branch on M inside one kernel slowed both orders).
  u32x4 xv[MH][KT];
  u32x4 wv[TT][KT];
  {
    const u32x4* xrow[MH];
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      const int mc = rl + 8 * h < M ? rl + 8 * h : M - 1;
      xrow[h] = reinterpret_cast<const u32x4*>(x + (uint64_t)(uint32_t)mc * ldx);
    }
    const u32x4* wrows[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int rr = TT == 1 ? (rl < RT ? row0 + rl : row0) : row0 + j * RT + (rl < RT ? rl : 0);
      const int lrow = rr < n_rows ? rr : n_rows - 1;
      const int row = PAIRS ? pair_row(lrow, split) : lrow;
      wrows[j] = reinterpret_cast<const u32x4*>(w + (uint64_t)(uint32_t)row * row_bytes);
    }
    const u32x4* wrow = wrows[0];
    if constexpr (MH == 1) {
      // one token half: the activation and weight chunks of each step in
      // turn (every tile's), so the weight stream starts with the first load
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int c = cw + 8 * t + cl;
        const int cc = c < kc ? c : kc - 1;
        xv[0][t] = xrow[0][cc];
#pragma unroll
        for (int j = 0; j < TT; ++j) wv[j][t] = __builtin_nontemporal_load(wrows[j] + cc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (!XFIRST) {
      // two halves, the second at most half full: per step the first
      // half's chunk, the weight chunks, the second half's chunk (M = 9:
      // 6.69 vs 6.96 us with the activations first)
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int c = cw + 8 * t + cl;
        const int cc = c < kc ? c : kc - 1;
        xv[0][t] = xrow[0][cc];
#pragma unroll
        for (int j = 0; j < TT; ++j) wv[j][t] = __builtin_nontemporal_load(wrows[j] + cc);
#pragma unroll
        for (int h = 1; h < MH; ++h) xv[h][t] = xrow[h][cc];
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // two fuller halves: every activation chunk first (twice the weight
      // bytes, from L2), then the weights (M = 16: 7.2 vs 7.6 us)
#pragma unroll
      for (int h = 0; h < MH; ++h)
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const int c = cw + 8 * t + cl;
          xv[h][t] = xrow[h][c < kc ? c : kc - 1];
        }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const int c = cw + 8 * t + cl;
#pragma unroll
        for (int j = 0; j < TT; ++j)
          wv[j][t] = __builtin_nontemporal_load(wrows[j] + (c < kc ? c : kc - 1));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const OutMap om = make_out_map(y0, y1, split, n_rows, a.out, row_base);
  fill_unused_parts(smem, Gv * TT * MH, PK, 128, tid, Gv * PK * 64);
  __builtin_amdgcn_sched_barrier(0);
  // 2. MFMA steps in order; chunks past K contribute zero.  acc[j * MH + h]:
  //    tile j, token half h
  f32x4 acc[TT * MH];
#pragma unroll
  for (int i = 0; i < TT * MH; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    const bool c_ok = c0 + 8 * t < kc;
    if constexpr (TT == 1) {
      // the weight operand, then each half's activations and product
      // (this order measured 0.5 % faster than the two-tile order at M =
      // 3..8 on [1792, 5120])
      const u32x4 wa = shuffle(wv[0][t]);
      const bf16x8 A = u4bf8(c_ok ? wa : zero4);
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const bool tok_ok = r8 + 8 * h < M;
        const u32x4 xb = shuffle(xv[h][t]);
        const bf16x8 B = u4bf8(c_ok && tok_ok ? xb : zero4);
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[h], 0, 0, 0);
      }
    } else {
      // the activations of each half once, then each tile's weights and
      // its products with every half
      bf16x8 B[MH];
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const bool tok_ok = r8 + 8 * h < M;
        const u32x4 xb = shuffle(xv[h][t]);
        B[h] = u4bf8(c_ok && tok_ok ? xb : zero4);
      }
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        const u32x4 wa = shuffle(wv[j][t]);
        const bf16x8 A = u4bf8(c_ok ? wa : zero4);
#pragma unroll
        for (int h = 0; h < MH; ++h)
          acc[j * MH + h] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[h], acc[j * MH + h], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the diagonal blocks to LDS: lane (i16, g) holds D[4g + v][i16]; the
  //    D row's sub-slice is (4g + v) / 8 = g / 2, the column's is i16 / 8.
  //    Layout [G][half][wave part][sub-slice][row][token]: the 128 sums of
  //    one wave part side by side, so that the threads of consecutive
  //    outputs read consecutive words.
  if ((g >> 1) == sub) {
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        float* red =
            smem + (((g2 * TT + j) * MH + h) * kMaxWaveParts + p) * 128 + sub * 64 + r8;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = (4 * g + v) & 7;
          red[r * 8] = acc[j * MH + h][v];
        }
      }
  }
  __syncthreads();

  // 4. per output: each sub-slice over the PK wave parts in part order,
  //    then sub-slice 0 + sub-slice 1 (the tiles of the workgroup in row
  //    order: tile g2 TT + j starts at row_base + (g2 TT + j) RT)
  if constexpr (!PAIRS) {
    smfma_store_outputs<MH, false>(smem, Gv * TT, Gv * PK, wave, lane, RT, row_base, M, n_rows,
                                   om, a.out);
  } else {
    // gate/up: one thread per output; even logical rows are gate rows j,
    // the up row is tile row r + 1
    const int n_out = Gv * 64;
    if (tid < n_out) {
      const int gg = tid >> 6;
      const int r = (tid >> 3) & 7;
      const int m = tid & 7;
      const int row = row_base + gg * RT + r;
      if (r < RT && m < M && row < n_rows && (r & 1) == 0) {
        const float* q0 = smem + gg * kMaxWaveParts * 128 + r * 8 + m;
        const float sum = sum_wave_parts(q0, 128) + sum_wave_parts(q0 + 64, 128);
        const float u_sum = sum_wave_parts(q0 + 8, 128) + sum_wave_parts(q0 + 64 + 8, 128);
        store_pair(y0, split, row, m, sum, u_sum);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MX weights (FMT 8: MXFP8, FMT 4: MXFP4; rows of K codes, then K/32 E8M0
// scales), at most 8 tokens.  Tile, sub-slices, work split, reduction and
// stores are those of smfma_kernel; the weights are decoded to bf16 in the
// registers that feed the matrix unit, so the products and their sums are
// those of bf16 weights equal to the decoded values.
//
// A 16-byte load of codes holds G units of 8 elements (G = 2 for MXFP8,
// 4 for MXFP4).  So that one load serves one MFMA lane for G steps, the
// k-slot mapping runs over groups of G steps: at step G u + e of a wave,
// MFMA lane (i16 = r8 + 8 sub, g) carries unit
//     c = cw + 8 G u + G (2 g + sub) + e
// of weight row r8 (A) and token r8 (B).  Load lane L holds row L / 8,
// units cw + 8 G u + G (L % 8) + 0 .. G - 1 -- a quarter-wave covers 2 rows
// x 128 contiguous bytes of codes -- and MFMA lane (r8, sub, g) takes them
// from load lane 8 r8 + 2 g + sub (four ds_bpermute per load).  The
// activations use the same mapping (load lane L: token L / 8, the same G
// units; G 16-byte loads).  A group's G units lie in one 32-element block
// (K is a multiple of 512), whose scale the MFMA lane reads itself.
// NVFP4 (FMT kFmtNv4): E2M1 codes as MXFP4 (G = 4) with one E4M3 scale per
// 16 elements, so a group spans two blocks and the lane reads both scale
// bytes; the finished sums are multiplied by their projection's fp32
// tensor scale before the single rounding (store_y SCALED).
template <int KT, int FMT, int MH = 1>
__global__ void __launch_bounds__(smfma_max_threads(KT, MH))
smfma_mx_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
                unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows,
                int32_t kc, int32_t M, int32_t split, int32_t geo, const Tail a) {
  static_assert(FMT == 8 || FMT == 4 || FMT == kFmtNv4, "MXFP8, MXFP4 or NVFP4");
  constexpr bool NV = FMT == kFmtNv4;
  constexpr int G = FMT == 8 ? 2 : 4;      // steps per 16-byte load of codes
  constexpr int NU = KT / G;               // code loads per lane
  constexpr uint32_t UB = FMT == 8 ? 8u : 4u;  // code bytes per unit
  static_assert(KT % G == 0, "whole step groups");
  static_assert(MH == 1 || MH == 2, "token halves");
  extern __shared__ float smem[];  // [G][MH][16 wave parts][2][8][8]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RT = geo & 0xff;
  const int PK = (geo >> 8) & 0xff;
  const int Gv = geo >> 16;
  const int p = Gv == 1 ? wave : wave % PK;
  const int g2 = Gv == 1 ? 0 : wave / PK;
  const int row_base = (int)blockIdx.x * (Gv * RT);
  const int row0 = row_base + g2 * RT;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int sub = i16 >> 3;
  const int r8 = i16 & 7;
  const int cw = p * (8 * KT);                        // first unit of the wave
  const int cg = cw + G * (2 * g + sub);              // this MFMA lane's unit at u = 0
  // scales after the codes: one per 4 units (MX), per 2 units (NVFP4)
  const uint32_t row_bytes = (uint32_t)kc * UB + ((uint32_t)kc >> (NV ? 1 : 2));
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  const int rl = lane >> 3;    // load lane: row / token
  const int pl = lane & 7;     // load lane: unit group in the step group
  const int src4 = (8 * r8 + 2 * g + sub) * 4;
  auto shuffle = [&](const u32x4& v) {
    u32x4 o;
    o.x = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.x);
    o.y = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.y);
    o.z = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.z);
    o.w = (unsigned)__builtin_amdgcn_ds_bpermute(src4, (int)(unsigned)v.w);
    return o;
  };

  // 1. all loads before the first MFMA, group by group: the codes (row rl
  //    of the tile clamped to the launch; the weight stream starts with
  //    the first load), this MFMA lane's block scale(s), then the group's
  //    activation chunks of each token half (token rl + 8h clamped; tokens
  //    past M are zeroed after the shuffle)
  u32x4 xv[MH][NU][G];
  u32x4 qv[NU];
  uint32_t sv[NU];
  {
    const u32x4* xrow[MH];
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      const int mc = rl + 8 * h < M ? rl + 8 * h : M - 1;
      xrow[h] = reinterpret_cast<const u32x4*>(x + (uint64_t)(uint32_t)mc * ldx);
    }
    const int rr = rl < RT ? row0 + rl : row0;
    const int row = rr < n_rows ? rr : n_rows - 1;
    const unsigned char* wrow = w + (uint64_t)(uint32_t)row * row_bytes;
    const int sr = r8 < RT ? row0 + r8 : row0;
    const int srw = sr < n_rows ? sr : n_rows - 1;
    const unsigned char* srow = w + (uint64_t)(uint32_t)srw * row_bytes + (uint32_t)kc * UB;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c0 = cw + 8 * G * u + G * pl;   // first unit of the load
      const int c = c0 < kc ? c0 : kc - G;
      qv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + (uint32_t)c * UB));
      const int cs = cg + 8 * G * u;
      if constexpr (NV) {
        // the group's 4 units span two 16-element blocks: both scale bytes
        const int cc = cs < kc ? cs : kc - 4;
        sv[u] = *reinterpret_cast<const uint16_t*>(srow + (cc >> 1));
      } else {
        sv[u] = srow[(cs < kc ? cs : kc - 1) >> 2];
      }
#pragma unroll
      for (int h = 0; h < MH; ++h)
#pragma unroll
        for (int e = 0; e < G; ++e) {
          const int cx = c0 + e;
          xv[h][u][e] = xrow[h][cx < kc ? cx : kc - 1];
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const OutMap om = make_out_map<NV>(y0, y1, split, n_rows, a.out, row_base);
  fill_unused_parts(smem, Gv * MH, PK, 128, tid, Gv * PK * 64);
  __builtin_amdgcn_sched_barrier(0);

  // 2. step groups in order, steps in order inside a group; units past K
  //    contribute zero
  f32x4 acc[MH];
#pragma unroll
  for (int h = 0; h < MH; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    __builtin_amdgcn_sched_barrier(0);
    const bool c_ok = cg + 8 * G * u < kc;
    const u32x4 q = shuffle(qv[u]);
    // MX: scale 2^(s - 127) as an fp32 (s = 0: the subnormal 2^-127);
    // NVFP4: the E4M3 scales of the group's two blocks (units 0, 1 and 2, 3)
    const uint32_t sb = sv[u];
    float sc, sc_hi;
    if constexpr (NV) {
      e4m3x2_to_f32(sb, &sc, &sc_hi);
    } else {
      sc = u2f(sb != 0u ? sb << 23 : 0x00400000u);
      sc_hi = sc;
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const float sce = e < 2 ? sc : sc_hi;
      bf16x2 d[4];
      if constexpr (FMT == 8) {
        const unsigned q0 = e == 0 ? q.x : q.z;
        const unsigned q1 = e == 0 ? q.y : q.w;
        d[0] = decode_e4m3_pair(q0, sc, false);
        d[1] = decode_e4m3_pair(q0, sc, true);
        d[2] = decode_e4m3_pair(q1, sc, false);
        d[3] = decode_e4m3_pair(q1, sc, true);
      } else {
        const unsigned qe = e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
        if constexpr (NV) {
          d[0] = decode_e2m1_pair_nv<0>(qe, sce);
          d[1] = decode_e2m1_pair_nv<1>(qe, sce);
          d[2] = decode_e2m1_pair_nv<2>(qe, sce);
          d[3] = decode_e2m1_pair_nv<3>(qe, sce);
        } else {
          d[0] = decode_e2m1_pair<0>(qe, sce);
          d[1] = decode_e2m1_pair<1>(qe, sce);
          d[2] = decode_e2m1_pair<2>(qe, sce);
          d[3] = decode_e2m1_pair<3>(qe, sce);
        }
      }
      const u32x4 wa =
          u32x4{__builtin_bit_cast(unsigned, d[0]), __builtin_bit_cast(unsigned, d[1]),
                __builtin_bit_cast(unsigned, d[2]), __builtin_bit_cast(unsigned, d[3])};
      const bf16x8 A = u4bf8(c_ok ? wa : zero4);
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const bool tok_ok = r8 + 8 * h < M;
        const u32x4 xb = shuffle(xv[h][u][e]);
        const bf16x8 B = u4bf8(c_ok && tok_ok ? xb : zero4);
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[h], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the diagonal blocks to LDS (as smfma_kernel)
  if ((g >> 1) == sub) {
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      float* red = smem + ((g2 * MH + h) * kMaxWaveParts + p) * 128 + sub * 64 + r8;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = (4 * g + v) & 7;
        red[r * 8] = acc[h][v];
      }
    }
  }
  __syncthreads();

  // 4. per output: each sub-slice over the PK wave parts in part order,
  //    then sub-slice 0 + sub-slice 1
  smfma_store_outputs<MH, NV>(smem, Gv, Gv * PK, wave, lane, RT, row_base, M, n_rows, om, a.out);
}

}  // namespace fp
