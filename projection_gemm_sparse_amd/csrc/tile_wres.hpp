// tile_wres.hpp -- matrix-core tile kernel for many tokens with the weight
// slice resident in LDS and the activations streamed by producer waves,
// bf16 in, fp32 accumulate, bf16 out.
//
// Instruction and operand layout as in tile.hpp: v_mfma_f32_16x16x32_bf16,
// A = 16 weight rows, B = 16 tokens, lane (i16, g) supplies row / token i16
// with piece g (16 bytes) of a 32-wide k step and receives D[4g + v][i16].
//
// Work split (as the ring tile kernel): a workgroup owns a block of 64
// weight rows, all BM = 32 B token slots and one of S slices of the k steps,
// consumed in stages of two k steps (64 k, 128 bytes of every row).  Four
// MFMA waves form a 2 x 2 grid: wave (wr, wm) multiplies rows 32 wr .. + 31
// with tokens BM/2 wm .. + BM/2 - 1 (2 x B accumulator tiles).
//
// What differs from the ring tile kernel is where the bytes in flight come
// from.  There, each stage buffer holds the stage's weight rows and token
// rows, so only the few stages of the ring are ever requested ahead, and a
// slice's weights (the HBM stream) trickle in a few kilobytes per CU per
// memory latency.  Here the MFMA waves request their workgroup's whole
// weight slice into LDS at the start (two 1 KiB instructions per wave and
// stage, non-temporal) -- every weight byte of the call is in flight at
// once, as in the streaming kernel -- and consume it stage by stage as it
// lands (the memory counter retires a wave's loads in issue order).  The
// activations (L2 hits) go through a ring of D stage buffers filled by
// separate producer waves: a wave's memory counter only counts its own
// loads, so the producers can refill the ring while the weight stream is
// still arriving.  Every stage ends with one workgroup barrier that all
// waves take: the producers wait for their stage's loads first, the MFMA
// waves for their weights of the stage.
//
// LDS slots (16 bytes) use an xor swizzle instead of padding: piece p
// (0..7) of row r of a stage sits at slot 8 r + (p ^ ((r >> 1) & 7)), so
// the 16 lanes of a quarter-wave reading one piece of 16 consecutive rows
// hit 16 distinct bank groups; the loads keep 8 lanes on each 128-byte row
// run (a lane loads the piece its slot holds).
//
// Reduction order, fixed by (K, S): each output's k steps in order inside
// its wave (the matrix unit's order inside a step), then the S slice sums in
// slice order (splitk_finish_vec in the launch, or splitk_reduce_kernel in a
// second launch).  The slice bounds and every output's MFMA sequence are
// those of the ring tile and tile kernels for the same S, so all three give
// the same bits; nothing depends on a row's position, so fused and
// one-launch-per-projection calls are bitwise equal.
#pragma once

#include "tile.hpp"

namespace fp {

constexpr int kWresRows = 64;          // weight rows per workgroup
constexpr int kWresStageSlots = 512;   // 64 rows x 8 pieces
// Producer waves per token block (8 instructions per stage each, at most 4
// for 32 tokens).
__host__ __device__ constexpr int wres_producers(int bm) { return bm <= 64 ? 1 : bm / 64; }
__host__ __device__ constexpr int wres_threads(int bm) { return 64 * (4 + wres_producers(bm)); }
// Ring depth and the most stages a slice may span (its weight slice sits in
// LDS beside the ring; the two stay within 160 KiB).  Four stages of
// activations ahead are enough: the ring refills from L2, and a deeper ring
// measured slower (more producer loads queued in front of the weights'
// first stages).
__host__ __device__ constexpr int wres_ring(int bm) {
  return bm <= 64 ? 4 : 3;
}
__host__ __device__ constexpr int wres_max_stages(int bm) {
  return bm <= 32 ? 16 : bm <= 64 ? 14 : bm <= 128 ? 12 : 8;
}
__host__ __device__ constexpr int wres_lds_bytes(int bm) {
  return (wres_max_stages(bm) * kWresStageSlots + wres_ring(bm) * bm * 8) * 16;
}

__device__ __forceinline__ int wres_slot(int r, int p) { return 8 * r + (p ^ ((r >> 1) & 7)); }

// Leading scalars as in tile_kernel; geo = S, plus kGeoSecondFinish.
template <int B>
__global__ void __launch_bounds__(wres_threads(32 * B))
wres_tile_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
                 unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows,
                 int32_t kc, int32_t M, int32_t split, int32_t geo, const Tail a) {
  constexpr int BM = 32 * B;
  constexpr int PX = wres_producers(BM);
  constexpr int D = wres_ring(BM);
  constexpr int NSTMAX = wres_max_stages(BM);
  constexpr int JX = BM / (8 * PX);        // activation instructions per producer and stage
  constexpr int NT = wres_threads(BM);
  static_assert(2 * NSTMAX <= 63 && (D - 2) * JX <= 63, "vmcnt field");
  static_assert(BM % (8 * PX) == 0, "whole producer instructions");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = geo & 0x1fff;
  const int rb = S == 1 ? (int)blockIdx.x : (int)blockIdx.x / S;
  const int s = S == 1 ? 0 : (int)blockIdx.x - rb * S;
  const int row_base = rb * kWresRows;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int n_steps = (kc + 3) >> 2;
  const int per_s = (n_steps + S - 1) / S;
  const int step0 = s * per_s;
  const int step1 = step0 + per_s < n_steps ? step0 + per_s : n_steps;
  // stages of two k steps (the host keeps n_st <= NSTMAX)
  const int n_st = step1 > step0 ? (step1 - step0 + 1) >> 1 : 0;
  const uint32_t row_bytes = (uint32_t)kc * 16u;
  const u32x4* wls = reinterpret_cast<const u32x4*>(lds_raw);
  const u32x4* xls = wls + NSTMAX * kWresStageSlots;
  // this lane's (row or token, piece) in a load instruction: 8 lanes per
  // 128-byte run, piece = slot ^ swizzle
  const int lr = lane >> 3;

  if (wave < 4) {
    // ------------------------------------------------ MFMA waves
    // 1. the whole weight slice: instructions 2 wave, 2 wave + 1 of each
    //    stage (rows 16 wave .. 16 wave + 15), stage by stage
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w, (uint32_t)n_rows * row_bytes);
    for (int st = 0; st < n_st; ++st) {
      const int step = step0 + 2 * st;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = 2 * wave + j;   // rows 8 q .. 8 q + 7 of the block
        const int r = 8 * q + lr;
        const int p = (lane & 7) ^ ((r >> 1) & 7);
        const int piece = step * 4 + p;
        const bool ok = row_base + r < n_rows && step + (p >> 2) < step1 && piece < kc;
        const uint32_t off = ok ? (uint32_t)(row_base + r) * row_bytes + (uint32_t)piece * 16u
                                : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wrs, (lds_void*)(lds_raw + (size_t)(st * kWresStageSlots + q * 64) * 16), 16, off,
            0, 0, kAuxNt);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int wr = wave >> 1;
    const int wm = wave & 1;
    f32x4 acc[2][B];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < B; ++k) acc[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < n_st; ++st) {
      // this wave's weights of stage st have landed once at most the
      // stages after it are outstanding
      const int ahead = n_st - 1 - st;
      static_for<0, NSTMAX>([&](auto ki) {
        constexpr int k = decltype(ki)::value;
        if (ahead == k) wait_vmcnt<2 * k>();
      });
      // every wave's weights and the producers' activations of stage st
      // are in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const u32x4* wst = wls + st * kWresStageSlots;
      const u32x4* xst = xls + (st % D) * (BM * 8);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (step0 + 2 * st + t < step1) {
          const int p = 4 * t + g;
          bf16x8 Af[2], Bf[B];
#pragma unroll
          for (int i = 0; i < 2; ++i) Af[i] = u4bf8(wst[wres_slot(32 * wr + 16 * i + i16, p)]);
#pragma unroll
          for (int k = 0; k < B; ++k) Bf[k] = u4bf8(xst[wres_slot(BM / 2 * wm + 16 * k + i16, p)]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < B; ++k)
              acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[i], Bf[k], acc[i][k], 0, 0, 0);
        }
      }
    }
    // 2. outputs (S == 1) or this slice's partial sums: lane (i16, g) of
    //    tile (i, k) holds rows 4 g + v of row tile i, token BM/2 wm + 16 k + i16
    const int row_w = row_base + 32 * wr + 4 * g;
    const int m_w = BM / 2 * wm + i16;
    if (S == 1) {
      const OutMap om = make_out_map(y0, y1, split, n_rows, a.out, row_base);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < B; ++k) {
          const int row = row_w + 16 * i;
          const int m = m_w + 16 * k;
          if (m < M && row < n_rows) store_y4(om, a.out, row, m, acc[i][k], n_rows);
        }
    } else {
      float* partial = a.partial;
      const uint32_t rp = (uint32_t)tile_partial_pitch(n_rows);
      const __amdgpu_buffer_rsrc_t prs = make_rsrc(partial, (uint32_t)S * (uint32_t)M * rp * 4u);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < B; ++k) {
          const int row = row_w + 16 * i;
          const int m = m_w + 16 * k;
          if (m < M && row < n_rows)
            store_partial4(prs, ((uint32_t)s * (uint32_t)M + (uint32_t)m) * rp + (uint32_t)row,
                           acc[i][k]);
        }
    }
  } else {
    // ------------------------------------------------ producer waves
    // token rows v JX / 8 ... of every stage: instruction j of producer v
    // fills slots 64 (v JX + j) .. + 63 of the stage buffer (tokens
    // 8 (v JX + j) .. + 7)
    const int v = wave - 4;
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)(M - 1) * ldx + row_bytes);
    auto issue = [&](int st) {
      const int step = step0 + 2 * st;
      unsigned char* buf = lds_raw + (size_t)(NSTMAX * kWresStageSlots + (st % D) * BM * 8) * 16;
#pragma unroll
      for (int j = 0; j < JX; ++j) {
        const int q = v * JX + j;
        const int tok = 8 * q + lr;
        const int p = (lane & 7) ^ ((tok >> 1) & 7);
        const int piece = step * 4 + p;
        const bool ok = tok < M && step + (p >> 2) < step1 && piece < kc;
        const uint32_t off = ok ? (uint32_t)tok * ldx + (uint32_t)piece * 16u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void*)(buf + (size_t)q * 64 * 16), 16,
                                                 off, 0, 0, 0);
      }
    };
    // the ring's first D - 1 stages in flight
#pragma unroll
    for (int st = 0; st < D - 1; ++st)
      if (st < n_st) issue(st);
    for (int st = 0; st < n_st; ++st) {
      // stage st has landed once at most the stages issued after it are
      // outstanding
      const int ahead = n_st - 1 - st < D - 2 ? n_st - 1 - st : D - 2;
      static_for<0, D - 1>([&](auto ki) {
        constexpr int k = decltype(ki)::value;
        if (ahead == k) wait_vmcnt<k * JX>();
      });
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // the buffer of stage st - 1 is free (every MFMA wave has passed this
      // barrier, so it is done with stage st - 1): refill it
      if (st + D - 1 < n_st) issue(st + D - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (S == 1 || (geo & kGeoSecondFinish)) return;  // splitk_reduce_kernel adds the slices
  // in-launch finish: every wave (producers included) takes part
  __syncthreads();
  const OutMap om = make_out_map(y0, y1, split, n_rows, a.out, row_base);
  splitk_finish_vec(a.partial, a.counters, rb, S, row_base, kWresRows, n_rows, M, NT, om, a.out,
                    reinterpret_cast<int*>(lds_raw));
}

}  // namespace fp
