// tile_ring.hpp -- matrix-core tile kernel for y = x . W^T with many tokens
// (M above the small-M kernel's range), bf16 in, fp32 accumulate, bf16 out,
// with the K slice streamed through a ring of LDS stages.
//
// Instruction and operand layout as in tile.hpp: v_mfma_f32_16x16x32_bf16,
// A = 16 weight rows, B = 16 tokens, lane (i16, g) supplies row / token i16
// with the eight bf16 values of piece g (16 bytes) of a 32-wide k step and
// receives D[4g + v][i16].
//
// Work split.  A workgroup of four waves owns a block of 64 weight rows,
// all BM = 16 * B * WM token slots (one block of tokens: M <= BM) and one of
// S slices of the k steps.  The waves form a WR x WM grid: wave (wr, wm)
// multiplies rows 16 * A * wr .. + 16 * A - 1 with tokens 16 * B * wm ..
// + 16 * B - 1 (A x B accumulator tiles), so every LDS fragment it reads
// feeds B or A MFMAs.  The slice is consumed in stages of two k steps (64
// k): a stage is the block's 64 weight rows and BM token rows of 128 bytes
// each, brought into LDS with 16-byte buffer loads that write LDS directly
// (one wave instruction fills 64 slots of 16 bytes; row pitch 9 slots, the
// ninth a zero pad, so the 16 lanes of a quarter-wave hit distinct banks).
// STAGES stage buffers form a ring: while the waves multiply stage t, the
// loads of stages t + 1 .. t + STAGES - 2 are in flight and those of stage
// t + STAGES - 1 are issued.  Weights are read once per call
// (non-temporally); the token rows of a slice are read by every row block
// from L2.
//
// Compared with loading a whole slice at once, the ring lets a slice span
// many stages, so few slices (S ~ CUs / row blocks) cover K and the fp32
// partial sums, S x M x rows, stay small next to the weights.
//
// Reduction order, fixed by (K, S): each output's k steps in order (the
// matrix unit's order inside a step), then the S slice sums in slice order
// (splitk_finish_vec in the launch, or splitk_reduce_kernel in a second
// launch: same order, same bits).  The slice bounds are those of the tile
// kernel for the same S, and so is every output's sequence of MFMA steps:
// both kernels give the same bits.  Nothing depends on a row's position, so
// fused and one-launch-per-projection calls are bitwise equal.
#pragma once

#include "tile.hpp"

namespace fp {

constexpr int kRingRows = 64;   // weight rows per workgroup
constexpr int kRingPitch = 9;   // slots per row and stage: 8 pieces + pad

// 16-byte slots of one stage buffer for BM token slots: whole wave
// instructions of four waves.
__host__ __device__ constexpr int ring_stage_slots(int bm) {
  return ((kRingRows + bm) * kRingPitch + 255) / 256 * 256;
}
__host__ __device__ constexpr int ring_lds_bytes(int bm, int stages) {
  return ring_stage_slots(bm) * 16 * stages;
}

// Leading scalars as in tile_kernel; geo = S, plus kGeoSecondFinish.
template <int WR, int A, int WM, int B, int STAGES>
__global__ void __launch_bounds__(256)
ring_tile_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
                 unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows,
                 int32_t kc, int32_t M, int32_t split, int32_t geo, const Tail a) {
  constexpr int BR = kRingRows;
  constexpr int BM = 16 * B * WM;
  constexpr int P = kRingPitch;
  constexpr int SLOTS = ring_stage_slots(BM);
  constexpr int J = SLOTS / 256;         // load instructions per wave and stage
  constexpr int W_INSTR = BR * P / 64;   // instructions of the weight rows (9)
  static_assert(WR * WM == 4 && 16 * A * WR == BR, "four waves over 64 rows");
  static_assert(STAGES >= 2 && (STAGES - 2) * J <= 63, "vmcnt field");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = geo & 0x1fff;
  const int rb = S == 1 ? (int)blockIdx.x : (int)blockIdx.x / S;
  const int s = S == 1 ? 0 : (int)blockIdx.x - rb * S;
  const int row_base = rb * BR;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int n_steps = (kc + 3) >> 2;
  const int per_s = (n_steps + S - 1) / S;
  const int step0 = s * per_s;
  const int step1 = step0 + per_s < n_steps ? step0 + per_s : n_steps;
  const int n_st = step1 > step0 ? (step1 - step0 + 1) >> 1 : 0;  // stages of 2 steps
  const uint32_t row_bytes = (uint32_t)kc * 16u;

  const __amdgpu_buffer_rsrc_t wr_rsrc = make_rsrc(w, (uint32_t)n_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t xr_rsrc = make_rsrc(x, (uint32_t)(M - 1) * ldx + row_bytes);

  // This lane's slot of each of its J load instructions (instruction
  // idx = j * 4 + wave fills slots 64 idx .. 64 idx + 63 of a stage): the
  // byte offset of its row's piece pc at the slice start, or kOob.
  uint32_t base[J];
  int pcs[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = (j * 4 + wave) * 64 + lane;
    int pc = 0;
    uint32_t off = kOob;
    if (q < BR * P) {
      const int r = q / P;
      pc = q - r * P;
      if (pc < 8 && row_base + r < n_rows)
        off = (uint32_t)(row_base + r) * row_bytes + (uint32_t)pc * 16u;
    } else if (q < (BR + BM) * P) {
      const int t = (q - BR * P) / P;
      pc = q - BR * P - t * P;
      if (pc < 8 && t < M) off = (uint32_t)t * ldx + (uint32_t)pc * 16u;
    }
    base[j] = off;
    pcs[j] = pc;
  }
  // stage st of the slice -> ring buffer st % STAGES
  auto issue = [&](int st) {
    const int step = step0 + 2 * st;
    unsigned char* buf = lds_raw + (size_t)(st % STAGES) * SLOTS * 16;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int idx = j * 4 + wave;
      const bool ok = base[j] != kOob && step + (pcs[j] >> 2) < step1 &&
                      step * 4 + pcs[j] < kc;
      const uint32_t off = ok ? base[j] + (uint32_t)step * 64u : kOob;
      lds_void* dst = (lds_void*)(buf + (size_t)idx * 64 * 16);
      if (idx < W_INSTR)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_rsrc, dst, 16, off, 0, 0, kAuxNt);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr_rsrc, dst, 16, off, 0, 0, 0);
    }
  };

  // prologue: the first STAGES - 1 stages in flight
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < n_st) issue(st);

  const int wr = wave / WM;
  const int wm = wave - wr * WM;
  const int arow = 16 * A * wr + i16;        // tile row of A fragment 0
  const int btok = BR + 16 * B * wm + i16;   // slot row of B fragment 0
  f32x4 acc[A][B];
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int k = 0; k < B; ++k) acc[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < n_st; ++st) {
    // this wave's loads of stage st have landed once at most the stages
    // issued after it (up to STAGES - 2 of them) are outstanding
    const int ahead = n_st - 1 - st < STAGES - 2 ? n_st - 1 - st : STAGES - 2;
    static_for<0, STAGES - 1>([&](auto ki) {
      constexpr int k = decltype(ki)::value;
      if (ahead == k) wait_vmcnt<k * J>();
    });
    // every wave's loads of stage st have landed, and every wave is done
    // with stage st - 1, whose buffer the next issue refills
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st + STAGES - 1 < n_st) issue(st + STAGES - 1);
    __builtin_amdgcn_sched_barrier(0);
    const u32x4* sb = reinterpret_cast<const u32x4*>(lds_raw + (size_t)(st % STAGES) * SLOTS * 16);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (step0 + 2 * st + t < step1) {
        bf16x8 Af[A], Bf[B];
#pragma unroll
        for (int i = 0; i < A; ++i) Af[i] = u4bf8(sb[(arow + 16 * i) * P + 4 * t + g]);
#pragma unroll
        for (int k = 0; k < B; ++k) Bf[k] = u4bf8(sb[(btok + 16 * k) * P + 4 * t + g]);
#pragma unroll
        for (int i = 0; i < A; ++i)
#pragma unroll
          for (int k = 0; k < B; ++k)
            acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[i], Bf[k], acc[i][k], 0, 0, 0);
      }
    }
  }

  // outputs: lane (i16, g) of tile (i, k) holds rows 4g + v of A fragment
  // i, token 16 * B * wm + 16 k + i16
  const OutMap om = make_out_map(y0, y1, split, n_rows, a.out, row_base);
  const int row_w = row_base + 16 * A * wr + 4 * g;
  const int m_w = 16 * B * wm + i16;
  if (S == 1) {
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int row = row_w + 16 * i;
        const int m = m_w + 16 * k;
        if (m < M && row < n_rows) store_y4(om, a.out, row, m, acc[i][k], n_rows);
      }
    return;
  }
  float* partial = a.partial;
  const uint32_t rp = (uint32_t)tile_partial_pitch(n_rows);
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(partial, (uint32_t)S * (uint32_t)M * rp * 4u);
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int row = row_w + 16 * i;
      const int m = m_w + 16 * k;
      if (m < M && row < n_rows)
        store_partial4(prs, ((uint32_t)s * (uint32_t)M + (uint32_t)m) * rp + (uint32_t)row,
                       acc[i][k]);
    }
  if (geo & kGeoSecondFinish) return;  // splitk_reduce_kernel adds the slices
  __syncthreads();  // every wave is done with the stage buffers
  splitk_finish_vec(partial, a.counters, rb, S, row_base, BR, n_rows, M, 256, om, a.out,
                    reinterpret_cast<int*>(lds_raw));
}

}  // namespace fp
