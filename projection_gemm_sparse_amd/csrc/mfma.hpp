// mfma.hpp -- MFMA tile kernel for y = x . W^T (bf16 in, fp32 accumulate).
//
// Instruction: v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] . B[32 x 16].
// Lane l supplies A's row l%16 and B's column l%16 with eight bf16 values of
// k-slot group g = l/16; the product sums over the 32 k-slots, so any k may
// sit in a slot as long as A and B carry the same k there.  D layout: lane l
// holds D[4*(l/16) + v][l%16], v = 0..3.
//
// K-slice packing.  With few tokens the 16 MFMA columns are mostly idle, so
// the 16 A rows are filled with RT = 16/Q weight rows times Q sub-slices of
// the wave's K range, and the 16 B columns with TQ = 16/Q tokens times the
// same Q sub-slices: A row s*RT + r carries weight row r on sub-slice s, B
// column s*TQ + m carries token m on sub-slice s.  The useful outputs are
// the diagonal blocks D[s*RT + r][s*TQ + m]; adding them over s gives row r,
// token m.  Q = 1 is the ordinary 16-row tile (and may hold several
// 16-token tiles, MT16 of them); Q = 2, 4, 8 give 8-, 4- and 2-row tiles for
// up to 8, 4 and 2 tokens, so a launch has enough workgroups without
// splitting K across workgroups.
//
// Loads.  The sub-slices are interleaved at 16-byte granularity: at MFMA
// step t of k tile kk, the lane of k-slot group g on sub-slice s reads chunk
//   kk*16Q + 4Q*t + Q*g + s
// of the wave's range, so the 4Q lanes that carry one weight row read 64Q
// contiguous bytes per load instruction (256 B at Q = 4).  W_cat is used as
// stored (no pre-swizzled copy, so writes through the projection views stay
// valid).  Every weight load of a wave is issued before its first MFMA.
// Activations come straight from global memory (they are small and stay in
// L2) unless several row groups of a workgroup share them (large token
// counts): then the workgroup stages its activation slice in LDS once,
// issuing all of a thread's staging loads before its first LDS store.
//
// Work split.  A workgroup owns GR row groups of RT rows and one of S
// slices of K; the PK waves of a row group split the slice into PK parts of
// KTW k tiles of 16Q chunks each.
// Reduction order: MFMA steps in tile order inside a wave; then, per output,
// the Q sub-slices and PK waves in a fixed order (sub-slice outer, wave
// inner) through LDS; then the S slices in slice order (last-arriving
// workgroup, see splitk_finish).  It depends only on (K, Q, KTW, PK, S).
#pragma once

#include "common.hpp"

namespace fp {

// Leading scalars preloaded into SGPRs (see skinny_kernel for w_pre, x_pre,
// y0, y1, ldx, n_rows_pre, kc_pre, M_pre, split); geo_pre = GR | PK << 8 |
// log2(ktw) << 16 | S << 18 (row groups per workgroup, waves per row group,
// k tiles per wave, K slices across workgroups).
template <int Q, int MT16, int KTW, bool XLDS>
__global__ void __launch_bounds__(mfma_max_threads(MT16, KTW, XLDS))
mfma_kernel(const unsigned char* __restrict__ w_pre, const unsigned char* __restrict__ x_pre,
            unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows_pre,
            int32_t kc_pre, int32_t M_pre, int32_t split, int32_t geo_pre, const Tail a) {
  constexpr int RT = 16 / Q;  // weight rows per row group
  constexpr int TQ = 16 / Q;  // tokens per sub-slice
  constexpr int MC = Q == 1 ? 16 : TQ;  // token columns kept per tile
  constexpr int TILE = RT * MC;         // useful outputs of one sub-slice tile
  static_assert(Q == 1 || MT16 == 1, "k-slice packing uses one token tile");
  static_assert(!XLDS || Q == 1, "staged activations only for unpacked tiles");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int GRv = geo_pre & 0xff;
  const int PKv = (geo_pre >> 8) & 0xff;
  const int ktw = 1 << ((geo_pre >> 16) & 3);
  const int Sv = geo_pre >> 18;
  const int Mv = M_pre;
  const int kc = kc_pre;
  const int pk = GRv == 1 ? wave : wave % PKv;
  const int gr = GRv == 1 ? 0 : wave / PKv;
  const int rb = Sv == 1 ? (int)blockIdx.x : (int)blockIdx.x / Sv;
  const int s = Sv == 1 ? 0 : (int)blockIdx.x - rb * Sv;
  const int64_t R = (int64_t)RT * GRv;
  const int64_t row_base = (int64_t)rb * R;
  const int64_t row0 = row_base + (int64_t)RT * gr;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int nthreads = GRv * PKv * 64;
  const int64_t ldx_pre = ldx;
  const int wave_chunks = 16 * Q * ktw;             // chunks of a wave
  const int slice_chunks = PKv * wave_chunks;       // chunks of a K slice
  const int cw0 = s * slice_chunks + pk * wave_chunks;

  // A lane: weight row (i16 % RT) on sub-slice (i16 / RT)
  const int a_sub = i16 / RT;
  const int a_row = i16 - a_sub * RT;
  // B lane: token (i16 % TQ) on sub-slice (i16 / TQ)
  const int b_sub = i16 / TQ;
  const int b_tok = i16 - b_sub * TQ;

  // Weight loads of the wave, all issued before the first MFMA.
  u32x4 wv[KTW][4];
  // Loads are branch-free: out-of-range elements load a clamped valid
  // address (rows past the end are computed and dropped), and weight chunks
  // past K or past the wave's tiles are replaced by zero only when consumed,
  // so the loads form one straight-line sequence consumed in issue order.
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  auto w_chunk = [&](int kk, int t) { return cw0 + kk * 16 * Q + 4 * Q * t + Q * g + a_sub; };
  auto load_weights = [&]() {
    const int64_t n_rows_l = n_rows_pre;
    const int64_t row = row0 + a_row;
    const u32x4* wrow = reinterpret_cast<const u32x4*>(
        w_pre + (row < n_rows_l ? row : n_rows_l - 1) * ((int64_t)kc * 16));
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = w_chunk(kk, t);
        wv[kk][t] = __builtin_nontemporal_load(wrow + (c < kc ? c : kc - 1));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // 1. activations and weights.  Read per wave, the activations (from L2)
  //    are loaded first so the weights can be consumed as they land; staged
  //    in LDS, the weight loads go first so they are in flight while the
  //    workgroup stages its activation slice.
  u32x4 xv[XLDS ? 1 : MT16][XLDS ? 1 : KTW][4];
  const int pitch = slice_chunks + 1;  // LDS row pitch in 16-byte units
  if constexpr (!XLDS) {
#pragma unroll
    for (int mt = 0; mt < MT16; ++mt) {
      const int m = mt * 16 + (Q == 1 ? i16 : b_tok);
      const int mc = m < Mv ? m : Mv - 1;
      const u32x4* xrow = reinterpret_cast<const u32x4*>(x_pre + (int64_t)mc * ldx_pre);
#pragma unroll
      for (int kk = 0; kk < KTW; ++kk) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = cw0 + kk * 16 * Q + 4 * Q * t + Q * g + b_sub;
          xv[mt][kk][t] = xrow[c < kc ? c : kc - 1];
        }
      }
    }
    load_weights();
    __builtin_amdgcn_sched_barrier(0);
  } else {
    load_weights();
    __builtin_amdgcn_sched_barrier(0);
    // rows 0 .. 16*MT16-1 (zero past M) of the slice's chunks; each thread
    // loads up to 8 chunks into registers before storing any of them
    u32x4* xs = reinterpret_cast<u32x4*>(lds);
    const int total = 16 * MT16 * slice_chunks;
    for (int base = 0; base < total; base += 8 * nthreads) {
      u32x4 st[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * nthreads + tid;
        st[e] = u32x4{0u, 0u, 0u, 0u};
        if (idx < total) {
          const int m = idx / slice_chunks;
          const int cc = idx - m * slice_chunks;
          const int c = s * slice_chunks + cc;
          if (m < Mv && c < kc) {
            st[e] = reinterpret_cast<const u32x4*>(x_pre + (int64_t)m * ldx_pre)[c];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * nthreads + tid;
        if (idx < total) {
          const int m = idx / slice_chunks;
          const int cc = idx - m * slice_chunks;
          xs[m * pitch + cc] = st[e];
        }
      }
    }
    __syncthreads();
  }

  const OutMap os = make_out_map(y0, y1, split, (int)n_rows_pre, a.out, (int)row_base);
  __builtin_amdgcn_sched_barrier(0);

  // 2. MFMA steps in tile order
  f32x4 acc[MT16];
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KTW; ++kk) {
    if (kk < ktw) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // consume the weight loads in issue order (progressive vmcnt waits)
        __builtin_amdgcn_sched_barrier(0);
        const bool a_ok = w_chunk(kk, t) < kc;
        const bf16x8 A = u4bf8(a_ok ? wv[kk][t] : zero4);
#pragma unroll
        for (int mt = 0; mt < MT16; ++mt) {
          bf16x8 B;
          if constexpr (XLDS) {
            const u32x4* xs = reinterpret_cast<const u32x4*>(lds);
            const int cc = pk * wave_chunks + kk * 16 + 4 * t + g;
            B = u4bf8(xs[(mt * 16 + i16) * pitch + cc]);
          } else {
            const int m = mt * 16 + (Q == 1 ? i16 : b_tok);
            const int c = cw0 + kk * 16 * Q + 4 * Q * t + Q * g + b_sub;
            B = u4bf8((m < Mv && c < kc) ? xv[mt][kk][t] : zero4);
          }
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[mt], 0, 0, 0);
        }
      }
    }
  }

  // 3. useful outputs to LDS: red[((gr*PK + pk)*Q + sub)*MT16 + mt][r][m];
  //    it reuses the staged activations' space once every wave is done
  //    with them
  if constexpr (XLDS) __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int arow = 4 * g + v;  // D row
      const int sa = arow / RT;
      const int sb = i16 / TQ;     // D column i16
      if (Q == 1 || sa == sb) {
        const int r = arow - sa * RT;
        const int m = i16 - sb * TQ;
        const int slot = ((gr * PKv + pk) * Q + sa) * MT16 + mt;
        red[slot * TILE + r * MC + m] = acc[mt][v];
      }
    }
  }
  __syncthreads();

  // 4. per output: sub-slices, then waves, in fixed order; store or write
  //    the slice's partial sum
  const int64_t n_rows = n_rows_pre;
  const int mcols = MC * MT16;
  const int n_out = GRv * RT * mcols;
  for (int o = tid; o < n_out; o += nthreads) {
    const int g2 = o / (RT * mcols);
    const int rem = o - g2 * (RT * mcols);
    const int r = rem / mcols;
    const int mm = rem - r * mcols;
    const int mt = mm / MC;
    const int m16 = mm - mt * MC;
    const int64_t row = row_base + (int64_t)RT * g2 + r;
    if (mm >= Mv || row >= n_rows) continue;
    float sum = 0.0f;
#pragma unroll
    for (int sub = 0; sub < Q; ++sub) {
      for (int q = 0; q < PKv; ++q) {
        const int slot = ((g2 * PKv + q) * Q + sub) * MT16 + mt;
        const float val = red[slot * TILE + r * MC + m16];
        sum = (sub == 0 && q == 0) ? val : sum + val;
      }
    }
    if (Sv == 1) {
      store_y<true>(os, a.out, (int)row, mm, sum);
    } else {
      store_partial(a.partial + ((int64_t)s * n_rows + row) * Mv + mm, sum);
    }
  }
  if (Sv == 1) return;
  int* flag = reinterpret_cast<int*>(red + (size_t)GRv * PKv * Q * MT16 * TILE);
  splitk_finish<true>((int)n_rows, a.partial, a.counters, rb, Sv, row_base, R, Mv,
                      GRv * PKv * 64, os, a.out, flag);
}

}  // namespace fp
