// mfma.hpp -- MFMA tile kernel for y = x . W^T (bf16 in, fp32 accumulate),
// used for token counts above the skinny kernel's range.
//
// Instruction: v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] . B[32 x 16].
// A is a 16-row tile of the weight (rows = outputs), B is 16 token rows of x
// seen as columns, D[i][j] is output row i for token j.  Lane l supplies A's
// row l%16 and B's column l%16 with eight bf16 values of one k-slot group
// g = l/16; the sum over the 32 k-slots is independent of which k a slot
// carries as long as A and B carry the same k in the same slot.  Lane group
// g of a 128-wide k tile therefore loads the 64 contiguous bytes at
// k = 32g .. 32g+31 of its row (four 16-byte loads), and step t of the
// tile feeds the t-th of them: each weight row is read as 256-byte runs, and
// W_cat is used as stored (plain row-major, no pre-swizzled copy, so writes
// through the projection views stay valid).
// D layout: lane l holds D[4*(l/16) + v][l%16], v = 0..3.
//
// Work split.  A workgroup owns 16 * GR rows (GR row groups of one 16-row
// tile) and one of S slices of K; the PK waves of a row group split the
// slice into PK parts of KTW consecutive 128-wide k tiles.  All of a wave's
// weight loads are issued up front.  The activation tile of the slice
// (all token rows, zero-padded to 16 * MT16) is staged once per workgroup
// in LDS and shared by every wave.
// Reduction order: MFMA k-steps in tile order inside a wave, then the PK
// waves in wave order (LDS), then the S slices in slice order (the
// last-arriving workgroup, as in the skinny kernel).  It depends only on
// (K, KTW, PK, S), never on the rows of a launch.
#pragma once

#include "common.hpp"

namespace fp {

struct MfmaArgs {
  const unsigned char* x;  // activations, M rows
  int64_t ldx_bytes;       // row stride of x in bytes (multiple of 16)
  int64_t row_bytes;       // K * 2
  int32_t M;               // token rows, <= 16 * MT16
  int32_t kc;              // 16-byte chunks per row (8 bf16 each)
  int32_t GR;              // 16-row groups per workgroup
  int32_t PK;              // waves per row group (K parts of a slice)
  int32_t S;               // K slices
  int32_t ktw;             // 128-wide k tiles per wave (<= KTW)
  RowSpace rs;
  float* partial;          // [S][n_rows][M] when S > 1
  uint32_t* counters;
};

template <int MT16, int KTW>
__global__ void __launch_bounds__(mfma_max_threads(MT16, KTW))
mfma_kernel(const MfmaArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pk = wave % a.PK;
  const int gr = wave / a.PK;
  const int rb = blockIdx.x / a.S;
  const int s = blockIdx.x - rb * a.S;
  const int64_t R = 16 * (int64_t)a.GR;
  const int64_t row_base = (int64_t)rb * R;
  const int64_t row0 = row_base + 16 * (int64_t)gr;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int slice_tiles = a.PK * a.ktw;            // k tiles per slice
  const int kt_slice0 = s * slice_tiles;           // first tile of the slice
  const int kt_wave0 = kt_slice0 + pk * a.ktw;     // first tile of the wave

  // 1. weight loads of the wave: row row0 + i16, tiles kt_wave0 .. +ktw
  u32x4 wv[KTW][4];
  {
    const unsigned char* wrow = row_pointer(a.rs, row0 + i16, a.row_bytes);
#pragma unroll
    for (int kk = 0; kk < KTW; ++kk) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = (kt_wave0 + kk) * 16 + 4 * g + t;
        if (wrow != nullptr && kk < a.ktw && c < a.kc) {
          wv[kk][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow) + c);
        } else {
          wv[kk][t] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  // 2. stage the slice's activation tile: rows 0 .. 16*MT16-1 (zero past M),
  //    chunks [kt_slice0*16, (kt_slice0 + slice_tiles)*16), row pitch padded
  //    by 16 bytes to spread LDS banks.
  const int slice_chunks = slice_tiles * 16;
  const int pitch = slice_chunks + 1;  // in 16-byte units
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  {
    const int total = 16 * MT16 * slice_chunks;
    for (int e = tid; e < total; e += blockDim.x) {
      const int m = e / slice_chunks;
      const int cc = e - m * slice_chunks;
      const int c = kt_slice0 * 16 + cc;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (m < a.M && c < a.kc) {
        val = reinterpret_cast<const u32x4*>(a.x + (int64_t)m * a.ldx_bytes)[c];
      }
      xs[m * pitch + cc] = val;
    }
  }
  __syncthreads();

  // 3. MFMA over the wave's tiles
  f32x4 acc[MT16];
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KTW; ++kk) {
    if (kk < a.ktw) {
      const int cc0 = (pk * a.ktw + kk) * 16 + 4 * g;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 A = u4bf8(wv[kk][t]);
#pragma unroll
        for (int mt = 0; mt < MT16; ++mt) {
          const bf16x8 B = u4bf8(xs[(mt * 16 + i16) * pitch + cc0 + t]);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[mt], 0, 0, 0);
        }
      }
    }
  }

  // 4. across the PK waves of the row group (LDS, wave order), then store
  //    or write the slice's partial sums.
  const int64_t n_rows = a.rs.n_rows;
  float* red = reinterpret_cast<float*>(lds + (size_t)16 * MT16 * pitch * 16);
  if (a.PK > 1) {
    __syncthreads();  // LDS activation tile no longer read after this point
#pragma unroll
    for (int mt = 0; mt < MT16; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        red[(((gr * a.PK + pk) * MT16 + mt) * 4 + v) * 64 + lane] = acc[mt][v];
      }
    }
    __syncthreads();
    const int n_el = a.GR * MT16 * 256;
    for (int e = tid; e < n_el; e += blockDim.x) {
      const int ln = e & 63;
      const int v = (e >> 6) & 3;
      const int mt = (e >> 8) % MT16;
      const int g2 = (e >> 8) / MT16;
      const float* rp = red + ((g2 * a.PK * MT16 + mt) * 4 + v) * 64 + ln;
      float sum = rp[0];
      for (int q = 1; q < a.PK; ++q) sum += rp[q * MT16 * 256];
      const int64_t row = row_base + 16 * (int64_t)g2 + 4 * (ln >> 4) + v;
      const int m = mt * 16 + (ln & 15);
      if (m < a.M && row < n_rows) {
        if (a.S == 1) store_out<true>(a.rs, row, m, sum);
        else a.partial[((int64_t)s * n_rows + row) * a.M + m] = sum;
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT16; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + 4 * g + v;
        const int m = mt * 16 + i16;
        if (m < a.M && row < n_rows) {
          if (a.S == 1) store_out<true>(a.rs, row, m, acc[mt][v]);
          else a.partial[((int64_t)s * n_rows + row) * a.M + m] = acc[mt][v];
        }
      }
    }
  }
  if (a.S == 1) return;
  int* flag = reinterpret_cast<int*>(red + (a.PK > 1 ? a.GR * a.PK * MT16 * 256 : 0));
  splitk_finish<true>(a.rs, a.partial, a.counters, rb, a.S, row_base, R, a.M, flag);
}

}  // namespace fp
