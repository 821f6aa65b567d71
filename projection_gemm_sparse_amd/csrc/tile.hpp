// tile.hpp -- matrix-core tile kernel for y = x . W^T with many tokens
// (M > 8), bf16 in, fp32 accumulate, bf16 out.
//
// Instruction: v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] . B[32 x 16]
// with A = 16 weight rows, B = 16 tokens.  Lane l supplies A's row l%16 and
// B's column l%16 with eight bf16 values of k-slot group g = l/16 (k-slots
// 8g .. 8g+7) and receives D[4g + v][l%16], v = 0..3.  A 32-wide k step is
// four 16-byte pieces of a row; lane (i, g) carries piece g of the step.
//
// Work split.  A workgroup owns NW row tiles of 16 rows (one per wave) and
// one of S slices of the k steps (at most CS * C steps each); every wave
// multiplies its 16 rows with all 16 * MT16 token slots.  Everything the
// workgroup needs is requested at its start, with 16-byte buffer loads
// straight into LDS (each wave instruction fills 1 KiB of LDS, and its 64
// lanes read consecutive pieces of one or two rows, so the loads stay
// contiguous in memory):
//   1. the activation slice, [16 * MT16 tokens] x [slice], shared by the
//      waves (read once per workgroup from L2);
//   2. each wave's weight slice, its 16 rows x [slice], in C chunks of CS
//      steps (every weight byte once per call, non-temporally; W_cat read as
//      stored), which the wave alone reads.
// Out-of-range pieces (rows past the launch, tokens past M, K's tail, the
// next slice's steps) are requested at an offset past the buffer's end and
// read as zero.  The memory counter retires loads in issue order: once the
// activations have landed (weights still in flight) a barrier publishes
// them, then each wave multiplies chunk c as soon as its own chunk-c loads
// have landed, reading both operands from LDS in the instruction's layout
// (odd row pitches keep the 16 lanes of a quarter-wave on distinct banks).
//
// Reduction order, fixed by (K, S): each output's k steps in order inside a
// wave (the matrix unit's own order inside a step), then, with S > 1, the S
// slice sums in slice order, added by the last workgroup of the row block to
// finish.  It depends neither on NW nor on a row's position, so the fused and
// one-launch-per-projection paths give bitwise equal outputs, as do repeats
// and graph replays.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace fp {

// Calls f(integral_constant<int, I>) for I = B .. E-1 (compile-time indices,
// e.g. for s_waitcnt immediates that depend on the loop position).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt with vmcnt <= N (expcnt and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer resource, dword 3 (gfx9)
constexpr uint32_t kOob = 0x80000000u;       // an offset past every buffer's end
constexpr int kAuxNt = 2;                    // buffer cache policy: non-temporal
constexpr int kAuxSc1 = 16;                  // buffer cache policy: sc1 (agent-coherent)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufFlags);
}

// Four consecutive partials of one token, element e of the token-major
// partial buffer pr: one 16-byte store, agent-coherent (sc1) as
// store_partial.
__device__ __forceinline__ void store_partial4(__amdgpu_buffer_rsrc_t pr, uint32_t e, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), pr, e * 4u, 0, kAuxSc1);
}

// LDS layout of a tile launch, in 16-byte slots (host and device):
// activations [16 * mt16 tokens] x [4 * per + 1] (odd pitch: bank spread),
// rounded up to whole wave instructions of 64 slots per wave; then, per wave
// and chunk, [16 rows] x [4 * cs + 1] rounded up to 64 slots.
__host__ __device__ constexpr int tile_x_slots(int mt16, int per, int nw) {
  return ((16 * mt16 * (4 * per + 1) + 64 * nw - 1) / (64 * nw)) * (64 * nw);
}
__host__ __device__ constexpr int tile_w_chunk_slots(int cs) {
  return ((16 * (4 * cs + 1) + 63) / 64) * 64;
}
__host__ __device__ constexpr int tile_slots(int mt16, int per, int nw, int cs, int c) {
  return tile_x_slots(mt16, per, nw) + nw * c * tile_w_chunk_slots(cs);
}

// Arrival counters of the tile launches sit one per 128-byte line: every
// workgroup of a launch arrives at about the same time, and atomics on one
// shared line are serialized (measured on MI355X, 224 workgroups on 28
// counters: 0.3-0.6 us less per call at 9 to 32 tokens once spread).  Row
// blocks have at least 32 rows, so counter rb * 32 stays inside the plan's
// counter words (one per row).
constexpr int kTileCounterStride = 32;

// The S partial slices of four consecutive token slots, added in slice
// order s = 0, 1, ..., S-1 (the first slice as is, then one fp32 add per
// slice and slot).  Loads are issued in groups of GRP before the adds of
// the group: one memory latency per group.  From a buffer resource (byte
// offset `off` of slice 0, `sstride` bytes between slices; agent-coherent
// non-temporal loads: each partial is read once) or from a plain pointer
// (slice stride `vstride` 16-byte vectors).
template <int GRP>
__device__ __forceinline__ f32x4 sum_slices_rsrc(__amdgpu_buffer_rsrc_t pr, uint32_t off,
                                                 uint32_t sstride, int S) {
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += GRP) {
    f32x4 v[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const uint32_t o = s0 + j < S ? off + (uint32_t)(s0 + j) * sstride : kOob;
      v[j] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, kAuxSc1 | kAuxNt));
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (s0 + j < S) {
        const float a0 = sum[0], a1 = sum[1], a2 = sum[2], a3 = sum[3];
        const float b0 = v[j][0], b1 = v[j][1], b2 = v[j][2], b3 = v[j][3];
        sum = s0 + j == 0 ? v[j] : f32x4{a0 + b0, a1 + b1, a2 + b2, a3 + b3};
      }
    }
  }
  return sum;
}

// The second-launch finish's form: plain pointers, non-temporal loads (each
// partial is read once; measured 0.15-0.2 us faster per call at 48..128
// tokens than cached loads).
template <int GRP>
__device__ __forceinline__ f32x4 sum_slices_ptr(const f32x4* p, int64_t vstride, int S) {
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += GRP) {
    f32x4 v[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j)
      v[j] = s0 + j < S ? __builtin_nontemporal_load(p + (s0 + j) * vstride) : sum;
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (s0 + j < S) {
        const float a0 = sum[0], a1 = sum[1], a2 = sum[2], a3 = sum[3];
        const float b0 = v[j][0], b1 = v[j][1], b2 = v[j][2], b3 = v[j][3];
        sum = s0 + j == 0 ? v[j] : f32x4{a0 + b0, a1 + b1, a2 + b2, a3 + b3};
      }
    }
  }
  return sum;
}

// Split-K partials of the tile kernels are token-major: slice s, token m,
// row r at partial[(s * M + m) * RP + r] with the row pitch RP = n_rows
// rounded up to a multiple of 4 (16 bytes), so that a lane's four
// accumulator rows of one token are one 16-byte run and a finish that takes
// four consecutive rows per thread reads and writes whole lines.
__host__ __device__ constexpr int tile_partial_pitch(int n_rows) { return (n_rows + 3) & ~3; }

// Sum of the S partial slices of a row block, in slice order, by the
// workgroup that arrives last; four consecutive rows of one token per
// thread and step (stored and read agent-coherent).
__device__ __forceinline__ void splitk_finish_vec(const float* partial, uint32_t* counters,
                                                  int rb, int S, int row_base, int R,
                                                  int n_rows, int M, int nthreads,
                                                  const OutMap& os, const OutTable& tab,
                                                  int* flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // this thread's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add((gu32*)(counters + rb * kTileCounterStride), 1u,
                                                __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == (unsigned)(S - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (*flag == 0) return;
  const int rows_here = n_rows - row_base < R ? n_rows - row_base : R;
  const int quads = (rows_here + 3) >> 2;
  const int n_vec = M * quads;
  const uint32_t rp = (uint32_t)tile_partial_pitch(n_rows);
  const uint32_t sstride = (uint32_t)M * rp * 4u;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(partial, (uint32_t)S * sstride);
  for (int t = threadIdx.x; t < n_vec; t += nthreads) {
    const int m = t / quads;
    const int row = row_base + 4 * (t - m * quads);
    const uint32_t off = ((uint32_t)m * rp + (uint32_t)row) * 4u;
    // the S slices in groups (8, or 16 above 8 slices): all loads of a
    // group are issued before the first add, then added in slice order
    const f32x4 sum = S <= 8 ? sum_slices_rsrc<8>(pr, off, sstride, S)
                             : sum_slices_rsrc<16>(pr, off, sstride, S);
    store_y4(os, tab, row, m, sum, n_rows);
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store((gu32*)(counters + rb * kTileCounterStride), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Leading scalars preloaded into SGPRs (see skinny_kernel for w, x, y0, y1,
// ldx, n_rows, kc, M, split); geo = S (k-step slices across workgroups),
// plus kGeoSecondFinish: the slices are added by splitk_reduce_kernel in a
// second launch instead of by the last workgroup of each row block.
constexpr int kGeoSecondFinish = 1 << 30;
// Threads per workgroup of the second-launch finish.
constexpr int kReduceThreads = 64;

template <int MT16, int NW, int CS, int C>
__global__ void __launch_bounds__(NW * 64)
tile_kernel(const unsigned char* __restrict__ w, const unsigned char* __restrict__ x,
            unsigned char* y0, unsigned char* y1, uint32_t ldx, int32_t n_rows, int32_t kc,
            int32_t M, int32_t split, int32_t geo, const Tail a) {
  constexpr int NT = NW * 64;
  constexpr int WP = 4 * CS + 1;                     // weight row pitch (slots)
  constexpr int WCS = tile_w_chunk_slots(CS);        // slots of one wave chunk
  constexpr int JW = WCS / 64;                       // wave instructions per chunk
  static_assert(C * JW <= 63, "vmcnt field");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = geo & 0x1fff;
  const int rb = S == 1 ? (int)blockIdx.x : (int)blockIdx.x / S;
  const int s = S == 1 ? 0 : (int)blockIdx.x - rb * S;
  const int row_base = rb * (16 * NW);
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int n_steps = (kc + 3) >> 2;
  const int per_s = (n_steps + S - 1) / S;  // <= CS * C
  const int step0 = s * per_s;
  const int step1 = step0 + per_s < n_steps ? step0 + per_s : n_steps;
  const int xpitch = 4 * per_s + 1;         // activation row pitch (slots)
  const int x_slots = tile_x_slots(MT16, per_s, NW);
  const uint32_t row_bytes = (uint32_t)kc * 16u;
  const int wrow0 = row_base + wave * 16;   // first row of this wave's tile

  // 1. activation slice -> LDS: slot q = token * xpitch + piece
  {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(M - 1) * ldx + row_bytes);
    for (int base = wave * 64; base < x_slots; base += NT) {
      const int q = base + lane;
      const int tok = q / xpitch;
      const int pc = q - tok * xpitch;
      const int piece = step0 * 4 + pc;
      const bool ok = tok < M && pc < 4 * (step1 - step0) && piece < kc;
      const uint32_t off = ok ? (uint32_t)tok * ldx + (uint32_t)piece * 16u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_void*)(lds_raw + (size_t)base * 16), 16, off, 0, 0, 0);
    }
  }
  // 2. this wave's weight slice -> LDS, chunk by chunk: slot q of chunk c is
  //    row q / WP of the tile, piece q % WP of the chunk's CS steps
  unsigned char* wl = lds_raw + (size_t)(x_slots + wave * C * WCS) * 16;
  {
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)n_rows * row_bytes);
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        const int q = j * 64 + lane;
        const int r = q / WP;
        const int pc = q - r * WP;
        const int step = step0 + c * CS + (pc >> 2);
        const int piece = step * 4 + (pc & 3);
        const bool ok = wrow0 + r < n_rows && pc < 4 * CS && step < step1 && piece < kc;
        const uint32_t off = ok ? (uint32_t)(wrow0 + r) * row_bytes + (uint32_t)piece * 16u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_void*)(wl + (size_t)(c * WCS + j * 64) * 16), 16, off, 0, 0, kAuxNt);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const OutMap om = make_out_map(y0, y1, split, n_rows, a.out, row_base);
  float* partial = a.partial;
  uint32_t* counters = a.counters;
  if (S > 1) asm volatile("" : "+s"(partial), "+s"(counters));
  __builtin_amdgcn_sched_barrier(0);
  // the activations have landed once at most C * JW loads (this wave's
  // weights) are outstanding; the barrier publishes every wave's share
  wait_vmcnt<C * JW>();
  // an execution barrier only: __syncthreads() would also wait for every
  // outstanding load (including this wave's weights), defeating the overlap
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 3. chunks in order, each as soon as this wave's loads of it have landed
  f32x4 acc[MT16];
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4* xs = reinterpret_cast<const u32x4*>(lds_raw);
  const u32x4* ws4 = reinterpret_cast<const u32x4*>(wl);
  static_for<0, C>([&](auto ci) {
    constexpr int c = decltype(ci)::value;
    wait_vmcnt<(C - 1 - c) * JW>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < CS; ++t) {
      const int st = c * CS + t;  // step within the slice
      if (step0 + st < step1) {
        const bf16x8 A = u4bf8(ws4[c * WCS + i16 * WP + 4 * t + g]);
#pragma unroll
        for (int mt = 0; mt < MT16; ++mt) {
          const bf16x8 B = u4bf8(xs[(mt * 16 + i16) * xpitch + st * 4 + g]);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[mt], 0, 0, 0);
        }
      }
    }
  });

  // 4. outputs: lane (i16, g) holds rows 4g + v of the wave's tile, token
  //    mt * 16 + i16
  const int row_t = wrow0 + 4 * g;
  if (S == 1) {
#pragma unroll
    for (int mt = 0; mt < MT16; ++mt) {
      const int m = mt * 16 + i16;
      if (m < M && row_t < n_rows) store_y4(om, a.out, row_t, m, acc[mt], n_rows);
    }
    return;
  }
  const uint32_t rp = (uint32_t)tile_partial_pitch(n_rows);
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(partial, (uint32_t)S * (uint32_t)M * rp * 4u);
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) {
    const int m = mt * 16 + i16;
    if (m < M && row_t < n_rows)
      store_partial4(prs, ((uint32_t)s * (uint32_t)M + (uint32_t)m) * rp + (uint32_t)row_t,
                     acc[mt]);
  }
  if (geo & kGeoSecondFinish) return;  // splitk_reduce_kernel adds the slices
  __syncthreads();  // every wave is done reading the activation slice
  splitk_finish_vec(partial, counters, rb, S, row_base, 16 * NW, n_rows, M, NT, om, a.out,
                    reinterpret_cast<int*>(lds_raw));
}

// The second-launch finish: defined only in the unit that compiles the non-template
// kernels (k_misc.hip), so each is emitted once.
#ifdef FP_DEFINE_MISC_KERNELS
// The second-launch finish of a split tile launch: thread t adds, for token
// t / ceil(n_rows / 4) and four consecutive rows, the S slices of the
// partials in slice order -- the order of splitk_finish_vec, so both
// finishes give the same bits -- and stores the outputs rounded once (a
// wave's 64 threads read and write 256 consecutive rows of one token).  A
// launch of many tokens has large partials per row block (S * 16 * NW rows
// * 16 * MT16 tokens); one workgroup per row block re-reading them (the
// in-launch finish) is then slower than spreading the sum over the whole
// GPU after a kernel boundary.
__global__ void __launch_bounds__(kReduceThreads)
splitk_reduce_kernel(const float* __restrict__ partial, int32_t n_rows, int32_t M, int32_t S,
                     const OutTable tab) {
  const int quads = (n_rows + 3) >> 2;
  const int64_t t = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
  if (t >= (int64_t)M * quads) return;
  const int m = (int)(t / quads);
  const int row = 4 * (int)(t - (int64_t)m * quads);
  const int64_t rp = tile_partial_pitch(n_rows);
  const f32x4* p = reinterpret_cast<const f32x4*>(partial + (int64_t)m * rp + row);
  const int64_t vstride = (int64_t)M * rp / 4;  // 16-byte vectors between slices
  // the slices in groups (8, or 16 above 8 slices): all loads of a group
  // are issued before the first add (one load latency per group, not per
  // slice), then added in slice order
  const f32x4 sum = S <= 8 ? sum_slices_ptr<8>(p, vstride, S) : sum_slices_ptr<16>(p, vstride, S);
  // the segment of the quad's first row (the last one that starts at or
  // before it) and the next one; store_y4 searches every segment for rows
  // past those
  int seg = 0;
  for (int i = 1; i < tab.n_seg; ++i) seg = row >= tab.begin[i] ? i : seg;
  const int seg1 = seg + 1 < tab.n_seg ? seg + 1 : seg;
  OutMap om;
  om.y0 = tab.y[seg];
  om.y1 = tab.y[seg1];
  om.b0 = tab.begin[seg];
  om.b1 = tab.begin[seg + 1];
  om.e1 = tab.begin[seg1 + 1];
  om.n_seg = tab.n_seg;
  om.ts0 = 1.0f;
  om.ts1 = 1.0f;
  store_y4(om, tab, row, m, sum, n_rows);
}

#endif  // FP_DEFINE_MISC_KERNELS

}  // namespace fp
