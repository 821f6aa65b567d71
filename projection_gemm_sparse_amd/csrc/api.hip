// api.hip -- host side of libfusedproj: plan bookkeeping, argument checks
// (all before any HIP call), tiling choice and kernel launches.
//
// The load-time half follows "tinygemm2 for the DeepSeek-V4.1 hidden-state
// projections" (TensorRT-LLM PR #20636), Description: the projection weights
// are copied once into one row-concatenated buffer and each projection gets
// a view into it; the decode-time half is one launch over all rows with the
// per-projection outputs written densely.  The host "supported" predicate
// and the refusal of unserved shapes follow the dense-MLP commit of
// "Staircase: GLM-5.2 NVFP4 low-latency decode target for Rubin (TP16)"
// (PR #20502).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "../../include/fusedproj.h"
#include "skinny.hpp"
#include "smfma.hpp"
#include "tile.hpp"
#include "tile_ring.hpp"
#include "tile_wres.hpp"
#include "epilogue.hpp"
#include "mxfp8.hpp"
#include "stream.hpp"
#include "kernels.h"

namespace {

constexpr uint64_t kPlanMagic = 0x66757365'6470726full;  // "fusedpro"
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kSkinnyMaxM = 8;      // largest M the skinny kernel serves
// Largest M the small-M matrix-core kernel serves: three token halves for
// bf16, two for block-scaled weights.
constexpr int kSmallMfmaMaxM = 24;
// Two row tiles per wave only for workgroups of at least this many K parts
// (K >= 2048 in bf16): with fewer waves per workgroup the two-tile form
// leaves a CU too few waves.  Small-M workgroups are counted resident up to
// kSmfmaMaxResident per CU (fewer where the CU's waves do not allow them).
// Measured on MI355X against the former limits (two tiles from any K, two
// workgroups per CU, ties to more rows), us per call: K = 768, 6144 rows
// M = 8 5.47 -> 4.24, M = 16 7.88 -> 6.48; K = 512, 6144 rows M = 12 10.53
// -> 6.27; K = 1024, 4096 rows M = 12 6.58 -> 4.88; K = 1536, 6144 rows
// M = 24 14.00 -> 9.26; K = 2048, 6144 rows M = 8 6.92 -> 6.57; the
// largest loss K = 512, 4096 rows M = 24 7.24 -> 7.74.
constexpr int kSmfmaTwoTileMinParts = 8;
constexpr int kSmfmaMaxResident = 4;
// Most slices the ring tile kernel's default takes where a CU gets two
// workgroups (the measured range).
constexpr int64_t kRingMaxSlices = 16;
constexpr int kSmallMfmaMaxMMx = 16;
// Crossover to the tile kernels (smallest M on the MFMA tile path),
// measured on MI355X at K = 5120, 1792 rows: the small-M matrix-core
// kernel with two token halves serves M = 9..16 and with three halves M =
// 17..24 faster than the tile kernels.
constexpr int kDefaultMfmaMinM = 25;
// Smallest M the small-M matrix-core kernel serves by default; the
// vector-ALU kernel runs below it.  Measured on MI355X at K = 5120, 1792
// rows (bf16): the vector-ALU kernel is faster up to M = 2 (5.22 vs 5.41
// us), the matrix-core kernel from M = 3 (5.41 vs 5.60 us at M = 3, 5.51 vs
// 5.68 at M = 4, 5.89 vs 6.64 at M = 8), where the vector-ALU kernel's
// multiply-adds and 64-value lane reduction start to show after the last
// weights land.
constexpr int kDefaultSmallMfmaMinM = 3;
// MX weights: measured at the same shape, the vector-ALU kernel stays
// faster through M = 4 (MXFP8 4.95 vs 5.36 us, MXFP4 4.37 vs 4.60).
constexpr int kDefaultSmallMfmaMinMMx = 5;
constexpr int kCus = 256;           // MI355X compute units
// Largest bf16 plan (weight bytes) of more than eight rows per CU that the
// small-M kernel serves from M = 3 (see default_small_mfma_min_m).
constexpr int64_t kSmallMfmaMaxBytesM3 = (int64_t)25200000;
// bf16: where the small-M kernel starts depends on the rows a CU gets and
// on the plan's size.  A sweep of both kernels' default layouts at M = 3..8
// (K = 1024..7168, 256..6144 rows) on MI355X: with at most two rows per CU
// the vector-ALU kernel is ahead at every M up to 8 (by up to 35 %: 512
// rows, K = 7168, M = 5 / 8, and 39 % at M = 3); with three or four rows
// per CU the small-M kernel is ahead from M = 3 at K <= 2048 (1024 rows,
// K = 2048, M = 8: 0.77 of the vector-ALU time), the vector-ALU kernel up
// to M = 4 at larger K (up to M = 8 with three rows per CU); with four to
// eight rows per CU the small-M kernel from M = 3 (the headline shape);
// above eight rows per CU the small-M kernel from M = 3 at K <= 4096 up to
// 25.2 MB of weights (K = 2048, 6144 rows M = 3: 0.97 of the vector-ALU
// time; K = 4096, 3072 rows: 0.94 at M = 4) and the vector-ALU kernel
// through M = 4 otherwise (K = 5120, 2304 rows: 1.05; the three-way
// fused-A shape, 33.8 MB: 8.02 vs 8.27 us at M = 3; K = 4096, 6144 rows:
// 1.14).  Over the 126 measured cells at M = 3 / 4 the rule loses 1.9 us
// in all against the best kernel (at most 7 % in one cell), where the
// former rule (small-M from M = 3 up to eight rows per CU) lost 21.3 us
// (39 %).
int default_small_mfma_min_m(int32_t dtype, int64_t K, int64_t n_total) {
  if (dtype == FP_MXFP8 || dtype == FP_MXFP4 || dtype == FP_NVFP4) return kDefaultSmallMfmaMinMMx;
  const int64_t cus = kCus;
  if (n_total <= 2 * cus) return kSkinnyMaxM + 1;
  if (n_total <= 4 * cus) {
    if (K <= 2048) return kDefaultSmallMfmaMinM;
    return n_total <= 3 * cus ? kSkinnyMaxM + 1 : kDefaultSmallMfmaMinMMx;
  }
  if (n_total <= 8 * cus) return kDefaultSmallMfmaMinM;
  const int64_t w_bytes = n_total * K * 2;
  return K <= 4096 && w_bytes <= kSmallMfmaMaxBytesM3 ? kDefaultSmallMfmaMinM
                                                      : kDefaultSmallMfmaMinMMx;
}
constexpr int64_t kMaxRows = (int64_t)1 << 30;  // rows and chunks per row, 32-bit indexing

thread_local int32_t g_last_hip = 0;

struct Tiling {
  int path = 0;   // FP_PATH_*
  int kparts = 0; // P or PK
  int chunks = 0; // CJ or KTW
  int splits = 0; // S
  int rows = 0;   // RW or GR
  int groups = 0; // G (skinny)
  int mt = 0;     // skinny MT bucket or mfma MT16
};

}  // namespace

struct fp_plan_s {
  uint64_t magic;
  int32_t dtype;
  int32_t esize;
  int64_t K;
  int64_t kc;  // 16-byte chunks per row (MXFP8: 8-element units, K / 8)
  int64_t wrow;  // bytes per weight row (MXFP8: K codes + K / 32 scales)
  int32_t n_proj;
  int64_t N[FP_MAX_PROJ];
  int64_t off[FP_MAX_PROJ];
  int64_t n_total;
  unsigned char* w_cat;
  unsigned char* ws;
  size_t ws_bytes;
  int64_t max_M;
  bool out_f32;     // bf16 operands with fp32 outputs (vector-ALU kernel only)
  int32_t osize;    // output element size
  int64_t mfma_min_m;
  int64_t small_mfma_min_m;
  float tscale[FP_MAX_PROJ];  // NVFP4: each projection's fp32 tensor scale (1 otherwise)
  bool has_override[FP_MAX_M + 1];
  fp_tiling override_t[FP_MAX_M + 1];
};

namespace {

int64_t skinny_max_m(const fp_plan_s* p) { return p->out_f32 ? 16 : kSkinnyMaxM; }

// Per dtype: activation element size, bytes per weight row and the 16-byte
// weight chunks per row the kernels count; false if K does not fit the
// kernels' 16-byte chunking (MXFP8: K a multiple of 512, so that a packed row
// of K codes and K/32 scales is a whole number of chunks).
bool dtype_geometry(int32_t dtype, int64_t K, int* esize, int64_t* wrow, int64_t* kc) {
  if (K < 1) return false;
  if (dtype == FP_BF16 || dtype == FP_F32) {
    const int es = dtype == FP_BF16 ? 2 : 4;
    if ((K * es) % 16 != 0) return false;
    *esize = es;
    *wrow = K * es;
    *kc = K * es / 16;
    return true;
  }
  if (dtype == FP_MXFP8 || dtype == FP_MXFP4 || dtype == FP_NVFP4) {
    // units of 8 elements (8 or 4 code bytes), as the bf16 kernel's chunks
    if (K % 512 != 0) return false;
    *esize = 2;
    *wrow = dtype == FP_MXFP8 ? K + K / 32 : dtype == FP_MXFP4 ? K / 2 + K / 32 : K / 2 + K / 16;
    *kc = K / 8;
    return true;
  }
  return false;
}

int skinny_var(const fp_plan_s* p) {
  return p->dtype == FP_MXFP8   ? fp::kVarMx8
         : p->dtype == FP_MXFP4 ? fp::kVarMx4
         : p->dtype == FP_NVFP4 ? fp::kVarNv4
                                : fp::kVarPlain;
}

// Block-scaled weight formats (MXFP8, MXFP4, NVFP4): decoded in the kernels,
// served up to 8 tokens by the vector-ALU and small-M matrix-core kernels.
bool is_mx(int32_t dtype) { return dtype == FP_MXFP8 || dtype == FP_MXFP4 || dtype == FP_NVFP4; }

// The vector-ALU kernel a tiling launches, nullptr where none is compiled
// (fp32 outputs: 1, 2, 4 and, up to 8 tokens, 8 rows per wave; gate/up
// pairs: even rows; long chunk runs: one or two rows).  The row search and
// the validity check ask this, so neither can pick a missing kernel.
const void* skinny_fn(const fp_plan_s* p, const Tiling& t, bool pairs) {
  return pairs ? fpk::skinny_pairs(t.mt, t.chunks, t.rows)
         : p->out_f32 ? fpk::skinny_f32out(t.mt, t.chunks, t.rows)
         : is_mx(p->dtype) ? fpk::skinny_mx(skinny_var(p), t.mt, t.chunks, t.rows)
                           : fpk::skinny(p->dtype == FP_BF16, t.mt, t.chunks, t.rows);
}

bool dtype_known(int32_t dtype) {
  return dtype == FP_BF16 || dtype == FP_F32 || dtype == FP_MXFP8 || dtype == FP_MXFP4 ||
         dtype == FP_NVFP4;
}

std::mutex g_mu;
std::unordered_set<const fp_plan_s*>& live_plans() {
  static std::unordered_set<const fp_plan_s*> s;
  return s;
}

bool plan_ok(const fp_plan_s* p) {
  if (p == nullptr) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (live_plans().count(p) == 0) return false;
  return p->magic == kPlanMagic;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int skinny_mt(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

// Largest M the vector-ALU kernel serves for a plan (fp32-output plans: 16).
int64_t skinny_max_m(const fp_plan_s* p);
int mfma_mt16(int64_t M) {
  const int64_t t = ceil_div(M, 16);
  return t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : t <= 8 ? 8 : 16;
}

int64_t counters_bytes(int64_t n_total) {
  return ceil_div(n_total * 4, 256) * 256;
}

// ------------------------------------------------------------------ tilings
// Plan-level part (summation order): depends on dtype, K, the M bucket and
// the plan's total rows only.
void default_skinny_order(int32_t dtype, int64_t kc, int64_t n_total, int mt,
                          Tiling* t) {
  (void)n_total;
  // One workgroup covers a whole row whenever it can (16 waves * 64 lanes *
  // 2 chunks): finishing a K split across workgroups costs three dependent
  // memory round trips, more than the idle CUs of a short launch lose.
  // The 16-token bucket (fp32 router outputs) holds twice the activations
  // per chunk: two chunks per lane keep its workgroups within the register
  // budget, and its thread bound (512) takes at most 8 K parts, so rows of
  // more than 1024 chunks (bf16 K > 8192) split K across workgroups.
  const int64_t S = ceil_div(kc, (mt >= 16 ? 8 : 16) * 64 * 2);
  const int64_t per = ceil_div(kc, S);
  const int64_t CJ = std::max<int64_t>(ceil_div(per, 16 * 64), mt >= 16 ? 2 : 1);
  const int64_t P = ceil_div(per, 64 * CJ);
  t->path = S > 1 ? FP_PATH_SKINNY_SPLITK : FP_PATH_SKINNY;
  t->kparts = (int)P;
  t->chunks = (int)CJ;
  t->splits = (int)S;
  (void)dtype;
}

// Tile (MFMA) kernel.  The order field is S, the k-step slices across
// workgroups (chosen from K and the M bucket only); the launch fields are
// NW, the 16-row tiles per workgroup, and the compiled slice bound (k steps
// staged in LDS per wave: CS steps per chunk times C chunks).
constexpr int kTilePers[] = {8, 10, 16, 20, 40};  // compiled slice bounds (k steps)
constexpr int kTileNws[] = {2, 4, 8};

// Ring tile kernel: a tiling of the MFMA path whose chunks field is a ring
// depth (stage buffers) selects it; kparts is then 4 (64-row blocks).
constexpr int kRingStages[] = {3, 4, 6};
// Weight-resident tile kernel: a tiling of the MFMA path whose chunks
// field is kWresCode selects it; kparts is then 4 (64-row blocks).
constexpr int kWresCode = 2;
bool is_wres(const Tiling& t) { return t.chunks == kWresCode; }
// Stages of two k steps one slice spans with S slices.
int64_t wres_stages(int64_t kc, int64_t S) {
  const int64_t per = ceil_div(ceil_div(kc, 4), S);
  return ceil_div(per, 2);
}
bool wres_fits(int64_t kc, int mt16, int64_t S) {
  return mt16 >= 2 && mt16 <= 16 && wres_stages(kc, S) <= fp::wres_max_stages(16 * mt16);
}

bool is_ring(const Tiling& t) {
  for (int st : kRingStages)
    if (t.chunks == st) return true;
  return false;
}
size_t ring_lds(int mt16, int stages) {
  return (size_t)fp::ring_lds_bytes(16 * mt16, stages);
}
bool ring_fits(int mt16, int stages) {
  const int J = fp::ring_stage_slots(16 * mt16) / 256;
  return ring_lds(mt16, stages) <= kMaxLds && (stages - 2) * J <= 63;
}

int tile_per_bound(int64_t per) {
  for (int b : kTilePers)
    if (per <= b) return b;
  return 0;
}

// Chunking of a compiled register bound: CS steps per chunk, C chunks.
void tile_chunks(int bound, int* cs, int* c) {
  *cs = (bound == 8 || bound == 16) ? 4 : 5;
  *c = bound / *cs;
}

size_t tile_lds(int mt16, int64_t per, int nw) {
  const int b = tile_per_bound(per);
  if (b == 0) return SIZE_MAX;
  int cs, c;
  tile_chunks(b, &cs, &c);
  return (size_t)fp::tile_slots(mt16, (int)per, nw, cs, c) * 16;
}

// Resident workgroups per CU for a tile launch (LDS and wave slots).
int64_t tile_resident(int mt16, int64_t per, int nw) {
  const size_t lds = std::max<size_t>(tile_lds(mt16, per, nw), 16);
  return std::max<int64_t>(1, std::min<int64_t>((int64_t)(kMaxLds / lds), 16 / nw));
}

// Best NW for a launch of n_rows rows with S slices (0 if none fits): one
// round of workgroups, as many busy CUs as possible, then fewer rows per CU.
// NW for a launch with S slices: four row tiles per workgroup (eight from
// 128 tokens) when that fits in LDS, else the largest that does (0: none).
int tile_pick_nw(int mt16, int64_t n_steps, int64_t S, int64_t n_rows) {
  (void)n_rows;
  const int64_t per = ceil_div(n_steps, S);
  const int pref = mt16 >= 8 ? 8 : 4;
  if (tile_lds(mt16, per, pref) <= kMaxLds) return pref;
  for (int nw : {8, 4, 2})
    if (tile_lds(mt16, per, nw) <= kMaxLds) return nw;
  return 0;
}

// The ring tile kernel addresses the weights with 32-bit buffer offsets.
bool ring_addressable(int64_t n_rows, int64_t kc) {
  return n_rows * kc * 16 < ((int64_t)1 << 31);
}

// Slices of the tile kernel for few tokens: the fewest whose slice fills a
// compiled slice bound nearly (no wasted LDS rows) and fits in LDS; 0 if
// none.
int64_t tile_pick_slices(int64_t n_steps, int mt16, int nw) {
  for (int64_t S = 1; S <= n_steps && S <= 0x1fff; ++S) {
    const int64_t per = ceil_div(n_steps, S);
    const int b = tile_per_bound(per);
    if (b == 0 || per + 2 < b) continue;
    if (tile_lds(mt16, per, nw) > kMaxLds) continue;
    return S;
  }
  return 0;
}

// Slice count of a split tile launch over `blocks` 64-row blocks that
// minimises the busiest CU's share of a row block, ceil(blocks S / CUs) /
// S, among slices of an even number of k steps (128-byte aligned: a slice
// that starts mid-line costs 30-40 %) and at least 4, with at most
// `per_cu` workgroups per CU and beyond kRingMaxSlices only one (small
// plans; `capped`: never); for the weight-resident kernel (`wres`, mt16
// token tiles) only slices that fit its LDS.  Ties go to more slices.
// S = 0: none.
struct Slices {
  int64_t S = 0;
  int64_t w = 1;  // workgroups on the busiest CU
};
Slices balanced_slices(int64_t n_steps, int64_t blocks, int64_t per_cu, int64_t kc, bool wres,
                       int mt16, bool capped = false) {
  Slices best;
  for (int64_t S = 1; blocks * S <= per_cu * kCus && S <= 0x1fff; ++S) {
    const int64_t per = ceil_div(n_steps, S);
    if (per < 4 || per % 2 != 0) continue;
    if (S > kRingMaxSlices && (capped || blocks * S > kCus)) continue;
    if (wres && !wres_fits(kc, mt16, S)) continue;
    const int64_t w = ceil_div(blocks * S, kCus);
    if (best.S == 0 || w * best.S <= best.w * S) {
      best.S = S;
      best.w = w;
    }
  }
  return best;
}

bool default_mfma_order(int64_t kc, int64_t M, int64_t n_total, Tiling* t) {
  const int mt16 = mfma_mt16(M);
  const int64_t n_steps = ceil_div(kc, 4);
  const int64_t blocks = ceil_div(n_total, fp::kRingRows);
  // Up to 32 tokens the tile and weight-resident kernels run one workgroup
  // per (64-row block, slice) and need them all resident at once; a plan
  // with more blocks than that allows takes the ring tile kernel (measured
  // on MI355X at K = 6144, 2752 rows, 9 slices: 14.88 / 15.19 us at M = 17 /
  // 32 against 19.18 / 19.17 for the tile kernel).
  // 17..32 tokens (where the small-M kernel does not serve): the
  // weight-resident kernel with balanced slices of one workgroup per CU
  // (its LDS holds one), or the ring kernel with balanced slices of up to
  // two per CU where that gives the busiest CU a smaller share.  Measured
  // on MI355X at M = 32 (us per call) against the former choice (the tile
  // kernel's fewest slices, weight-resident where one round): K = 5120,
  // 1024 rows weight-resident 16 slices 8.2 against 8 slices 9.5; K =
  // 7168, 1024 rows 16 slices 9.2 against 12 (19 steps) 10.9; K = 4096,
  // 1024 rows 7.8 against 7 slices 10.1; K = 2048, 1024 rows 6.7 against 4
  // slices 8.2; at most 8 % above the best slice count of either kernel
  // (K = 2048, 2048 rows).
  if (mt16 == 2 && ring_addressable(n_total, kc)) {
    // at most kRingMaxSlices here (a 192-row plan at K = 7168: 12 slices
    // 9.8 us at M = 17, 74 slices of 4 steps 10.3)
    const Slices w = balanced_slices(n_steps, blocks, 1, kc, true, mt16, true);
    const Slices r = balanced_slices(n_steps, blocks, 2, kc, false, mt16, true);
    // equal shares: the weight-resident kernel where both take the same
    // slices, the ring where it gets there with more (two per CU)
    const bool wres_first = w.S > 0 && (r.S == 0 || w.w * r.S < r.w * w.S ||
                                        (w.w * r.S == r.w * w.S && w.S >= r.S));
    if (wres_first) {
      t->path = FP_PATH_MFMA;
      t->splits = (int)w.S;
      t->kparts = 4;
      t->chunks = kWresCode;
      return true;
    }
    if (r.S > 0) {
      t->path = FP_PATH_MFMA;
      t->splits = (int)r.S;
      t->kparts = 4;
      t->chunks = 4;
      return true;
    }
  }
  const int64_t few_pick = mt16 <= 2 ? tile_pick_slices(n_steps, mt16, 4) : 0;
  const bool ring = mt16 >= 4 || (few_pick > 0 && blocks * few_pick > kCus &&
                                  ring_addressable(n_total, kc));
  if (ring) {
    // The ring tile kernel, four stage buffers (three for 256-token blocks,
    // the most LDS holds), over the plan's 64-row blocks: one workgroup per
    // CU, and up to 64 tokens up to 9 slices while that keeps at most three
    // per CU (then balanced below); at least two stages per slice.  Measured
    // on MI355X (second-launch finish from 17 tokens): K = 5120, 1792 rows,
    // 9 slices: 12.9 us at M = 64 and 16.8 at M = 128, against 19.7 / 22.0
    // for the tile kernel; K = 6144, 2752 rows: 9 slices ahead of 5, 6 and 7
    // up to 64 tokens (M = 17: 14.88 against 17.51 .. 16.13; M = 64: 18.38
    // against 21.05 with 5) and of 12 (three workgroups on some CUs), but
    // one workgroup per CU above 64 tokens (M = 96: 5 slices 25.32, 9 slices
    // 28.62, the weight-resident kernel at 9 slices 26.06).  The choice
    // depends on (K, M bucket, plan rows) only.
    int64_t S = std::max<int64_t>(1, kCus / blocks);
    if (mt16 <= 4) {
      // Up to 64 tokens (two rings fit in a CU's LDS): the slice count that
      // minimises the busiest CU's share of a row block, ceil(blocks S /
      // CUs) / S, among slices of an even number of k steps (128-byte
      // aligned: a slice that starts mid-line costs 30-40 %) and at least 4,
      // at most two workgroups per CU, and beyond kRingMaxSlices slices only
      // one workgroup per CU (small plans); ties to more slices.  Fitted to a sweep of S = 4..16 on MI355X (K =
      // 2048..7168, 1024..4096 rows, M = 16 / 32 / 64): within 0.6 % of the
      // best slice count on average, 7 % at worst, where the former rule
      // (toward 9, at most three per CU) lost up to 30 %.  Examples (us per
      // call): K = 7168, 4096 rows M = 32 8 slices 17.9 against 25.3 with 9;
      // K = 4096, 2048 rows M = 64 16 slices 10.7 against 16.1 with 9; 1792
      // rows at K = 5120 keep 9 (one per CU), 2752 rows at K = 6144 keep 11.
      const Slices bs = balanced_slices(n_steps, blocks, 2, kc, false, mt16);
      if (bs.S > 0) S = bs.S;
      else S = std::max<int64_t>(S, std::min<int64_t>(9, 3 * kCus / blocks));
    }
    S = std::min<int64_t>(S, std::max<int64_t>(1, n_steps / 4));
    S = std::min<int64_t>(S, 0x1fff);
    t->path = FP_PATH_MFMA;
    t->splits = (int)S;
    t->kparts = 4;
    t->chunks = mt16 >= 16 ? 3 : 4;
    // 65..128 tokens: the weight-resident kernel (same slices, same bits)
    // when its slice fits in LDS; measured on MI355X at K = 5120, 1792 rows,
    // 9 slices: 16.2 vs 17.0 us at M = 128, 15.3 vs 15.8 at M = 96 (the
    // ring kernel stays ahead at 64 tokens: 13.0 vs 13.9)
    if (mt16 == 8 && wres_fits(kc, mt16, S)) t->chunks = kWresCode;
    return true;
  }
  // Measured on MI355X (K = 5120, 1792 rows): four row tiles per workgroup,
  // and the fewest slices whose slice fills a compiled slice bound nearly
  // (no wasted LDS rows) and fits in LDS.  The choice depends on (K, M
  // bucket, plan rows) only, so every launch of a plan adds the same slices
  // in the same order.
  const int nw = 4;
  int64_t pick = few_pick;
  if (pick == 0) {
    // short K or odd shapes: any slice count that fits
    for (int64_t S = 1; S <= n_steps && S <= 0x1fff && pick == 0; ++S) {
      const int64_t per = ceil_div(n_steps, S);
      if (tile_per_bound(per) == 0) continue;
      for (int w : kTileNws)
        if (tile_lds(mt16, per, w) <= kMaxLds) pick = S;
    }
  }
  if (pick == 0) return false;
  t->path = FP_PATH_MFMA;
  t->splits = (int)pick;
  t->kparts = 0;  // NW, per launch
  t->chunks = 0;  // register bound, per launch
  // 17..32 tokens: the weight-resident kernel with the same slices (same
  // bits) when its slice fits in LDS and the launch stays within one round
  // of workgroups; measured on MI355X at K = 5120, 1792 rows, 8 slices:
  // 10.0 vs 10.9 us at M = 17, 10.8 vs 11.2 at M = 32
  if (mt16 == 2 && wres_fits(kc, mt16, pick) &&
      ceil_div(n_total, fp::kWresRows) * pick <= kCus) {
    t->kparts = 4;
    t->chunks = kWresCode;
  }
  return true;
}

// Small-M matrix-core order fields: PK waves of KT steps (8 chunks each).
bool default_smfma_order(int64_t kc, Tiling* t) {
  const int64_t steps = ceil_div(kc, 8);
  const int KT = steps <= 64 ? 4 : steps <= 128 ? 8 : 16;
  const int64_t PK = ceil_div(steps, KT);
  if (PK > fp::kMaxWaveParts) return false;
  t->path = FP_PATH_MFMA_SMALL;
  t->kparts = (int)PK;
  t->chunks = KT;
  t->splits = 1;
  return true;
}

// Launch-level part (work per workgroup): may depend on the launch's rows.
// Rows per workgroup R = G * RW are chosen so that every workgroup is
// resident at once (one round: all weight loads in flight together) and,
// among those, to minimise the rows of the busiest CU,
// ceil(ceil(n_rows / R) / CUs) * R (ties: the larger R, fewer workgroups);
// RW <= min(8, 64 / MT) and G * P waves fit one workgroup.  Without a
// one-round choice the largest R is taken.
void resolve_skinny_rows(const fp_plan_s* p, int64_t n_rows, int mt, Tiling* t, bool pairs) {
  const int var = skinny_var(p);
  const int rw_max = std::min(8, 64 / mt);
  const int64_t rows = n_rows * t->splits;  // work units: (row, K slice)
  if (t->rows > 0 && t->groups > 0) return;
  int best_rw = pairs ? 2 : 1, best_g = 1;
  int64_t best_cost = INT64_MAX;
  for (int rw = pairs ? 2 : 1; rw <= rw_max; rw += pairs ? 2 : 1) {
    if (t->rows > 0 && rw != t->rows) continue;
    Tiling built = *t;
    built.rows = rw;
    if (skinny_fn(p, built, pairs) == nullptr) continue;
    // only layouts whose workgroup fits the instantiation's thread bound
    // (long fp32 rows at 5..8 tokens: seven rows per workgroup would need
    // more registers than ten K parts leave)
    const int g_cap = fp::skinny_max_threads(t->mt, rw, t->chunks, var) / (64 * t->kparts);
    for (int g = 1; g <= g_cap; ++g) {
      if (t->groups > 0 && g != t->groups) continue;
      const int64_t R = (int64_t)rw * g;
      const int64_t nb = ceil_div(rows, R);
      // resident workgroups per CU: 32 wave slots; the kernels' register
      // use (under 100 VGPRs) lets two workgroups of up to 16 waves share
      // a CU, more are not assumed
      const int waves = g * t->kparts;
      const int64_t resident = std::max(1, std::min(2, 32 / waves));
      const bool one_round = nb <= resident * kCus;
      const int64_t cost = one_round ? ceil_div(nb, kCus) * R : INT64_MAX / 2 - R;
      if (cost < best_cost || (cost == best_cost && R > (int64_t)best_rw * best_g)) {
        best_cost = cost;
        best_rw = rw;
        best_g = g;
      }
    }
  }
  t->rows = best_rw;
  t->groups = best_g;
}

// Token slots of the small-M kernel: one, two or three halves of 8.
int smfma_mt(int64_t M) { return M > 16 ? 24 : M > 8 ? 16 : 8; }

// Small-M kernel rows: `rows` 1..8 is one tile of that many rows per wave;
// an even 10..16 is two tiles of rows / 2 (bf16, not gate/up) that share
// each wave's activation operand.
int smfma_tiles(const Tiling& t) { return t.rows > 8 ? 2 : 1; }
int smfma_rt(const Tiling& t) { return t.rows / smfma_tiles(t); }

// Waves of the small-M kernel one CU holds, from the register estimate of
// its instantiation (KT steps, MH token halves, TT row tiles).  It never
// exceeds what the compiled kernels reach on gfx950 (KT 8: 24 waves with
// one half and one tile, 16 with two halves or two tiles, 12 with both;
// the estimate gives 20, 12, 16 and 12).
int smfma_cu_waves(int kt, int mh, int tt) {
  const int regs = fp::smfma_regs(kt, mh, tt);
  return 4 * std::max(1, std::min(8, 512 / ((regs + 7) / 8 * 8)));
}

// Rows per workgroup R = G * TT * RT.  Every workgroup loads the whole
// activation block once per row group, so the bytes a CU takes in are
// (workgroups on the CU) x (R weight rows + G x mt activation rows); the
// choice keeps every workgroup resident at once (one round) and, among
// those, minimises that figure for the busiest CU (ties: fewer row groups,
// then the larger R; block-scaled kernels: the larger R), with at most
// kSmfmaMaxResident workgroups per CU counted resident (block-scaled: two)
// and the waves a CU holds taken from the kernel's register estimate
// (bf16; block-scaled kernels: 32).  Two tiles per wave
// are offered to bf16 plans (not gate/up) of kSmfmaTwoTileMinParts K parts
// or more, or of any K where no one-round layout exists without them.
// Without a one-round choice the largest R is taken; the result says
// whether a one-round layout exists.
//
// Measured on MI355X (weights rotated past the MALL, us per call): K =
// 6144, 2752 rows, M = 8: two tiles of 6 rows per wave (230 workgroups)
// 8.86 against one tile of 6 (459) 10.61; M = 5: 8.54 vs 8.88.  Short K,
// where the former rule (rows on the busiest CU alone) took one-row groups
// that each reload the activations, M = 8: K = 512, 1792 rows 3.27 vs 7.03
// (seven groups of one row); K = 1024, 2048 rows 3.00 vs 5.01; K = 2048
// 3.86 vs 4.69.
bool resolve_smfma_rows_pass(int64_t n_rows, Tiling* t, bool pairs, bool bf16, bool few_parts_tt2);

bool resolve_smfma_rows(int64_t n_rows, Tiling* t, bool pairs, bool bf16) {
  if (t->rows > 0 && t->groups > 0) return true;
  // two tiles per wave for workgroups of few K parts only where no one-round
  // layout exists without them (then the largest rows win: 65536 rows, K =
  // 1024, M = 5: two tiles of 8 rows 24.5 us against one tile 27.2)
  Tiling one = *t;
  if (resolve_smfma_rows_pass(n_rows, &one, pairs, bf16, false)) {
    *t = one;
    return true;
  }
  return resolve_smfma_rows_pass(n_rows, t, pairs, bf16, true);
}

bool resolve_smfma_rows_pass(int64_t n_rows, Tiling* t, bool pairs, bool bf16,
                             bool few_parts_tt2) {
  int best_rows = pairs ? 2 : 1, best_g = 1;
  int64_t best_cost = INT64_MAX;
  const int mh = t->mt / 8;
  for (int tt = 1; tt <= 2; ++tt) {
    if (tt == 2 && (!bf16 || pairs || mh > 2)) continue;
    if (tt == 2 && !few_parts_tt2 && t->kparts < kSmfmaTwoTileMinParts) continue;
    for (int rt = pairs ? 2 : 1; rt <= 8; rt += pairs ? 2 : 1) {
      if (tt == 2 && rt < 5) continue;  // rows <= 8 denote one tile
      const int rows = tt * rt;
      if (t->rows > 0 && rows != t->rows) continue;
      const int g_cap =
          std::max(1, fp::smfma_max_threads(t->chunks, mh, tt) / (64 * t->kparts));
      for (int g = 1; g <= g_cap; ++g) {
        if (t->groups > 0 && g != t->groups) continue;
        // the cross-wave sums of every (row group, tile, token half) in LDS
        if ((int64_t)g * tt * mh * 2 * 64 * fp::kMaxWaveParts * 4 > kMaxLds) continue;
        const int64_t R = (int64_t)rows * g;
        const int64_t nb = ceil_div(n_rows, R);
        const int waves = g * t->kparts;
        if (waves * 64 > fp::smfma_max_threads(t->chunks, mh, tt)) continue;
        // block-scaled kernels: 32 waves per CU assumed, as measured for
        // their rows choice
        const int cu_waves = bf16 ? smfma_cu_waves(t->chunks, mh, tt) : 32;
        // block-scaled kernels: two per CU and ties to more rows, as
        // measured for their rows choice
        const int64_t resident =
            std::max(1, std::min(bf16 ? kSmfmaMaxResident : 2, cu_waves / waves));
        const bool one_round = nb <= resident * kCus;
        const int64_t cost =
            one_round ? ceil_div(nb, kCus) * (R + (int64_t)g * t->mt) : INT64_MAX / 2 - R;
        const bool fewer_groups = bf16 && g < best_g;
        const bool same_groups = !bf16 || g == best_g;
        if (cost < best_cost || (cost == best_cost && (fewer_groups ||
                                                     (same_groups && R > (int64_t)best_rows * best_g)))) {
          best_cost = cost;
          best_rows = rows;
          best_g = g;
        }
      }
    }
  }
  t->rows = best_rows;
  t->groups = best_g;
  return best_cost < INT64_MAX / 4;  // a one-round layout was found
}

size_t smfma_lds(const Tiling& t) {
  return (size_t)t.groups * smfma_tiles(t) * (t.mt / 8) * 2 * 64 * fp::kMaxWaveParts * 4;
}

size_t skinny_lds(const Tiling& t) {
  const int V = t.rows * t.mt;
  int VP = 1;
  while (VP < V) VP <<= 1;
  return (size_t)t.groups * VP * fp::kMaxWaveParts * 4 + 16;
}

// Partial-sum bytes one row block of a split tile launch leaves for its
// finish, above which the slices are added in a second launch spread over
// the GPU instead of by the row block's last workgroup.
constexpr int64_t kSecondFinishBytes = 64 * 1024;

void resolve_tile_launch(const fp_plan_s* p, int64_t n_rows, Tiling* t) {
  if (is_ring(*t) || is_wres(*t)) {
    if (t->kparts <= 0) t->kparts = 4;
    t->rows = 1;
    if (t->groups <= 0) {
      const int64_t block_bytes = (int64_t)t->splits * fp::kRingRows * 16 * t->mt * 4;
      t->groups = t->splits > 1 && block_bytes > kSecondFinishBytes ? 2 : 1;
    }
    return;
  }
  const int64_t n_steps = ceil_div(p->kc, 4);
  const int64_t per = ceil_div(n_steps, std::max(1, t->splits));
  if (t->kparts <= 0) t->kparts = tile_pick_nw(t->mt, n_steps, t->splits, n_rows);
  if (t->chunks <= 0) t->chunks = tile_per_bound(per);
  t->rows = 1;  // unused by the tile kernel
  // groups: 1 = slices finished in the launch, 2 = in a second launch
  if (t->groups <= 0) {
    const int64_t block_bytes = (int64_t)t->splits * 16 * t->kparts * 16 * t->mt * 4;
    t->groups = t->splits > 1 && block_bytes > kSecondFinishBytes ? 2 : 1;
  }
}

// Partial-sum floats a tiling needs for a launch of n_rows rows and M tokens.
int64_t partial_floats(const Tiling& t, int64_t n_rows, int64_t M) {
  if (t.splits <= 1) return 0;
  // the tile kernels keep token-major slices with a 4-row pitch
  if (t.path == FP_PATH_MFMA) return (int64_t)t.splits * M * fp::tile_partial_pitch((int)n_rows);
  return (int64_t)t.splits * n_rows * M;
}

// Where a launch keeps its split-K state: the arrival counters (one uint32
// per row, zero between calls) and the fp32 partial sums, with the bytes
// available for each.  Normally the plan's workspace; fp_forward_noalloc
// uses the library's static scratch instead.
struct WsView {
  unsigned char* counters;
  unsigned char* partial;
  int64_t counter_bytes;
  int64_t partial_bytes;  // negative: no room at all
};

WsView plan_ws(const fp_plan_s* p) {
  const int64_t cb = counters_bytes(p->n_total);
  WsView w;
  w.counters = p->ws;
  w.partial = p->ws + cb;
  w.counter_bytes = cb;
  const size_t rest = p->ws_bytes < (size_t)cb ? 0 : p->ws_bytes - (size_t)cb;
  w.partial_bytes = p->ws_bytes < (size_t)cb           ? -1
                    : rest > (size_t)INT64_MAX ? INT64_MAX
                                               : (int64_t)rest;
  return w;
}

const void* mfma_fn(const Tiling& t);
const void* smfma_fn(const Tiling& t, bool pairs, int32_t dtype, int64_t M);

bool tiling_valid(const fp_plan_s* p, int64_t M, int64_t n_rows, const Tiling& t,
                  const WsView& ws, bool pairs) {
  if (t.splits < 1 || t.kparts < 1 || t.chunks < 1 || t.rows < 1) return false;
  // packed into 8- and 16-bit fields of the kernels' scalar arguments
  if (t.splits > 0x1fff || t.kparts > 0xff || t.rows > 0xff || t.groups > 0xff) return false;
  if (t.path == FP_PATH_MFMA && is_wres(t)) {
    if (p->dtype != FP_BF16 || t.kparts != 4 || !wres_fits(p->kc, t.mt, t.splits)) return false;
    if (t.groups != 1 && t.groups != 2) return false;
    if (16 * (int64_t)t.mt < M) return false;
    if ((int64_t)t.splits * n_rows * 16 * t.mt * 4 >= ((int64_t)1 << 31)) return false;
    if (n_rows * p->kc * 16 >= ((int64_t)1 << 31)) return false;
  } else if (t.path == FP_PATH_MFMA && is_ring(t)) {
    if (p->dtype != FP_BF16 || t.kparts != 4 || !ring_fits(t.mt, t.chunks)) return false;
    if (t.groups != 1 && t.groups != 2) return false;
    if (16 * (int64_t)t.mt < M) return false;
    // buffer offsets are 32-bit, with 0x80000000 reserved as out of range
    if ((int64_t)t.splits * n_rows * 16 * t.mt * 4 >= ((int64_t)1 << 31)) return false;
    if (!ring_addressable(n_rows, p->kc)) return false;
  } else if (t.path == FP_PATH_MFMA) {
    if (p->dtype != FP_BF16) return false;
    const int64_t n_steps = ceil_div(p->kc, 4);
    const int64_t per = ceil_div(n_steps, t.splits);
    bool nw_ok = false, per_ok = false;
    for (int nw : kTileNws) nw_ok = nw_ok || nw == t.kparts;
    for (int b : kTilePers) per_ok = per_ok || b == t.chunks;
    if (!nw_ok || !per_ok || per > t.chunks) return false;
    if (t.groups != 1 && t.groups != 2) return false;
    if (tile_lds(t.mt, per, t.kparts) > kMaxLds) return false;
    if (16 * (int64_t)t.mt < M) return false;
    // buffer offsets are 32-bit
    if ((int64_t)t.splits * n_rows * 16 * t.mt * 4 >= ((int64_t)1 << 31)) return false;
  } else if (t.path == FP_PATH_MFMA_SMALL) {
    if (!(p->dtype == FP_BF16 || is_mx(p->dtype))) return false;
    if (M > kSmallMfmaMaxM || t.mt < M) return false;
    if (is_mx(p->dtype) && (M > kSmallMfmaMaxMMx || t.mt > 16)) return false;
    if (t.rows > 8 && t.mt > 16) return false;  // two tiles: at most two halves
    if (!(t.chunks == 4 || t.chunks == 8 || t.chunks == 16)) return false;
    if (t.splits != 1 || t.kparts > fp::kMaxWaveParts || t.rows > 16 || t.groups < 1) return false;
    if (t.rows > 8 && (t.rows % 2 != 0 || p->dtype != FP_BF16)) return false;
    if ((int64_t)t.groups * t.kparts * 64 >
        fp::smfma_max_threads(t.chunks, t.mt / 8, smfma_tiles(t)))
      return false;
    if ((int64_t)t.kparts * t.chunks * 8 < p->kc) return false;
    if (smfma_lds(t) > kMaxLds) return false;
  } else if (t.path == FP_PATH_SKINNY || t.path == FP_PATH_SKINNY_SPLITK) {
    if (M > skinny_max_m(p) || t.kparts > fp::kMaxWaveParts) return false;
    // fp32 outputs are held to 1e-5 * S: every output passes through at
    // most 8 + 6 + 15 adds before the slices and S - 1 after them, which
    // 128 slices keep below the 166 that bound allows
    if ((p->dtype == FP_F32 || p->out_f32) && t.splits > 128) return false;
    if (t.mt > 8 && !(p->out_f32 && t.chunks <= 2 && t.rows <= 4)) return false;
    if (t.rows > 8 || t.rows * t.mt > 64) return false;
    const bool cj_ok = t.chunks <= 2 || (t.mt <= 2 && t.rows <= 2 &&
        (t.chunks == 4 || t.chunks == 5 || t.chunks == 6 || t.chunks == 8 ||
         t.chunks == 10 || t.chunks == 12));
    if (!cj_ok) return false;
    if (t.groups < 1) return false;
    if (is_mx(p->dtype) && t.chunks > 2) return false;
    if ((int64_t)t.groups * t.kparts * 64 >
        fp::skinny_max_threads(t.mt, t.rows, t.chunks, skinny_var(p)))
      return false;
    if ((int64_t)t.splits * t.kparts * 64 * t.chunks < p->kc) return false;
    if (skinny_lds(t) > kMaxLds) return false;
  } else {
    return false;
  }
  // only a tiling whose kernel is compiled
  const void* fn = t.path == FP_PATH_MFMA         ? mfma_fn(t)
                   : t.path == FP_PATH_MFMA_SMALL ? smfma_fn(t, pairs, p->dtype, M)
                                                  : skinny_fn(p, t, pairs);
  if (fn == nullptr) return false;
  // the tile kernels' in-launch finish addresses the partials with 32-bit
  // byte offsets
  const int64_t pbytes = partial_floats(t, n_rows, M) * 4;
  if (t.path == FP_PATH_MFMA && pbytes >= ((int64_t)1 << 32)) return false;
  return counters_bytes(p->n_total) <= ws.counter_bytes && pbytes <= ws.partial_bytes;
}

// The tiling for (M, launch rows); the summation-order fields come from the
// plan's default or the user's override for M and never from n_rows.
bool choose_tiling(const fp_plan_s* p, int64_t M, int64_t n_rows, Tiling* t,
                   bool pairs = false, const WsView* ws = nullptr) {
  *t = Tiling();
  // outputs are indexed m * N_i + r with 32-bit integers
  if (M * n_rows > INT32_MAX) return false;
  if (M >= 1 && M <= FP_MAX_M && p->has_override[M]) {
    const fp_tiling& o = p->override_t[M];
    t->path = o.path;
    t->kparts = o.kparts;
    t->chunks = o.chunks;
    t->splits = o.splits;
    t->rows = o.rows;
    t->groups = o.groups;
    if (t->path == FP_PATH_SKINNY || t->path == FP_PATH_SKINNY_SPLITK) {
      t->path = t->splits > 1 ? FP_PATH_SKINNY_SPLITK : FP_PATH_SKINNY;
    }
  } else {
    // fp32-output plans run the vector-ALU kernel only
    const bool mfma = p->dtype == FP_BF16 && !p->out_f32 &&
                      (M >= p->mfma_min_m || M > kSmallMfmaMaxM);
    // bf16 and block-scaled weights: the small-M kernel up to 16 tokens,
    // when its workgroup of K parts fits the kernel's thread bound (long K
    // with two token halves does not: up to 8 tokens the vector-ALU kernel
    // serves, above that bf16 takes the matrix-core path).  A bf16 plan
    // whose two-half launches cannot keep every workgroup resident at once
    // (more rows than one workgroup per CU holds) takes the matrix-core
    // path too: measured on MI355X at K = 6144, 2752 rows, M = 9 / 16: ring
    // tile kernel 12.28 / 12.64 us against the small-M kernel's two rounds,
    // 13.87 / 14.01.
    bool small = (p->dtype == FP_BF16 || is_mx(p->dtype)) &&
                 !p->out_f32 && !mfma &&
                 (M >= p->small_mfma_min_m || M > kSkinnyMaxM) &&
                 default_smfma_order(p->kc, t);
    if (small) {
      bool one_round = false;
      auto probe_fits = [&]() {
        Tiling probe = *t;
        probe.mt = smfma_mt(M);
        one_round = resolve_smfma_rows(p->n_total, &probe, pairs, p->dtype == FP_BF16);
        return (int64_t)probe.groups * probe.kparts * 64 <=
               fp::smfma_max_threads(probe.chunks, probe.mt / 8, smfma_tiles(probe));
      };
      bool fits = probe_fits();
      // Block-scaled weights have no tile kernel to fall back on: where two
      // token halves at eight K steps per wave need more waves than the
      // thread bound allows (K = 6656..8192: 13..16 parts against 12), the
      // sixteen-step form (no scratch, 163..192 VGPRs) halves the waves.
      if (!fits && is_mx(p->dtype) && t->chunks < 16) {
        const int64_t pk16 = ceil_div(ceil_div(p->kc, 8), 16);
        if (pk16 <= fp::kMaxWaveParts) {
          t->chunks = 16;
          t->kparts = (int)pk16;
          fits = probe_fits();
        }
      }
      if (!fits)
        small = false;
      else if (!one_round && !pairs && p->dtype == FP_BF16 && M > 8 &&
               ring_addressable(p->n_total, p->kc))
        small = false;
    }
    const bool to_mfma = mfma || (!small && p->dtype == FP_BF16 && !p->out_f32 &&
                                  M > kSkinnyMaxM);
    if (to_mfma) {
      if (!default_mfma_order(p->kc, M, p->n_total, t)) return false;
    } else if (small) {
      // order fields already set
    } else {
      if (M > skinny_max_m(p)) return false;
      default_skinny_order(p->dtype, p->kc, p->n_total, skinny_mt(M), t);
    }
  }
  if (p->out_f32 && t->path != FP_PATH_SKINNY && t->path != FP_PATH_SKINNY_SPLITK) return false;
  if (is_mx(p->dtype) && t->path != FP_PATH_SKINNY && t->path != FP_PATH_SKINNY_SPLITK &&
      t->path != FP_PATH_MFMA_SMALL)
    return false;
  if (t->path == FP_PATH_MFMA) {
    t->mt = mfma_mt16(M);
    if (t->splits < 1) return false;
    resolve_tile_launch(p, n_rows, t);
  } else if (t->path == FP_PATH_MFMA_SMALL) {
    t->mt = smfma_mt(M);
    if (t->kparts < 1 || t->chunks < 1) return false;
    resolve_smfma_rows(n_rows, t, pairs, p->dtype == FP_BF16);
  } else {
    t->mt = skinny_mt(M);
    if (t->kparts < 1) return false;
    resolve_skinny_rows(p, n_rows, t->mt, t, pairs);
  }
  // a gate/up launch keeps both rows of a pair in one row group (and one
  // tile per wave)
  if (pairs && (t->rows % 2 != 0 || t->splits != 1)) return false;
  if (pairs && t->path == FP_PATH_MFMA_SMALL && smfma_tiles(*t) != 1) return false;
  return tiling_valid(p, M, n_rows, *t, ws != nullptr ? *ws : plan_ws(p), pairs);
}

// A host-only stand-in plan with default settings and unlimited workspace,
// for questions about default tilings.
void standin_plan(fp_plan_s* tmp, int32_t dtype, int64_t K, int64_t n_total,
                  int64_t max_M) {
  std::memset(tmp, 0, sizeof *tmp);
  tmp->magic = kPlanMagic;
  tmp->dtype = dtype;
  int es = 2;
  int64_t wrow = 0, kc = 0;
  dtype_geometry(dtype, K, &es, &wrow, &kc);
  tmp->esize = es;
  tmp->osize = es;
  tmp->wrow = wrow;
  tmp->K = K;
  tmp->kc = kc;
  tmp->n_proj = 1;
  tmp->N[0] = n_total;
  tmp->n_total = n_total;
  tmp->max_M = max_M;
  tmp->mfma_min_m = kDefaultMfmaMinM;
  tmp->small_mfma_min_m = default_small_mfma_min_m(dtype, K, n_total);
  tmp->ws_bytes = SIZE_MAX;
}

size_t workspace_need(int32_t dtype, int64_t K, int64_t n_total, int64_t max_M) {
  // counters for every possible row block, plus the largest partial buffer
  // over the default tilings of every M up to max_M (fused launch: all rows)
  fp_plan_s tmp;
  standin_plan(&tmp, dtype, K, n_total, max_M);
  int64_t most = 0;
  for (int64_t M = 1; M <= max_M; ++M) {
    Tiling t;
    if (!choose_tiling(&tmp, M, n_total, &t)) continue;
    most = std::max(most, partial_floats(t, n_total, M));
  }
  // the MFMA path at every M (a later fp_plan_set_mfma_min_m can move the
  // crossover down) and the fp32-output defaults (a later
  // fp_plan_set_out_dtype) for bf16
  if (dtype == FP_BF16) {
    for (int64_t M = 1; M <= max_M; ++M) {
      Tiling t;
      if (!default_mfma_order(tmp.kc, M, n_total, &t)) continue;
      most = std::max(most, partial_floats(t, n_total, M));
    }
    tmp.out_f32 = true;
    tmp.osize = 4;
    for (int64_t M = 1; M <= max_M; ++M) {
      Tiling t;
      if (!choose_tiling(&tmp, M, n_total, &t)) continue;
      most = std::max(most, partial_floats(t, n_total, M));
    }
  }
  return (size_t)(counters_bytes(n_total) + most * 4);
}

// ------------------------------------------------------------------ kernels
// Kernel addresses come from the per-family units (kernels.h).
const void* mfma_fn(const Tiling& t) {
  return is_wres(t)   ? fpk::wres(t.mt)
         : is_ring(t) ? fpk::ring(t.mt, t.chunks)
                      : fpk::tile(t.mt, t.kparts, t.chunks);
}

const void* smfma_fn(const Tiling& t, bool pairs, int32_t dtype, int64_t M) {
  if (is_mx(dtype)) return pairs ? nullptr : fpk::smfma_mx(dtype, t.mt / 8, t.chunks);
  return fpk::smfma(t.chunks, pairs, t.mt, M, smfma_tiles(t));
}

std::mutex g_attr_mu;
std::unordered_set<const void*>& big_lds_kernels() {
  static std::unordered_set<const void*> s;
  return s;
}

fp_status hip_fail(hipError_t e) {
  g_last_hip = (int32_t)e;
  return FP_ERR_HIP;
}

fp_status launch(const void* fn, int64_t blocks, int threads, size_t lds,
                 void** args, hipStream_t stream) {
  if (fn == nullptr || blocks <= 0) return FP_ERR_UNSUPPORTED;
  if (lds > 64 * 1024) {
    std::lock_guard<std::mutex> lk(g_attr_mu);
    if (big_lds_kernels().count(fn) == 0) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return hip_fail(e);
      big_lds_kernels().insert(fn);
    }
  }
  // The launch's own return code is checked; hipGetLastError is not used
  // because it would also report (and clear) errors left by other code.
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3((unsigned)threads),
                                 args, lds, stream);
  if (e != hipSuccess) return hip_fail(e);
  return FP_OK;
}

// The rows one launch computes: rows [0, n_rows) of the weight buffer w
// (row r at w + r * K * esize), split into n_seg output segments; segment i
// owns rows [begin[i], begin[i+1]) and writes the dense [M, N_i] tensor y[i].
struct LaunchRows {
  const unsigned char* w;
  int n_rows;
  int n_seg;
  unsigned char* y[fp::kMaxSeg];
  int begin[fp::kMaxSeg + 1];
  float scale[fp::kMaxSeg];  // segment tensor scales (NVFP4)
};

// One launch over `lr` with tiling t.  Every kernel takes the same 14
// leading argument dwords, all preloaded into SGPRs at wave launch (the
// hardware limit; a 15th would be read from memory before the first load):
// w, x, y0, y1, ldx in bytes, n_rows, kc, M, split and one kernel-specific
// geometry word; then the trailing Tail (output table for more than two
// segments, split-K workspace).
fp_status run(const fp_plan_s* p, const Tiling& t, const LaunchRows& lr,
              const void* x, int64_t M, int64_t ldx, hipStream_t stream,
              bool pairs = false, const WsView* ws = nullptr) {
  const unsigned char* w_a = lr.w;
  const unsigned char* x_a = static_cast<const unsigned char*>(x);
  unsigned char* y0_a = lr.y[0];
  unsigned char* y1_a = lr.n_seg >= 2 ? lr.y[1] : lr.y[0];
  uint32_t ldx_a = (uint32_t)(ldx * p->esize);
  int32_t n_rows_a = lr.n_rows;
  int32_t kc_a = (int32_t)p->kc;
  int32_t M_a = (int32_t)M;
  int32_t split_a = lr.n_seg > 2 ? -1 : (lr.n_seg == 2 ? lr.begin[1] : lr.n_rows);
  fp::Tail tail;
  std::memset(&tail, 0, sizeof tail);
  tail.out.n_seg = lr.n_seg;
  for (int i = 0; i < fp::kMaxSeg; ++i) {
    tail.out.y[i] = i < lr.n_seg ? lr.y[i] : nullptr;
    tail.out.begin[i] = i < lr.n_seg ? lr.begin[i] : lr.n_rows;
    tail.out.tscale[i] = i < lr.n_seg ? lr.scale[i] : 1.0f;
  }
  tail.out.begin[fp::kMaxSeg] = lr.n_rows;
  const WsView wsv = ws != nullptr ? *ws : plan_ws(p);
  tail.partial = reinterpret_cast<float*>(wsv.partial);
  tail.counters = reinterpret_cast<uint32_t*>(wsv.counters);
  int32_t geo_a = 0;
  void* args[] = {&w_a, &x_a, &y0_a, &y1_a, &ldx_a, &n_rows_a, &kc_a, &M_a, &split_a,
                  &geo_a, &tail};
  if (t.path == FP_PATH_MFMA_SMALL) {
    geo_a = smfma_rt(t) | (t.kparts << 8) | (t.groups << 16);
    const int64_t R = (int64_t)t.rows * t.groups;
    return launch(smfma_fn(t, pairs, p->dtype, M_a), ceil_div(lr.n_rows, R),
                  t.groups * t.kparts * 64, smfma_lds(t), args, stream);
  }
  if (pairs && t.path != FP_PATH_SKINNY) return FP_ERR_UNSUPPORTED;
  if (t.path == FP_PATH_MFMA) {
    // the tile kernels address x with 32-bit buffer offsets
    if ((M - 1) * (int64_t)ldx_a + p->kc * 16 >= ((int64_t)1 << 31)) return FP_ERR_UNSUPPORTED;
    const bool second = t.splits > 1 && t.groups == 2;
    geo_a = t.splits | (second ? fp::kGeoSecondFinish : 0);
    const int64_t per = ceil_div(ceil_div(p->kc, 4), t.splits);
    const int64_t blocks = ceil_div(lr.n_rows, 16 * (int64_t)t.kparts) * t.splits;
    const size_t lds = is_wres(t)   ? (size_t)fp::wres_lds_bytes(16 * t.mt)
                       : is_ring(t) ? ring_lds(t.mt, t.chunks)
                                  : std::max<size_t>(tile_lds(t.mt, per, t.kparts), 16);
    const int threads = is_wres(t) ? fp::wres_threads(16 * t.mt) : t.kparts * 64;
    fp_status st = launch(mfma_fn(t), blocks, threads, lds, args, stream);
    if (st != FP_OK || !second) return st;
    // the slices, added in slice order over the whole GPU
    const float* part_a = tail.partial;
    int32_t s_a = t.splits;
    void* rargs[] = {&part_a, &n_rows_a, &M_a, &s_a, &tail.out};
    return launch(fpk::splitk_reduce(), ceil_div(M * ceil_div(lr.n_rows, 4), fp::kReduceThreads),
                  fp::kReduceThreads, 0, rargs, stream);
  }
  geo_a = t.kparts | (t.groups << 8) | (t.splits << 16);
  const int64_t R = (int64_t)t.groups * t.rows;
  const int64_t blocks = ceil_div(lr.n_rows, R) * t.splits;
  return launch(skinny_fn(p, t, pairs), blocks, t.groups * t.kparts * 64, skinny_lds(t), args,
                stream);
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

// Checks shared by fp_supported and the forward calls (host only).
fp_status check_x(const fp_plan_s* p, int64_t M, const void* x, int64_t ldx) {
  if (M < 0) return FP_ERR_INVALID_ARG;
  if (M == 0) return FP_OK;
  if (x == nullptr || ldx < p->K) return FP_ERR_INVALID_ARG;
  if (M > p->max_M) return FP_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || (ldx * p->esize) % 16 != 0) return FP_ERR_UNSUPPORTED;
  if (ldx * p->esize > INT32_MAX) return FP_ERR_UNSUPPORTED;  // 32-bit row stride
  if (p->dtype == FP_F32 && M > kSkinnyMaxM) return FP_ERR_UNSUPPORTED;
  if (p->out_f32 && M > skinny_max_m(p)) return FP_ERR_UNSUPPORTED;
  // the kernels index an output element m * N_i + r with 32-bit integers
  for (int i = 0; i < p->n_proj; ++i)
    if (M * p->N[i] > INT32_MAX) return FP_ERR_UNSUPPORTED;
  return FP_OK;
}

fp_status check_outputs(const fp_plan_s* p, int64_t M, const void* x, int64_t ldx,
                        void* const* y) {
  if (y == nullptr) return FP_ERR_INVALID_ARG;
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x);
  const uintptr_t xe = xb + (uintptr_t)(((M - 1) * ldx + p->K) * p->esize);
  const uintptr_t wb = reinterpret_cast<uintptr_t>(p->w_cat);
  const uintptr_t we = wb + (uintptr_t)(p->n_total * p->wrow);
  const uintptr_t sb = reinterpret_cast<uintptr_t>(p->ws);
  const uintptr_t se = sb + p->ws_bytes;
  for (int i = 0; i < p->n_proj; ++i) {
    if (y[i] == nullptr || !aligned(y[i], (uintptr_t)p->osize)) return FP_ERR_INVALID_ARG;
    const uintptr_t b = reinterpret_cast<uintptr_t>(y[i]);
    const uintptr_t e = b + (uintptr_t)(M * p->N[i] * p->osize);
    if (overlaps(b, e, xb, xe) || overlaps(b, e, wb, we) || overlaps(b, e, sb, se))
      return FP_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j) {
      const uintptr_t b2 = reinterpret_cast<uintptr_t>(y[j]);
      const uintptr_t e2 = b2 + (uintptr_t)(M * p->N[j] * p->osize);
      if (overlaps(b, e, b2, e2)) return FP_ERR_INVALID_ARG;
    }
  }
  return FP_OK;
}

}  // namespace

extern "C" {

size_t fp_workspace_bytes(int32_t dtype, int64_t K, int32_t n_proj, const int64_t* N,
                          int64_t max_M) {
  if (!dtype_known(dtype) || K < 1 || n_proj < 1 ||
      n_proj > FP_MAX_PROJ || N == nullptr || max_M < 1 || max_M > FP_MAX_M)
    return 0;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(dtype, K, &esize, &wrow, &kc)) return 0;
  int64_t n_total = 0;
  for (int i = 0; i < n_proj; ++i) {
    if (N[i] < 1) return 0;
    n_total += N[i];
  }
  return workspace_need(dtype, K, n_total, max_M);
}

fp_status fp_plan_create(int32_t dtype, int64_t K, int32_t n_proj, const int64_t* N,
                         const void* const* w_src, void* w_cat, void* workspace,
                         size_t ws_bytes, int64_t max_M, void* stream, fp_plan_t* out) {
  if (out == nullptr) return FP_ERR_INVALID_ARG;
  *out = nullptr;
  if (!dtype_known(dtype)) return FP_ERR_INVALID_ARG;
  if (K < 1 || n_proj < 1 || n_proj > FP_MAX_PROJ || N == nullptr) return FP_ERR_INVALID_ARG;
  if (max_M < 1 || max_M > FP_MAX_M) return FP_ERR_INVALID_ARG;
  if (w_cat == nullptr || workspace == nullptr) return FP_ERR_INVALID_ARG;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(dtype, K, &esize, &wrow, &kc)) return FP_ERR_UNSUPPORTED;
  if (!aligned(w_cat, 256) || !aligned(workspace, 256)) return FP_ERR_UNSUPPORTED;
  int64_t n_total = 0;
  for (int i = 0; i < n_proj; ++i) {
    if (N[i] < 1) return FP_ERR_INVALID_ARG;
    n_total += N[i];
  }
  // the kernels index rows and 16-byte chunks with 32-bit integers
  if (n_total > kMaxRows || kc > kMaxRows || wrow > INT32_MAX) return FP_ERR_UNSUPPORTED;
  if (ws_bytes < workspace_need(dtype, K, n_total, max_M)) return FP_ERR_WORKSPACE;

  fp_plan_s* p = new (std::nothrow) fp_plan_s;
  if (p == nullptr) return FP_ERR_INVALID_ARG;
  std::memset(p, 0, sizeof *p);
  p->magic = kPlanMagic;
  p->dtype = dtype;
  p->esize = esize;
  p->osize = esize;
  p->K = K;
  p->kc = kc;
  p->wrow = wrow;
  p->n_proj = n_proj;
  int64_t off = 0;
  for (int i = 0; i < n_proj; ++i) {
    p->N[i] = N[i];
    p->off[i] = off;
    off += N[i];
  }
  p->n_total = n_total;
  p->w_cat = static_cast<unsigned char*>(w_cat);
  p->ws = static_cast<unsigned char*>(workspace);
  p->ws_bytes = ws_bytes;
  p->max_M = max_M;
  p->mfma_min_m = kDefaultMfmaMinM;
  for (int i = 0; i < FP_MAX_PROJ; ++i) p->tscale[i] = 1.0f;
  p->small_mfma_min_m = default_small_mfma_min_m(dtype, K, n_total);

  hipStream_t st = static_cast<hipStream_t>(stream);
  // concatenate: W_cat[off_i + r, :] = W_i[r, :]
  for (int i = 0; i < n_proj && w_src != nullptr; ++i) {
    unsigned char* dst = p->w_cat + p->off[i] * wrow;
    if (w_src[i] == nullptr || w_src[i] == dst) continue;
    hipError_t e = hipMemcpyAsync(dst, w_src[i], (size_t)(N[i] * wrow),
                                  hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e);
    }
  }
  // zero the arrival counters with a kernel (capture-friendly, no memset node)
  int64_t nc = counters_bytes(n_total) / 4;
  uint32_t* cptr = reinterpret_cast<uint32_t*>(p->ws);
  uint32_t zero = 0u;
  void* fargs[] = {&cptr, &nc, &zero};
  hipError_t e = hipLaunchKernel(fpk::fill_u32(),
                                 dim3((unsigned)ceil_div(nc, 256)), dim3(256), fargs, 0, st);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e);
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    live_plans().insert(p);
  }
  *out = p;
  return FP_OK;
}

fp_status fp_plan_view(fp_plan_t plan, int32_t i, void** w_i, int64_t* row_offset,
                       int64_t* rows) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (i < 0 || i >= plan->n_proj) return FP_ERR_INVALID_ARG;
  if (w_i) *w_i = plan->w_cat + plan->off[i] * plan->wrow;
  if (row_offset) *row_offset = plan->off[i];
  if (rows) *rows = plan->N[i];
  return FP_OK;
}

fp_status fp_plan_destroy(fp_plan_t plan) {
  if (plan == nullptr) return FP_ERR_INVALID_ARG;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (live_plans().erase(plan) == 0) return FP_ERR_INVALID_ARG;
  }
  plan->magic = 0;
  delete plan;
  return FP_OK;
}

fp_status fp_supported(fp_plan_t plan, int64_t M, const void* x, int64_t ldx) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK || M == 0) return s;
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t)) return FP_ERR_UNSUPPORTED;
  return FP_OK;
}

fp_status fp_forward(const void* x, int64_t M, int64_t ldx, fp_plan_t plan, void* stream,
                     void* const* y) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK) return s;
  if (M == 0) return FP_OK;
  s = check_outputs(plan, M, x, ldx, y);
  if (s != FP_OK) return s;
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t)) return FP_ERR_UNSUPPORTED;
  LaunchRows lr;
  std::memset(&lr, 0, sizeof lr);
  lr.w = plan->w_cat;
  lr.n_seg = plan->n_proj;
  lr.n_rows = (int)plan->n_total;
  for (int i = 0; i < plan->n_proj; ++i) {
    lr.y[i] = static_cast<unsigned char*>(y[i]);
    lr.begin[i] = (int)plan->off[i];
    lr.scale[i] = plan->tscale[i];
  }
  lr.begin[plan->n_proj] = (int)plan->n_total;
  return run(plan, t, lr, x, M, ldx, static_cast<hipStream_t>(stream));
}

fp_status fp_forward_separate(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                              void* stream, void* const* y,
                              const void* const* w_override) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK) return s;
  if (M == 0) return FP_OK;
  s = check_outputs(plan, M, x, ldx, y);
  if (s != FP_OK) return s;
  Tiling ts[FP_MAX_PROJ];
  for (int i = 0; i < plan->n_proj; ++i) {
    if (!choose_tiling(plan, M, plan->N[i], &ts[i])) return FP_ERR_UNSUPPORTED;
    if (w_override != nullptr && w_override[i] != nullptr &&
        !aligned(w_override[i], 16))
      return FP_ERR_UNSUPPORTED;
  }
  for (int i = 0; i < plan->n_proj; ++i) {
    LaunchRows lr;
    std::memset(&lr, 0, sizeof lr);
    lr.n_seg = 1;
    lr.n_rows = (int)plan->N[i];
    const unsigned char* w = plan->w_cat + plan->off[i] * plan->wrow;
    if (w_override != nullptr && w_override[i] != nullptr)
      w = static_cast<const unsigned char*>(w_override[i]);
    lr.w = w;
    lr.y[0] = static_cast<unsigned char*>(y[i]);
    lr.begin[0] = 0;
    lr.begin[1] = (int)plan->N[i];
    lr.scale[0] = plan->tscale[i];
    s = run(plan, ts[i], lr, x, M, ldx, static_cast<hipStream_t>(stream));
    if (s != FP_OK) return s;
  }
  return FP_OK;
}

}  // extern "C"

namespace {

bool range_overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return overlaps(a0, a0 + (uintptr_t)a_bytes, b0, b0 + (uintptr_t)b_bytes);
}

// The fused launch over every projection of a plan, output i to y[i].
LaunchRows fused_rows(const fp_plan_s* p, void* const* y) {
  LaunchRows lr;
  std::memset(&lr, 0, sizeof lr);
  lr.w = p->w_cat;
  lr.n_seg = p->n_proj;
  lr.n_rows = (int)p->n_total;
  for (int i = 0; i < p->n_proj; ++i) {
    lr.begin[i] = (int)p->off[i];
    lr.y[i] = static_cast<unsigned char*>(y[i]);
    lr.scale[i] = p->tscale[i];
  }
  lr.begin[p->n_proj] = (int)p->n_total;
  return lr;
}

// One RMSNorm launch over `n` tensors (host validated), M rows each.
fp_status launch_rmsnorm(int n, const unsigned char* const* y, const unsigned char* const* gamma,
                         unsigned char* const* out, const int64_t* N, int64_t M, float eps,
                         hipStream_t stream) {
  fp::NormTable t;
  std::memset(&t, 0, sizeof t);
  for (int i = 0; i < n; ++i) {
    t.y[i] = y[i];
    t.gamma[i] = gamma[i];
    t.out[i] = out[i];
    t.N[i] = (int32_t)N[i];
  }
  t.M = (int32_t)M;
  t.eps = eps;
  void* args[] = {&t};
  return launch(fpk::rmsnorm(), (int64_t)n * M, 64, 0, args,
                stream);
}

}  // namespace

extern "C" {

fp_status fp_forward_rmsnorm(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                             void* stream, const void* const* gamma, float eps,
                             void* const* out) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (gamma == nullptr || out == nullptr) return FP_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !(eps < INFINITY)) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK) return s;
  if (M == 0) return FP_OK;
  // bf16 outputs: bf16 and MXFP8 plans
  if ((plan->dtype != FP_BF16 && !is_mx(plan->dtype)) || plan->out_f32)
    return FP_ERR_UNSUPPORTED;
  s = check_outputs(plan, M, x, ldx, out);
  if (s != FP_OK) return s;
  int n = 0;
  const unsigned char* ny[FP_MAX_PROJ];
  const unsigned char* ng[FP_MAX_PROJ];
  unsigned char* no[FP_MAX_PROJ];
  int64_t nn[FP_MAX_PROJ];
  for (int i = 0; i < plan->n_proj; ++i) {
    if (gamma[i] == nullptr) continue;
    const int64_t N = plan->N[i];
    if (N % 8 != 0 || N > fp::kNormMaxN) return FP_ERR_UNSUPPORTED;
    if (!aligned(out[i], 16) || !aligned(gamma[i], 16)) return FP_ERR_UNSUPPORTED;
    for (int j = 0; j < plan->n_proj; ++j)
      if (range_overlaps(gamma[i], N * 2, out[j], M * plan->N[j] * 2)) return FP_ERR_INVALID_ARG;
    ny[n] = static_cast<const unsigned char*>(out[i]);
    ng[n] = static_cast<const unsigned char*>(gamma[i]);
    no[n] = static_cast<unsigned char*>(out[i]);
    nn[n] = N;
    ++n;
  }
  if ((int64_t)n * M > INT32_MAX) return FP_ERR_UNSUPPORTED;
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t)) return FP_ERR_UNSUPPORTED;
  // the projection writes every output; the normalisation then works in place
  s = run(plan, t, fused_rows(plan, out), x, M, ldx, static_cast<hipStream_t>(stream));
  if (s != FP_OK || n == 0) return s;
  return launch_rmsnorm(n, ny, ng, no, nn, M, eps, static_cast<hipStream_t>(stream));
}

fp_status fp_forward_swiglu(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                            void* stream, void* h) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (plan->n_proj != 2 || plan->N[0] != plan->N[1]) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK) return s;
  if (M == 0) return FP_OK;
  if (h == nullptr) return FP_ERR_INVALID_ARG;
  const int64_t N = plan->N[0];
  if (plan->dtype != FP_BF16 || plan->out_f32 || M > kSkinnyMaxM || N % 8 != 0)
    return FP_ERR_UNSUPPORTED;
  if (!aligned(h, 16)) return FP_ERR_UNSUPPORTED;
  const int64_t hb = M * N * 2;
  if (range_overlaps(h, hb, x, ((M - 1) * ldx + plan->K) * 2) ||
      range_overlaps(h, hb, plan->w_cat, plan->n_total * plan->wrow) ||
      range_overlaps(h, hb, plan->ws, (int64_t)plan->ws_bytes))
    return FP_ERR_INVALID_ARG;
  // one launch over the 2N rows taken in (gate j, up j) pairs
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t, true)) return FP_ERR_UNSUPPORTED;
  if (!(t.path == FP_PATH_SKINNY || t.path == FP_PATH_MFMA_SMALL)) return FP_ERR_UNSUPPORTED;
  void* hh[2] = {h, h};
  return run(plan, t, fused_rows(plan, hh), x, M, ldx, static_cast<hipStream_t>(stream), true);
}

fp_status fp_rmsnorm(const void* y, int64_t M, int64_t N, const void* gamma, float eps,
                     void* out, void* stream) {
  if (M < 0 || N < 1 || !(eps >= 0.0f) || !(eps < INFINITY)) return FP_ERR_INVALID_ARG;
  if (M == 0) return FP_OK;
  if (y == nullptr || gamma == nullptr || out == nullptr) return FP_ERR_INVALID_ARG;
  if (N % 8 != 0 || N > fp::kNormMaxN || M > INT32_MAX) return FP_ERR_UNSUPPORTED;
  if (!aligned(y, 16) || !aligned(gamma, 16) || !aligned(out, 16)) return FP_ERR_UNSUPPORTED;
  // in place (out == y) is allowed; any other overlap is not
  if (out != y && range_overlaps(out, M * N * 2, y, M * N * 2)) return FP_ERR_INVALID_ARG;
  if (range_overlaps(out, M * N * 2, gamma, N * 2)) return FP_ERR_INVALID_ARG;
  const unsigned char* y_a = static_cast<const unsigned char*>(y);
  const unsigned char* g_a = static_cast<const unsigned char*>(gamma);
  unsigned char* o_a = static_cast<unsigned char*>(out);
  return launch_rmsnorm(1, &y_a, &g_a, &o_a, &N, M, eps, static_cast<hipStream_t>(stream));
}

fp_status fp_swiglu(const void* g, const void* u, int64_t M, int64_t N, void* h,
                    void* stream) {
  if (M < 0 || N < 1) return FP_ERR_INVALID_ARG;
  if (M == 0) return FP_OK;
  if (g == nullptr || u == nullptr || h == nullptr) return FP_ERR_INVALID_ARG;
  if (N % 8 != 0) return FP_ERR_UNSUPPORTED;
  const int64_t chunks = M * N / 8;
  if (chunks > INT32_MAX - 256) return FP_ERR_UNSUPPORTED;
  if (!aligned(g, 16) || !aligned(u, 16) || !aligned(h, 16)) return FP_ERR_UNSUPPORTED;
  const int64_t b = M * N * 2;
  // h may replace g or u element for element; any other overlap is not allowed
  if ((h != g && range_overlaps(h, b, g, b)) || (h != u && range_overlaps(h, b, u, b)))
    return FP_ERR_INVALID_ARG;
  const unsigned char* g_a = static_cast<const unsigned char*>(g);
  const unsigned char* u_a = static_cast<const unsigned char*>(u);
  unsigned char* h_a = static_cast<unsigned char*>(h);
  int32_t n_a = (int32_t)chunks;
  void* args[] = {&g_a, &u_a, &h_a, &n_a};
  return launch(fpk::swiglu(), ceil_div(chunks, 256), 256,
                0, args, static_cast<hipStream_t>(stream));
}

fp_status fp_mxfp8_to_bf16(const void* w, int64_t rows, int64_t K, void* out, void* stream) {
  if (rows < 0 || K < 1) return FP_ERR_INVALID_ARG;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(FP_MXFP8, K, &esize, &wrow, &kc)) return FP_ERR_UNSUPPORTED;
  if (rows == 0) return FP_OK;
  if (w == nullptr || out == nullptr) return FP_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(out, 16)) return FP_ERR_UNSUPPORTED;
  if (range_overlaps(w, rows * wrow, out, rows * K * 2)) return FP_ERR_INVALID_ARG;
  const unsigned char* w_a = static_cast<const unsigned char*>(w);
  unsigned char* o_a = static_cast<unsigned char*>(out);
  int32_t kc_a = (int32_t)(K / 16);  // 16-code chunks
  int64_t n_a = rows * kc_a;
  void* args[] = {&w_a, &o_a, &kc_a, &n_a};
  return launch(fpk::mxfp8_to_bf16(), ceil_div(n_a, 256), 256,
                0, args, static_cast<hipStream_t>(stream));
}

fp_status fp_stream_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  if (bytes < 0) return FP_ERR_INVALID_ARG;
  if (bytes == 0) return FP_OK;
  if (buf == nullptr || sink == nullptr) return FP_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4) || bytes % 16 != 0) return FP_ERR_UNSUPPORTED;
  if (bytes >= ((int64_t)1 << 31)) return FP_ERR_UNSUPPORTED;
  if (range_overlaps(buf, bytes, sink, 4 * fp::kStreamGroups)) return FP_ERR_INVALID_ARG;
  const unsigned char* b_a = static_cast<const unsigned char*>(buf);
  uint32_t bytes_a = (uint32_t)bytes;
  uint32_t per_a = (uint32_t)ceil_div(bytes / 16, fp::kStreamGroups);
  uint32_t* s_a = static_cast<uint32_t*>(sink);
  void* args[] = {&b_a, &bytes_a, &per_a, &s_a};
  return launch(fpk::stream_read(), fp::kStreamGroups,
                fp::kStreamThreads, 0, args, static_cast<hipStream_t>(stream));
}

fp_status fp_stream_read_shaped(const void* buf, int64_t bytes, int32_t groups, int32_t threads,
                                int32_t batch, void* sink, void* stream) {
  if (bytes < 0 || groups < 1 || threads < 64) return FP_ERR_INVALID_ARG;
  if (bytes == 0) return FP_OK;
  if (buf == nullptr || sink == nullptr) return FP_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4) || bytes % 16 != 0) return FP_ERR_UNSUPPORTED;
  if (bytes >= ((int64_t)1 << 31) || groups > 65536 || threads % 64 != 0) return FP_ERR_UNSUPPORTED;
  if (!(batch == 8 || batch == 16 || batch == 32)) return FP_ERR_UNSUPPORTED;
  if (threads > fp::stream_shaped_max_threads(batch)) return FP_ERR_UNSUPPORTED;
  if (range_overlaps(buf, bytes, sink, 4 * (int64_t)groups)) return FP_ERR_INVALID_ARG;
  const unsigned char* b_a = static_cast<const unsigned char*>(buf);
  uint32_t bytes_a = (uint32_t)bytes;
  uint32_t per_a = (uint32_t)ceil_div(bytes / 16, groups);
  uint32_t* s_a = static_cast<uint32_t*>(sink);
  void* args[] = {&b_a, &bytes_a, &per_a, &s_a};
  return launch(fpk::stream_read_shaped(batch), groups, threads, 0, args,
                static_cast<hipStream_t>(stream));
}

fp_status fp_mxfp4_to_bf16(const void* w, int64_t rows, int64_t K, void* out, void* stream) {
  if (rows < 0 || K < 1) return FP_ERR_INVALID_ARG;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(FP_MXFP4, K, &esize, &wrow, &kc)) return FP_ERR_UNSUPPORTED;
  if (rows == 0) return FP_OK;
  if (w == nullptr || out == nullptr) return FP_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(out, 16)) return FP_ERR_UNSUPPORTED;
  if (range_overlaps(w, rows * wrow, out, rows * K * 2)) return FP_ERR_INVALID_ARG;
  const unsigned char* w_a = static_cast<const unsigned char*>(w);
  unsigned char* o_a = static_cast<unsigned char*>(out);
  int32_t kc_a = (int32_t)(K / 32);  // 16-byte chunks of 32 codes: one per block
  int64_t n_a = rows * kc_a;
  void* args[] = {&w_a, &o_a, &kc_a, &n_a};
  return launch(fpk::mxfp4_to_bf16(), ceil_div(n_a, 256), 256,
                0, args, static_cast<hipStream_t>(stream));
}

fp_status fp_nvfp4_to_bf16(const void* w, int64_t rows, int64_t K, float g, void* out,
                           void* stream) {
  if (rows < 0 || K < 1 || !std::isfinite(g)) return FP_ERR_INVALID_ARG;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(FP_NVFP4, K, &esize, &wrow, &kc)) return FP_ERR_UNSUPPORTED;
  if (rows == 0) return FP_OK;
  if (w == nullptr || out == nullptr) return FP_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(out, 16)) return FP_ERR_UNSUPPORTED;
  if (range_overlaps(w, rows * wrow, out, rows * K * 2)) return FP_ERR_INVALID_ARG;
  const unsigned char* w_a = static_cast<const unsigned char*>(w);
  unsigned char* o_a = static_cast<unsigned char*>(out);
  int32_t kc_a = (int32_t)(K / 32);  // 16-byte chunks of 32 codes: two blocks each
  int64_t n_a = rows * kc_a;
  float g_a = g;
  void* args[] = {&w_a, &o_a, &kc_a, &n_a, &g_a};
  return launch(fpk::nvfp4_to_bf16(), ceil_div(n_a, 256), 256,
                0, args, static_cast<hipStream_t>(stream));
}

fp_status fp_plan_set_tensor_scales(fp_plan_t plan, const float* scales) {
  if (!plan_ok(plan) || scales == nullptr) return FP_ERR_INVALID_ARG;
  if (plan->dtype != FP_NVFP4) return FP_ERR_UNSUPPORTED;
  for (int i = 0; i < plan->n_proj; ++i)
    if (!std::isfinite(scales[i])) return FP_ERR_INVALID_ARG;
  for (int i = 0; i < plan->n_proj; ++i) plan->tscale[i] = scales[i];
  return FP_OK;
}

fp_status fp_plan_query(fp_plan_t plan, int64_t M, int32_t* path, int32_t* launches_fused,
                        int32_t* launches_separate) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (M < 0) return FP_ERR_INVALID_ARG;
  if (M == 0) {
    if (path) *path = FP_PATH_NONE;
    if (launches_fused) *launches_fused = 0;
    if (launches_separate) *launches_separate = 0;
    return FP_OK;
  }
  if (M > plan->max_M || (plan->dtype == FP_F32 && M > kSkinnyMaxM) ||
      (plan->out_f32 && M > skinny_max_m(plan)))
    return FP_ERR_UNSUPPORTED;
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t)) return FP_ERR_UNSUPPORTED;
  // a split tile launch finished in a second launch counts two
  auto count = [](const Tiling& u) {
    return u.path == FP_PATH_MFMA && u.splits > 1 && u.groups == 2 ? 2 : 1;
  };
  int32_t n_sep = 0;
  for (int i = 0; i < plan->n_proj; ++i) {
    Tiling ti;
    if (!choose_tiling(plan, M, plan->N[i], &ti)) return FP_ERR_UNSUPPORTED;
    n_sep += count(ti);
  }
  if (path) *path = t.path;
  if (launches_fused) *launches_fused = count(t);
  if (launches_separate) *launches_separate = n_sep;
  return FP_OK;
}

fp_status fp_plan_set_out_dtype(fp_plan_t plan, int32_t out_dtype) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (out_dtype != FP_BF16 && out_dtype != FP_F32) return FP_ERR_INVALID_ARG;
  if (plan->dtype == FP_F32) return out_dtype == FP_F32 ? FP_OK : FP_ERR_UNSUPPORTED;
  if (is_mx(plan->dtype)) return out_dtype == FP_BF16 ? FP_OK : FP_ERR_UNSUPPORTED;
  plan->out_f32 = out_dtype == FP_F32;
  plan->osize = plan->out_f32 ? 4 : 2;
  return FP_OK;
}

fp_status fp_plan_set_mfma_min_m(fp_plan_t plan, int64_t min_m) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (min_m < 2 || min_m > FP_MAX_M + 1) return FP_ERR_INVALID_ARG;
  plan->mfma_min_m = min_m;
  return FP_OK;
}

fp_status fp_plan_set_tiling(fp_plan_t plan, int64_t M, const fp_tiling* t) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  if (M < 1 || M > plan->max_M) return FP_ERR_INVALID_ARG;
  if (t == nullptr) {
    plan->has_override[M] = false;
    return FP_OK;
  }
  const bool prev = plan->has_override[M];
  const fp_tiling prev_t = plan->override_t[M];
  plan->override_t[M] = *t;
  plan->has_override[M] = true;
  // must be runnable for the fused launch and for every separate launch
  Tiling chk;
  bool ok = choose_tiling(plan, M, plan->n_total, &chk);
  for (int i = 0; ok && i < plan->n_proj; ++i) ok = choose_tiling(plan, M, plan->N[i], &chk);
  if (!ok) {
    // distinguish a workspace shortfall from an unrunnable tiling
    const size_t saved = plan->ws_bytes;
    plan->ws_bytes = SIZE_MAX;
    bool ok_big = choose_tiling(plan, M, plan->n_total, &chk);
    for (int i = 0; ok_big && i < plan->n_proj; ++i)
      ok_big = choose_tiling(plan, M, plan->N[i], &chk);
    plan->ws_bytes = saved;
    plan->has_override[M] = prev;
    plan->override_t[M] = prev_t;
    return ok_big ? FP_ERR_WORKSPACE : FP_ERR_UNSUPPORTED;
  }
  return FP_OK;
}

fp_status fp_plan_get_tiling(fp_plan_t plan, int64_t M, int64_t n_rows, fp_tiling* out) {
  if (!plan_ok(plan) || out == nullptr) return FP_ERR_INVALID_ARG;
  if (M < 1 || M > plan->max_M || n_rows < 1 || n_rows > plan->n_total)
    return FP_ERR_INVALID_ARG;
  Tiling t;
  if (!choose_tiling(plan, M, n_rows, &t)) return FP_ERR_UNSUPPORTED;
  out->path = t.path;
  out->kparts = t.kparts;
  out->chunks = t.chunks;
  out->splits = t.splits;
  out->rows = t.rows;
  out->groups = t.groups;
  return FP_OK;
}

fp_status fp_default_tiling(int32_t dtype, int64_t K, int64_t n_total, int64_t M,
                            int64_t n_rows, fp_tiling* out) {
  if (out == nullptr || !dtype_known(dtype) || K < 1 ||
      n_total < 1)
    return FP_ERR_INVALID_ARG;
  int esize = 0;
  int64_t wrow = 0, kc = 0;
  if (!dtype_geometry(dtype, K, &esize, &wrow, &kc)) return FP_ERR_UNSUPPORTED;
  if (M < 1 || M > FP_MAX_M || n_rows < 1 || n_rows > n_total) return FP_ERR_INVALID_ARG;
  fp_plan_s tmp;
  standin_plan(&tmp, dtype, K, n_total, FP_MAX_M);
  Tiling t;
  if (!choose_tiling(&tmp, M, n_rows, &t)) return FP_ERR_UNSUPPORTED;
  out->path = t.path;
  out->kparts = t.kparts;
  out->chunks = t.chunks;
  out->splits = t.splits;
  out->rows = t.rows;
  out->groups = t.groups;
  return FP_OK;
}

const char* fp_status_str(int32_t status) {
  switch (status) {
    case FP_OK: return "ok";
    case FP_ERR_INVALID_ARG: return "invalid argument";
    case FP_ERR_UNSUPPORTED: return "unsupported by the fused kernels";
    case FP_ERR_HIP: return "HIP error";
    case FP_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int32_t fp_last_hip_error(void) { return g_last_hip; }

}  // extern "C"

// ---------------------------------------------------------- no-allocation form
// fp_forward_noalloc keeps the split-K state of its launches in `scratch`, a
// device array of this library (each GPU the library runs on holds its own
// copy until the process ends), instead of the plan's workspace.  Layout:
// the arrival counters (one uint32 per row of the plan, zero between calls)
// in the first kScratchCounterBytes, the fp32 partial sums after them, so
// plans of any row count leave each other's counters untouched.  Every call
// on one GPU shares the array; calls that overlap on one GPU race.
namespace {

constexpr size_t kScratchBytes = (size_t)24 << 20;
constexpr size_t kScratchCounterBytes = (size_t)256 << 10;  // 65536 rows
constexpr int kScratchMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per device: the address of its copy of `scratch` (host code never uses
// the array's own name as a device address).
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kScratchMaxDevices];

// The current device's scratch address.  On the first call on a device
// (with that device current) it looks the address up and clears the
// counter words with the fill kernel on `stream` (a kernel, not a memset:
// graph-capture friendly).  Allocates nothing.
fp_status scratch_for_stream(hipStream_t stream, unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kScratchMaxDevices) return FP_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e);
    if (sdev != dev) return FP_ERR_INVALID_ARG;  // the stream's device must be current
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorUnknown);
    uint32_t* cptr = static_cast<uint32_t*>(ptr);
    int64_t nc = (int64_t)(kScratchCounterBytes / 4);
    uint32_t zero = 0u;
    void* fargs[] = {&cptr, &nc, &zero};
    e = hipLaunchKernel(fpk::fill_u32(), dim3((unsigned)ceil_div(nc, 256)), dim3(256), fargs, 0,
                        stream);
    if (e != hipSuccess) return hip_fail(e);
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return FP_OK;
}

}  // namespace

extern "C" {

fp_status fp_forward_noalloc(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                             void* stream, void* const* y) {
  if (!plan_ok(plan)) return FP_ERR_INVALID_ARG;
  fp_status s = check_x(plan, M, x, ldx);
  if (s != FP_OK) return s;
  if (M == 0) return FP_OK;
  s = check_outputs(plan, M, x, ldx, y);
  if (s != FP_OK) return s;
  // the scratch's capacity takes the place of the plan's workspace; the
  // tiling is the plan's (same kernels, same bits as fp_forward)
  if (counters_bytes(plan->n_total) > (int64_t)kScratchCounterBytes) return FP_ERR_WORKSPACE;
  WsView cap;
  cap.counters = nullptr;
  cap.partial = nullptr;
  cap.counter_bytes = (int64_t)kScratchCounterBytes;
  cap.partial_bytes = (int64_t)(kScratchBytes - kScratchCounterBytes);
  Tiling t;
  if (!choose_tiling(plan, M, plan->n_total, &t, false, &cap)) {
    // runnable with the plan's own workspace: the partials exceed the scratch
    Tiling t2;
    return choose_tiling(plan, M, plan->n_total, &t2) ? FP_ERR_WORKSPACE : FP_ERR_UNSUPPORTED;
  }
  unsigned char* base = nullptr;
  s = scratch_for_stream(static_cast<hipStream_t>(stream), &base);
  if (s != FP_OK) return s;
  WsView ws = cap;
  ws.counters = base;
  ws.partial = base + kScratchCounterBytes;
  LaunchRows lr;
  std::memset(&lr, 0, sizeof lr);
  lr.w = plan->w_cat;
  lr.n_seg = plan->n_proj;
  lr.n_rows = (int)plan->n_total;
  for (int i = 0; i < plan->n_proj; ++i) {
    lr.y[i] = static_cast<unsigned char*>(y[i]);
    lr.begin[i] = (int)plan->off[i];
    lr.scale[i] = plan->tscale[i];
  }
  lr.begin[plan->n_proj] = (int)plan->n_total;
  return run(plan, t, lr, x, M, ldx, static_cast<hipStream_t>(stream), false, &ws);
}

}  // extern "C"
