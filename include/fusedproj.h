/*
 * fusedproj.h -- C ABI of libfusedproj, the fused decode-time hidden-state
 * projection for MI355X (gfx950).
 *
 * The operation.  Several linear projections that read the same activations
 * x[M, K] (for example DeepSeek-V4.1's wq_a 5120->1280 and wkv 5120->512)
 * have their weights W_i[N_i, K] copied once into one row-concatenated
 * buffer W_cat[sum_i N_i, K]; one skinny GEMM y = x . W_cat^T then computes
 * all of them and each projection's result is returned as its own dense
 * [M, N_i] tensor:
 *     y_i[m, r] = sum_k x[m, k] * W_i[r, k]            (no bias)
 * Sources (TensorRT-LLM pull-request pages):
 *   "tinygemm2 for the DeepSeek-V4.1 hidden-state projections" (PR #20636),
 *     Description: the [1792, 5120] concatenation done after weight load,
 *     the two weights rebound as views into it, reloads writing through the
 *     views, the fused call returning dense [M, N] halves, and the fallback
 *     list for inputs the fast path does not serve; Test Coverage: graph
 *     replay bitwise equal to eager.
 *   "Fuse indexer wk + weights_proj into single GEMM in TF32 for DS-V3.2"
 *     (PR #12055), Description: the FP32 variant (computed here with exact
 *     fp32 FMA, not TF32).
 *   "Staircase: GLM-5.2 NVFP4 low-latency decode target for Rubin (TP16)"
 *     (PR #20502), fused-A and dense-MLP commits: fixed-order fp32 sums,
 *     rounded to bf16 once; a host "supported" query and refusal of shapes
 *     the kernels do not serve.
 *
 * Conventions for every function below.
 *   - All pointers named w_*, x, y, w_cat and workspace are DEVICE pointers
 *     (memory the caller allocated on the plan's GPU); N and other arrays
 *     are HOST pointers.  `stream` is a hipStream_t passed as void*
 *     (NULL = the device's null stream).
 *   - Matrices are row-major with unit column stride.  Sizes, offsets and
 *     strides are int64_t element counts.
 *   - Every function returns an fp_status.  All argument and shape checks
 *     happen before any HIP call, so a call that fails validation has no
 *     side effect.  No exception crosses the ABI.
 *   - The library never allocates device memory and never synchronizes:
 *     fp_plan_create and the forward calls only enqueue work on `stream`.
 *   - Ownership: the caller owns w_cat, workspace, x and every y; a plan
 *     borrows w_cat and workspace and must be destroyed before they are
 *     freed.  A plan holds only host state besides those borrowed buffers.
 *   - Concurrency: the forward calls of one plan use the plan's workspace;
 *     two calls of the same plan must not run concurrently (on two streams);
 *     create one plan per stream for that.
 */
#ifndef FUSEDPROJ_H
#define FUSEDPROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fp_plan_s* fp_plan_t;

/* Storage and arithmetic type.  FP_BF16: bf16 inputs and outputs, fp32
 * accumulation, each output rounded once to bf16 (round to nearest even).
 * FP_F32: fp32 inputs and outputs with fp32 fused multiply-add.
 * FP_MXFP8: MXFP8 weights (the MXFP8 projections named in PR #20636,
 * Description; read as the open microscaling format: E4M3 codes, one E8M0
 * scale 2^(s-127) per 32 consecutive elements along K), bf16 activations and
 * outputs, fp32 accumulation, outputs rounded once to bf16.  Weight rows
 * are packed: the K codes, then the K/32 scales (K + K/32 bytes per row; K
 * a multiple of 512).  Every weight element is decoded exactly (an E4M3
 * value times a power of two) for scaled values inside bf16's normal range;
 * NaN codes and scales (0x7F/0xFF, 255) and scales above 2^119 are outside
 * the served domain.  Served for 1 <= M <= 16: the vector-ALU kernel up
 * to 4 tokens, the small-M matrix-core kernel (weights decoded to bf16 in
 * the registers feeding the matrix unit; two token halves above 8) from 5
 * (by default; tilings may pick either kernel up to 8 tokens).  Two token
 * halves need K <= 8192 (one workgroup spans K); 9..16 tokens on longer
 * rows return FP_ERR_UNSUPPORTED.
 * FP_MXFP4: the same with E2M1 elements (sign, 2 exponent bits of bias 1,
 * 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), the FP4 form of the fused
 * weight named in PR #8771; two codes per byte, element 2i in the low
 * nibble; a row is its K/2 code bytes, then its K/32 scales (K/2 + K/32
 * bytes, K a multiple of 512).
 * FP_NVFP4: the FP4 checkpoint form of the pages' fused weight (PR #8771,
 * first titled as NVFP4 only; the GLM-5.2 NVFP4 target of PR #20502), read
 * as the public two-level NVFP4 format: E2M1 codes as FP_MXFP4, one E4M3
 * scale per 16 consecutive elements along K, and one fp32 scale per
 * projection (fp_plan_set_tensor_scales, default 1).  A row is its K/2
 * code bytes, then its K/16 scale bytes (K/2 + K/16 bytes, K a multiple of
 * 512).  Each weight is decoded exactly as E2M1 x E4M3 (at most 6
 * significant bits); each output's fp32 sum is multiplied by its
 * projection's tensor scale in fp32, then rounded once to bf16.  Served as
 * FP_MXFP4 (1 <= M <= 16). */
typedef enum { FP_BF16 = 0, FP_F32 = 1, FP_MXFP8 = 2, FP_MXFP4 = 3, FP_NVFP4 = 4 } fp_dtype;

typedef enum {
  FP_OK = 0,
  FP_ERR_INVALID_ARG = 1,  /* null/negative/inconsistent argument, stale plan */
  FP_ERR_UNSUPPORTED = 2,  /* valid request the kernels do not serve (e.g.
                              misaligned x, M above the plan's max_M): the
                              caller falls back to its plain linear layers */
  FP_ERR_HIP = 3,          /* a HIP call failed; see fp_last_hip_error() */
  FP_ERR_WORKSPACE = 4     /* workspace smaller than fp_workspace_bytes() */
} fp_status;

/* Kernel paths reported by fp_plan_query. */
typedef enum {
  FP_PATH_NONE = 0,        /* M == 0: nothing is launched */
  FP_PATH_SKINNY = 1,      /* weight-streaming vector-ALU kernel, one launch */
  FP_PATH_SKINNY_SPLITK = 2, /* same kernel with the K contraction split
                              across workgroups and a fixed-order finish
                              inside the same launch */
  FP_PATH_MFMA = 3,        /* MFMA tile kernels (bf16, M above the crossover,
                              or plans the small-M kernel cannot cover in
                              one round): the tile and weight-resident
                              kernels (K slice in LDS) to 32 tokens and for
                              65..128, the ring tile kernel (K slice streamed
                              through a ring of LDS stages) for 33..64,
                              above 128 and on large plans */
  FP_PATH_MFMA_SMALL = 4   /* matrix-core kernel for few tokens (bf16 M <= 24,
                              block-scaled M <= 16): 8-row x 2-sub-slice
                              tiles, one or two per wave, one launch */
} fp_path;

#define FP_MAX_PROJ 16     /* projections per plan */
#define FP_MAX_M 256       /* largest token count a plan can serve */

/* Bytes of device workspace a plan needs (split-K partial sums and the
 * self-resetting arrival counters), for dtype `dtype`, contraction length K,
 * the n_proj row counts N[] and token counts up to max_M.  The fp32 sums
 * of a row's K slices are kept apart and added in a fixed order ("FP32 in a
 * fixed order", dense-MLP commit of PR #20502; the fused-A commit splits
 * its 6144 contraction over two CTAs the same way), which is what needs
 * this memory.  Returns 0 on an
 * invalid argument (and for shapes that need no workspace it still returns a
 * small positive size for the counters). */
size_t fp_workspace_bytes(int32_t dtype, int64_t K, int32_t n_proj,
                          const int64_t* N, int64_t max_M);

/* Load-time half ("post_load_weights" of PR #20636, Description).
 * Records the projection layout and, on `stream`, copies each w_src[i]
 * (device, [N[i], K] contiguous row-major; FP_MXFP8 / FP_MXFP4: N[i]
 * packed rows of K + K/32 / K/2 + K/32 bytes) into rows off_i ..
 * off_i+N[i]-1 of w_cat (device, [sum N, K] row-major, or sum N packed rows
 * for the MX formats, 256-byte
 * aligned), where off_0 = 0 and off_{i+1} = off_i + N[i].  A NULL w_src (or
 * a NULL entry, or an entry equal to its destination) skips that copy: the
 * caller fills the rows itself, typically through the views fp_plan_view
 * returns.  The workspace (device, ws_bytes >= fp_workspace_bytes(...),
 * 256-byte aligned) has its counters cleared on `stream` by a fill kernel.
 * Requirements: 1 <= n_proj <= FP_MAX_PROJ, every N[i] >= 1, K >= 1 with
 * K * sizeof(element) a multiple of 16 (MX formats: K a multiple of 512),
 * 1 <= max_M <= FP_MAX_M.
 * On success *out receives the plan. */
fp_status fp_plan_create(int32_t dtype, int64_t K, int32_t n_proj,
                         const int64_t* N, const void* const* w_src,
                         void* w_cat, void* workspace, size_t ws_bytes,
                         int64_t max_M, void* stream, fp_plan_t* out);

/* View of projection i inside w_cat: *w_i = w_cat + off_i * K elements,
 * *row_offset = off_i, *rows = N[i].  Any output pointer may be NULL.
 * Writing new weights through a view (an in-place checkpoint reload, as in
 * PR #20636) keeps the fused path valid: no kernel reads a derived copy. */
fp_status fp_plan_view(fp_plan_t plan, int32_t i, void** w_i,
                       int64_t* row_offset, int64_t* rows);

/* Frees the plan's host state.  The borrowed buffers are untouched: the
 * concatenated weight and its views outlive the plan, as the fused buffer
 * of PR #20636 (Description) outlives the modules that view it.  A stale or
 * already destroyed plan returns FP_ERR_INVALID_ARG. */
fp_status fp_plan_destroy(fp_plan_t plan);

/* Host-only predicate (no HIP call): FP_OK if fp_forward serves token count
 * M with x (device pointer, row stride ldx elements), FP_ERR_UNSUPPORTED if
 * the kernels do not (M > max_M, x or its row stride not 16-byte aligned,
 * fp32 with M > 8, launches past 32-bit indexing: M * N_i outputs of one
 * projection at or above 2^31, or on the matrix-core tile path more than
 * 2^31 bytes of weights, activations or split-K partials per launch),
 * FP_ERR_INVALID_ARG for invalid arguments (ldx < K,
 * M < 0, NULL x with M > 0, stale plan).  The pattern of the dense-MLP
 * commit of PR #20502: a host query, refusal otherwise. */
fp_status fp_supported(fp_plan_t plan, int64_t M, const void* x, int64_t ldx);

/* Dequantise MXFP8 weight rows: w (device, `rows` packed rows of K codes and
 * K/32 scales, 16-byte aligned) to out (device, dense [rows, K] bf16,
 * 16-byte aligned, not overlapping w), with the decode the FP_MXFP8
 * projection uses.  For a caller that needs the weights as bf16 (a fallback
 * linear layer).  K a multiple of 512. */
fp_status fp_mxfp8_to_bf16(const void* w, int64_t rows, int64_t K, void* out,
                           void* stream);

/* Dequantise MXFP4 weight rows (K/2 code bytes, low nibble first, then K/32
 * scales; 16-byte aligned) to dense [rows, K] bf16 (16-byte aligned, not
 * overlapping w), with the decode the FP_MXFP4 projection uses.  K a
 * multiple of 512. */
fp_status fp_mxfp4_to_bf16(const void* w, int64_t rows, int64_t K, void* out,
                           void* stream);

/* Dequantise NVFP4 weight rows (K/2 code bytes, low nibble first, then
 * K/16 E4M3 scales) with tensor scale g: out[r, k] = bf16(e2m1 * e4m3 * g),
 * the E2M1 x E4M3 product exact, times g in fp32, rounded once (nearest
 * even).  w, out as fp_mxfp8_to_bf16 (device, 16-byte aligned, not
 * overlapping); K a multiple of 512 (else FP_ERR_UNSUPPORTED); g finite
 * (else FP_ERR_INVALID_ARG).  Asynchronous on `stream`. */
fp_status fp_nvfp4_to_bf16(const void* w, int64_t rows, int64_t K, float g, void* out,
                           void* stream);

/* NVFP4 plans: the fp32 tensor scale of each projection (host array of the
 * plan's n_proj values, finite; copied).  FP_ERR_UNSUPPORTED for other
 * dtypes, FP_ERR_INVALID_ARG for a null plan, null array or a non-finite
 * value (nothing changed then).  Host-only; call it before the plan's
 * forward calls (captured graphs keep the scales of their capture). */
fp_status fp_plan_set_tensor_scales(fp_plan_t plan, const float* scales);

/* Measurement aid (no projection): read `bytes` of device memory at `buf`
 * the way the fused call reads W_cat -- 256 workgroups of 640 threads,
 * workgroup b reading the b-th contiguous 1/256 of the buffer with 16-byte
 * non-temporal loads, all of a lane's loads issued before any is used --
 * and do nothing else.  Its time per call is the read-only streaming
 * ceiling of the projection kernels on the machine it runs on (the
 * "weights rotated past L2" protocol of "tinygemm2 for the DeepSeek-V4.1
 * hidden-state projections", Description).  buf 16-byte aligned, bytes a
 * multiple of 16 below 2^31 (else FP_ERR_UNSUPPORTED); sink: device, 256
 * words, not overlapping buf, written only in a case that never occurs
 * for real data (it keeps the loads from being removed).  Asynchronous on
 * `stream`. */
fp_status fp_stream_read(const void* buf, int64_t bytes, void* sink, void* stream);

/* Measurement aid: fp_stream_read with the launch shape as a parameter --
 * `groups` workgroups (1..65536) of `threads` threads (a multiple of 64, at
 * most 1024 for batch 8 and 16, 512 for batch 32), workgroup b reading the
 * b-th contiguous 1/groups of the buffer, `batch` (8, 16 or 32) 16-byte
 * non-temporal loads in flight per lane.  Times of the shapes on one pool
 * show whether the streaming ceiling depends on the launch shape (the
 * "weights rotated past L2" protocol of "tinygemm2 for the DeepSeek-V4.1
 * hidden-state projections", Description, applied to a read-only stream).
 * buf and bytes as fp_stream_read; sink: device, `groups` words, not
 * overlapping buf.  FP_ERR_UNSUPPORTED for shapes outside these limits,
 * FP_ERR_INVALID_ARG for negative or null arguments.  Asynchronous on
 * `stream`. */
fp_status fp_stream_read_shaped(const void* buf, int64_t bytes, int32_t groups,
                                int32_t threads, int32_t batch, void* sink, void* stream);

/* The fused call: one launch computes every projection ("one call for the
 * fused weight", the halves "returned with dense strides": PR #20636,
 * Description; outputs rounded to bf16 once from fp32 sums added in a fixed
 * order: fused-A commit of PR #20502).
 * x: device, M rows with row stride ldx >= K elements (x[m, k] at
 *    x + m*ldx + k), 16-byte aligned rows.
 * y: host array of n_proj device pointers; y[i] receives the dense
 *    [M, N_i] result (y_i[m, r] at y[i] + m*N_i + r).  Outputs must not
 *    overlap each other, x, w_cat or the workspace.
 * M == 0 returns FP_OK and launches nothing.  Results are deterministic: a
 * repeat, a graph replay and fp_forward_separate give bitwise equal y. */
fp_status fp_forward(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                     void* stream, void* const* y);

/* The comparison path: one launch per projection, each over its own rows.
 * w_override: NULL, or a host array of n_proj entries where a non-NULL
 * entry is a device [N_i, K] weight used instead of the view (a replaced
 * Parameter that no longer aliases w_cat, PR #20636 Test Coverage).  With
 * no override the outputs are bitwise equal to fp_forward's. */
fp_status fp_forward_separate(const void* x, int64_t M, int64_t ldx,
                              fp_plan_t plan, void* stream, void* const* y,
                              const void* const* w_override);

/* ---------------------------------------------------------------------
 * Epilogues: the step that consumes the projection.  Both read the
 * projection after its single rounding to bf16, as the unfused chain (one
 * projection launch per projection, then a second kernel) does, and both
 * give results bitwise equal to that chain (fp_forward_separate followed by
 * fp_rmsnorm / fp_swiglu on its outputs).  RMSNorm: bf16 and MX plans;
 * SwiGLU: bf16 plans; other cases return FP_ERR_UNSUPPORTED with no launch.
 * --------------------------------------------------------------------- */

/* Fused projection + RMSNorm per projection (q_norm over the q_a columns and
 * kv_norm over the kv columns that consume the fused wq_a/wkv projection in
 * PR #20636, Description):
 *     v = bf16(x . W_i^T)                      (the projection, rounded once)
 *     out_i[m, j] = bf16( v[m, j] * rinv_m * gamma_i[j] ),
 *     rinv_m = 1 / sqrt( (1/N_i) sum_j v[m, j]^2 + eps )     (fp32 arithmetic)
 * Two launches for any number of projections: the fused projection into
 * out[], then one normalisation launch over every normalised (projection,
 * token) row, in place.  (A finish inside the projection launch was measured
 * slower on MI355X: its cross-workgroup arrival alone costs about a kernel
 * boundary.)  Serves every M the plan's fused call serves.
 * gamma: host array of n_proj entries; entry i is a device bf16 [N_i] gain
 *   (16-byte aligned, N_i a multiple of 8, N_i <= 2048) or NULL, in which
 *   case out_i receives the projection itself.
 * out: host array of n_proj device pointers, dense [M, N_i] bf16, 16-byte
 *   aligned where normalised; no overlap with each other, x, w_cat, the
 *   workspace or a gain.
 * eps: finite, >= 0. */
fp_status fp_forward_rmsnorm(const void* x, int64_t M, int64_t ldx,
                             fp_plan_t plan, void* stream,
                             const void* const* gamma, float eps,
                             void* const* out);

/* Fused gate/up projection + SwiGLU (dense-MLP commit of PR #20502), one
 * launch: the plan holds exactly two projections of equal width N (the gate
 * rows, then the up rows, N a multiple of 8); the launch takes the rows in
 * (gate j, up j) pairs so that one workgroup owns both rows of an output
 * column, and
 *     g = bf16(x . W_gate^T),  u = bf16(x . W_up^T)
 *     h[m, j] = bf16( g / (1 + exp(-g)) * u )     (fp32 arithmetic)
 * 1 <= M <= 8.  h: device, dense [M, N] bf16, 16-byte aligned, no overlap
 * with x, w_cat or the workspace.  FP_ERR_INVALID_ARG if the plan is not
 * such a pair. */
fp_status fp_forward_swiglu(const void* x, int64_t M, int64_t ldx,
                            fp_plan_t plan, void* stream, void* h);

/* The unfused second step of the chain: RMSNorm of y (device, dense [M, N]
 * bf16) with gain gamma (device, bf16 [N]) into out (device, dense [M, N]
 * bf16; out == y normalises in place, other overlaps are refused), with the
 * arithmetic of fp_forward_rmsnorm.  All three pointers 16-byte aligned,
 * N a multiple of 8 and at most 2048.  M == 0 launches nothing. */
fp_status fp_rmsnorm(const void* y, int64_t M, int64_t N, const void* gamma,
                     float eps, void* out, void* stream);

/* The unfused second step of the gate/up chain: h = bf16(silu(g) * u)
 * elementwise over dense [M, N] bf16 tensors g, u, h (device, 16-byte
 * aligned, N a multiple of 8; h may be g or u, other overlaps are refused),
 * with the arithmetic of fp_forward_swiglu. */
fp_status fp_swiglu(const void* g, const void* u, int64_t M, int64_t N,
                    void* h, void* stream);

/* Which kernel fp_forward runs for M, and how many kernel launches
 * fp_forward and fp_forward_separate make (0 for M == 0; a split tile
 * launch whose slices are added in a second launch counts two).  Any output
 * pointer may be NULL.  Host-only. */
fp_status fp_plan_query(fp_plan_t plan, int64_t M, int32_t* path,
                        int32_t* launches_fused, int32_t* launches_separate);

/* Output type of a plan's projections (default: the input type).  A bf16
 * plan may store fp32 outputs (FP_F32): the fp32 sums are stored without
 * rounding, as the router GEMV of PR #20502 (dense-MLP/router commits: bf16
 * operands, fp32 logits, checked against an FP64 reference) needs.  Such a
 * plan runs the vector-ALU kernel for 1 <= M <= 16 (9..16 tokens on rows
 * of more than 8192 elements split K across workgroups, added in the same
 * launch; M above 16 is FP_ERR_UNSUPPORTED), takes fp32 output buffers in
 * every forward call, and
 * has no epilogue forms.  An fp32 plan accepts only FP_F32.  Host-only; call
 * it before the plan's forward calls. */
fp_status fp_plan_set_out_dtype(fp_plan_t plan, int32_t out_dtype);

/* Smallest M served by the MFMA tile path (bf16 plans; default: the
 * measured crossover).  Values below 2 or above FP_MAX_M+1 are rejected.
 * Changing it changes which kernel (hence which summation order) serves an
 * M, so results for that M may differ bitwise from before the change. */
fp_status fp_plan_set_mfma_min_m(fp_plan_t plan, int64_t min_m);

/* Tiling of one token count (benchmarking and testing aid).  Every tiling
 * the kernels accept gives results within the same error bound; the
 * summation order, hence the exact bits, depends on path and the order
 * fields (skinny: kparts, chunks, splits; mfma-small: kparts, chunks;
 * mfma: splits) -- never on rows, groups or the tile kernels' kparts and
 * chunks (the two tile kernels give the same bits for the same splits) --
 * so fused and separate calls of one plan stay bitwise equal under any
 * tiling.
 *   path    FP_PATH_SKINNY / FP_PATH_SKINNY_SPLITK (same kernel; the
 *           splits field decides), FP_PATH_MFMA_SMALL (M <= 24; block-
 *           scaled weights M <= 16) or
 *           FP_PATH_MFMA (the tile kernels, bf16)
 *   kparts  skinny: waves splitting one K slice (P, <= 16); mfma-small:
 *           waves splitting K (PK, <= 16); mfma: 16-row tiles per
 *           workgroup (tile kernel: 2, 4 or 8, 0 = chosen per launch;
 *           ring kernel: 4)
 *   chunks  skinny: 16-byte chunks per lane and row (CJ, 1..2);
 *           mfma-small: MFMA steps of 64 k per wave (KT: 4, 8, 16);
 *           mfma: 3, 4 or 6 select the ring kernel with that many stage
 *           buffers of 64 k (3 only for more than 128 tokens, 6 only up to
 *           64); otherwise the tile kernel's compiled bound of 32-wide k
 *           steps per slice (8, 10, 16, 20 or 40, at least
 *           ceil(ceil(K/32) / splits); 0 = smallest)
 *   splits  K slices across workgroups (S >= 1), finished in-launch
 *           (mfma-small: 1)
 *   rows    skinny: rows per wave (RW, 1..8); mfma-small: rows per row
 *           group, 1..8 as one tile, or an even 10..16 as two tiles of
 *           rows / 2 per wave sharing the activations (bf16, not gate/up);
 *           0 = chosen per launch from its row count; mfma: unused
 *   groups  skinny and mfma-small: row groups per workgroup (G); 0 =
 *           chosen per launch; mfma: how the K slices are added -- 1 by
 *           the last workgroup of each row block, in the launch; 2 by a
 *           second launch spread over the GPU (same order, same bits); 0 =
 *           chosen per launch (second launch when a row block's partials
 *           exceed 64 KiB) */
typedef struct {
  int32_t path;
  int32_t kparts;
  int32_t chunks;
  int32_t splits;
  int32_t rows;
  int32_t groups;
} fp_tiling;

/* Override the tiling used for token count M (1 <= M <= the plan's max_M),
 * or restore the default with t == NULL.  Host-only.  Returns
 * FP_ERR_UNSUPPORTED for a tiling the kernels cannot run (block larger than
 * 1024 threads, LDS above 160 KiB, K not covered, no such kernel) and
 * FP_ERR_WORKSPACE if its split-K partials do not fit the plan's
 * workspace. */
fp_status fp_plan_set_tiling(fp_plan_t plan, int64_t M, const fp_tiling* t);

/* The tiling fp_forward would use for M on a launch of n_rows rows (pass
 * the plan's total rows for the fused call), with rows/groups resolved. */
fp_status fp_plan_get_tiling(fp_plan_t plan, int64_t M, int64_t n_rows,
                             fp_tiling* out);

/* Host-only, no plan needed: the tiling a plan of (dtype, K, n_total rows)
 * uses by default (default crossover, no override) for token count M on a
 * launch of n_rows rows (1 <= n_rows <= n_total).  FP_ERR_UNSUPPORTED if no
 * kernel serves M. */
fp_status fp_default_tiling(int32_t dtype, int64_t K, int64_t n_total, int64_t M,
                            int64_t n_rows, fp_tiling* out);

/* The fused call without a caller-provided workspace, for callers that
 * cannot allocate device memory at call time or hold a workspace per plan
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments, checks, kernels and results are fp_forward's
 * (bitwise equal outputs), but the split-K arrival counters and partial
 * sums live in a static device array of the library -- 24 MiB per GPU,
 * held until the process ends: the first 256 KiB hold the counters (plans
 * of at most 65536 rows), the rest the partials -- instead of the plan's
 * workspace, which this call does not touch.  It calls no allocating
 * routine.  The first call on a device looks the array up and clears its
 * counter words with a fill kernel on `stream`; every call leaves the
 * counters at zero.  `stream` must belong to the current device
 * (FP_ERR_INVALID_ARG otherwise).  FP_ERR_WORKSPACE when the call's
 * counters or partials exceed the array (the plan's rows, or a tiling with
 * more split-K partials than fit), with no launch.  All calls on one GPU
 * share the array: calls that overlap on one GPU (two streams, two
 * threads) race and must be ordered by the caller. */
fp_status fp_forward_noalloc(const void* x, int64_t M, int64_t ldx, fp_plan_t plan,
                             void* stream, void* const* y);

/* Static text for a status code: the reason a call was refused, for the
 * caller's fallback to its plain linear layers (the fallback list of PR
 * #20636, Description; "raise otherwise" in the dense-MLP commit of PR
 * #20502). */
const char* fp_status_str(int32_t status);

/* The hipError_t of the last failing HIP call made by this thread (the
 * detail behind FP_ERR_HIP; the C ABI carries no exceptions, the
 * boundary the dense-MLP commit of PR #20502 draws with its host query). */
int32_t fp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDPROJ_H */
