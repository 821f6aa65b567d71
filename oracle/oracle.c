/*
 * oracle.c -- plain, slow, obviously correct CPU reference of the fused
 * decode-time hidden-state projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library (it decodes bf16 and rounds to bf16 with its own code).
 *
 * What it computes (the plain definition the fusion must reach):
 *   for every projection i, token row m and output row r
 *     y_i[m][r] = sum_k X[m][k] * W_i[r][k]          (no bias)
 *     S_i[m][r] = sum_k |X[m][k] * W_i[r][k]|        (error-bound scale)
 * The fusion of several projections that read the same activations into one
 * GEMM over the row-concatenated weight returns exactly these per-projection
 * linear layers, only with fewer launches:
 *   - "tinygemm2 for the DeepSeek-V4.1 hidden-state projections"
 *     (TensorRT-LLM PR #20636), Description: wq_a and wkv concatenated into
 *     one [1792, 5120] weight, the halves returned as dense [1, N] tensors,
 *     checked against an FP32 F.linear reference (Test Coverage).
 *   - "Fuse indexer wk + weights_proj into single GEMM in TF32 for DS-V3.2"
 *     (TensorRT-LLM PR #12055), Description: two FP32 projections, one GEMM.
 *
 * Arithmetic: each stored element is decoded to its exact value, each
 * product is formed in IEEE double (exact: a bf16 x bf16 product has at most
 * 16 significant bits and an fp32 x fp32 product at most 48, both below 53),
 * and products are added in double in increasing k.  The only rounding is
 * the double accumulation, at most K * 2^-53 * S in total.  An FP64
 * reference is the pattern of the router GEMV commit of "Staircase: GLM-5.2
 * NVFP4 low-latency decode target for Rubin (TP16)" (TensorRT-LLM PR #20502).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: IEEE semantics are
 * needed; OpenMP only spreads oracle_linear_omp's output elements).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact value of a bf16 bit pattern: bf16 is the upper half of an IEEE
 * binary32, so widening is a 16-bit left shift of the pattern. */
static double bf16_bits_value(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double f32_bits_value(uint32_t bits) {
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* dtype codes of this file: 0 = bf16 (uint16 patterns), 1 = fp32 (uint32). */
static double element(int dtype, const void* base, int64_t idx) {
  if (dtype == 0) return bf16_bits_value(((const uint16_t*)base)[idx]);
  return f32_bits_value(((const uint32_t*)base)[idx]);
}

/*
 * One linear projection: y[m][r] and S[m][r] for m < M, r < N.
 *   x : M rows, row stride ldx elements (ldx >= K), unit column stride
 *   w : N rows of K elements, row stride K
 *   y, s : M x N doubles, row-major
 * Returns 0, or -1 on a bad argument.
 */
int oracle_linear(int dtype, int64_t M, int64_t N, int64_t K, int64_t ldx,
                  const void* x, const void* w, double* y, double* s) {
  if ((dtype != 0 && dtype != 1) || M < 0 || N < 0 || K < 0 || ldx < K)
    return -1;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < N; ++r) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = element(dtype, x, m * ldx + k) * element(dtype, w, r * K + k);
        acc += p;
        mag += fabs(p);
      }
      y[m * N + r] = acc;
      s[m * N + r] = mag;
    }
  }
  return 0;
}

/*
 * oracle_linear with the (m, r) output elements spread over the host's
 * threads (OpenMP): each element is still the same sequential loop over k,
 * so the results are bitwise those of oracle_linear.  The multi-core form of
 * the CPU baseline; the acceptance tests use oracle_linear.
 */
int oracle_linear_omp(int dtype, int64_t M, int64_t N, int64_t K, int64_t ldx,
                      const void* x, const void* w, double* y, double* s) {
  if ((dtype != 0 && dtype != 1) || M < 0 || N < 0 || K < 0 || ldx < K)
    return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < N; ++r) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = element(dtype, x, m * ldx + k) * element(dtype, w, r * K + k);
        acc += p;
        mag += fabs(p);
      }
      y[m * N + r] = acc;
      s[m * N + r] = mag;
    }
  }
  return 0;
}

/* Threads oracle_linear_omp runs on (1 when built without OpenMP). */
int oracle_omp_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Round a double to the nearest bf16, ties to even, with IEEE gradual
 * underflow (bf16 has float's exponent range: normal exponents -126..127,
 * 7 stored fraction bits, subnormal quantum 2^-133) and overflow to inf.
 * The reading of "rounded to BF16 once" in the fused-A commit of PR #20502
 * is IEEE round-to-nearest-even.  Written from the format definition: find
 * the quantum of the value's binade, divide (exact: a power of two), round to
 * an integer with nearbyint (ties-to-even in the default rounding mode),
 * multiply back.
 */
uint16_t oracle_round_bf16(double v) {
  if (isnan(v)) return (uint16_t)0x7fc0;
  uint16_t sign = signbit(v) ? (uint16_t)0x8000 : (uint16_t)0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7f80);
  int e;
  frexp(a, &e);             /* a = f * 2^e with f in [0.5, 1) */
  int E = e - 1;            /* a in [2^E, 2^(E+1)) */
  if (E < -126) E = -126;   /* subnormal range shares the smallest quantum */
  double q = ldexp(1.0, E - 7);
  double r = nearbyint(a / q) * q;
  const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (r > max_finite) return (uint16_t)(sign | 0x7f80);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7fff));
}

/* Vector form of oracle_round_bf16 for n doubles. */
void oracle_round_bf16_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);
}

/*
 * RMSNorm of each row of a bf16 matrix v[M][N] with a bf16 gain g[N]:
 *   ms[m]     = (1/N) * sum_j V[m][j]^2
 *   rinv[m]   = 1 / sqrt(ms[m] + eps)
 *   out[m][j] = V[m][j] * rinv[m] * G[j]
 * all in double, V and G the exact values of the stored patterns, no
 * rounding of the result (callers round with oracle_round_bf16).  The
 * normalisation that follows the fused projection: q_norm over the q_a
 * columns and kv_norm over the kv columns ("tinygemm2 for the
 * DeepSeek-V4.1 hidden-state projections", PR #20636, Description: the
 * projection's consumers are these RMSNorms), applied to the projection's
 * bf16 output as the unfused chain would (the GEMM rounds to bf16 once,
 * the norm reads that).  eps is the caller's value (the pages state none).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rmsnorm_bf16(int64_t M, int64_t N, const uint16_t* v, const uint16_t* g,
                        double eps, double* out, double* rinv) {
  if (M < 0 || N < 1 || !(eps >= 0.0)) return -1;
  for (int64_t m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t j = 0; j < N; ++j) {
      double a = bf16_bits_value(v[m * N + j]);
      ss += a * a;
    }
    double r = 1.0 / sqrt(ss / (double)N + eps);
    if (rinv) rinv[m] = r;
    for (int64_t j = 0; j < N; ++j)
      out[m * N + j] = bf16_bits_value(v[m * N + j]) * r * bf16_bits_value(g[j]);
  }
  return 0;
}

/*
 * SwiGLU of bf16 gate and up values, elementwise:
 *   h = silu(G) * U,   silu(G) = G / (1 + exp(-G))
 * in double, from the exact values of the stored patterns, unrounded.  The
 * gate/up + SwiGLU step of the dense-MLP commit of "Staircase: GLM-5.2
 * NVFP4 low-latency decode target for Rubin (TP16)" (PR #20502): the gate
 * and up sums are rounded to bf16 before SwiGLU (the callers pass those
 * rounded values) and h is rounded to bf16 once afterwards.
 */
int oracle_swiglu_bf16(int64_t n, const uint16_t* g, const uint16_t* u, double* h) {
  if (n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) {
    double a = bf16_bits_value(g[i]);
    h[i] = a / (1.0 + exp(-a)) * bf16_bits_value(u[i]);
  }
  return 0;
}

/*
 * MXFP8 weights (microscaling: 8-bit E4M3 elements sharing one 8-bit E8M0
 * power-of-two scale per block of 32 consecutive elements along K).  The
 * pages name MXFP8 projections for the DeepSeek-V4.1 wq_a / wkv weights
 * ("tinygemm2 for the DeepSeek-V4.1 hidden-state projections", PR #20636,
 * Description) without defining the encoding; the reading here is the open
 * microscaling format, written from its definition:
 *   E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 *         exponent 0: subnormal (m / 8) * 2^-6; otherwise (1 + m / 8) *
 *         2^(e - 7); exponent 15 with mantissa 7 is NaN (no infinities;
 *         largest finite 448).
 *   E8M0: an unsigned biased exponent, value 2^(s - 127); 255 is NaN.
 * Storage (this library's layout): each weight row is its K codes followed
 * by its K / 32 scales, so a row takes K + K / 32 bytes.
 */
static double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

static double e8m0_value(uint8_t s) {
  if (s == 255) return NAN;
  return ldexp(1.0, (int)s - 127);
}

double oracle_e4m3_value(uint8_t c) { return e4m3_value(c); }
double oracle_e8m0_value(uint8_t s) { return e8m0_value(s); }

/*
 * One projection with MXFP8 weights and bf16 activations:
 *   y[m][r] = sum_k X[m][k] * Q[r][k] * 2^(s[r][k / 32] - 127)
 *   S[m][r] = sum_k |X[m][k] * Q[r][k] * 2^(s[r][k / 32] - 127)|
 * X the exact bf16 values (row stride ldx >= K), Q the E4M3 values, w the
 * packed rows (K codes, then K / 32 scales; row stride K + K / 32 bytes).
 * Products are exact in double (at most 8 x 4 significant bits times a
 * power of two), sums in double in increasing k.  K must be a multiple of
 * 32.  Returns 0, or -1 on a bad argument.
 */
int oracle_linear_mxfp8(int64_t M, int64_t N, int64_t K, int64_t ldx, const uint16_t* x,
                        const uint8_t* w, double* y, double* s) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || ldx < K) return -1;
  const int64_t row = K + K / 32;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < N; ++r) {
      const uint8_t* q = w + r * row;
      const uint8_t* sc = q + K;
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = bf16_bits_value(x[m * ldx + k]) * (e4m3_value(q[k]) * e8m0_value(sc[k / 32]));
        acc += p;
        mag += fabs(p);
      }
      y[m * N + r] = acc;
      s[m * N + r] = mag;
    }
  }
  return 0;
}

/*
 * MXFP4 weights: 4-bit E2M1 elements sharing one E8M0 scale per block of 32
 * consecutive elements along K (the microscaling FP4 format; the pages'
 * quantized variants of the fused weight are FP4 checkpoints: "Fuse QK
 * down_proj with indexer K + weight_proj for FP4 ckpt", PR #8771).
 *   E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *         exponent 0: subnormal m * 0.5; otherwise (1 + m / 2) * 2^(e - 1);
 *         no infinities or NaN (values 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 * Storage (this library's layout): a row is its K / 2 code bytes, element
 * 2i in the low nibble of byte i and element 2i + 1 in the high nibble,
 * followed by its K / 32 scales (K / 2 + K / 32 bytes per row).
 */
static double e2m1_value(uint8_t c) {
  const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -v : v;
}

double oracle_e2m1_value(uint8_t c) { return e2m1_value(c & 0xF); }

int oracle_linear_mxfp4(int64_t M, int64_t N, int64_t K, int64_t ldx, const uint16_t* x,
                        const uint8_t* w, double* y, double* s) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || ldx < K) return -1;
  const int64_t row = K / 2 + K / 32;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < N; ++r) {
      const uint8_t* q = w + r * row;
      const uint8_t* sc = q + K / 2;
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const uint8_t code = (k & 1) ? (uint8_t)(q[k / 2] >> 4) : (uint8_t)(q[k / 2] & 0xF);
        double p = bf16_bits_value(x[m * ldx + k]) * (e2m1_value(code) * e8m0_value(sc[k / 32]));
        acc += p;
        mag += fabs(p);
      }
      y[m * N + r] = acc;
      s[m * N + r] = mag;
    }
  }
  return 0;
}

/*
 * NVFP4 weights: E2M1 elements (as above) with one E4M3 scale per block of
 * 16 consecutive elements along K and one fp32 scale g per tensor:
 *   w[r][k] = e2m1(q[r][k]) * e4m3(sc[r][k / 16]) * g
 * The pages' FP4 fused weight is the NVFP4 checkpoint of "Fuse QK down_proj
 * with indexer K + weight_proj for FP4 ckpt" (PR #8771, first titled as
 * NVFP4 only) and of the GLM-5.2 NVFP4 target (PR #20502); they do not
 * define the encoding, read as the public two-level NVFP4 format above.
 * Storage (this library's layout): a row is its K / 2 code bytes (element
 * 2i in the low nibble of byte i), then its K / 16 scale bytes (K / 2 +
 * K / 16 bytes per row).
 *   y[m][r] = sum_k X[m][k] * w[r][k],  S[m][r] = sum_k |X[m][k] * w[r][k]|
 * Each product is exact in double (bf16 x E2M1 x E4M3 x fp32: at most
 * 8 + 2 + 4 + 24 significant bits), sums in double in increasing k.  K a
 * multiple of 16; g finite.  Returns 0, or -1 on a bad argument.
 */
int oracle_linear_nvfp4(int64_t M, int64_t N, int64_t K, int64_t ldx, const uint16_t* x,
                        const uint8_t* w, float g, double* y, double* s) {
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || ldx < K || !isfinite(g)) return -1;
  const int64_t row = K / 2 + K / 16;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t r = 0; r < N; ++r) {
      const uint8_t* q = w + r * row;
      const uint8_t* sc = q + K / 2;
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const uint8_t code = (k & 1) ? (uint8_t)(q[k / 2] >> 4) : (uint8_t)(q[k / 2] & 0xF);
        const double wv = e2m1_value(code) * e4m3_value(sc[k / 16]) * (double)g;
        const double p = bf16_bits_value(x[m * ldx + k]) * wv;
        acc += p;
        mag += fabs(p);
      }
      y[m * N + r] = acc;
      s[m * N + r] = mag;
    }
  }
  return 0;
}
