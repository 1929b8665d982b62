/*
 * nvfp4_oracle.c -- plain, slow, obviously-correct CPU reference for the NVFP4
 * weight-only (W4A16) matmul.  fp64 throughout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; it shares no code, table or constant generator with the HIP
 * kernels.  Only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg may load it.
 *
 * What it follows (FlashRT, "Qwen3.6-27B NVFP4 on RTX 5090", section 1 "Model
 * dependencies", the compressed-tensors nvfp4-pack-quantized schema list):
 *   weight_packed        u8  (out, in/2)   FP4 E2M1 codes, two per byte
 *   weight_scale         E4M3 (out, in/16) one scale per 16 consecutive inputs
 *   weight_global_scale  fp32 scalar, equal to 448 / amax
 * and the dequantisation w = e2m1 * e4m3 / g.  The same section names the
 * format "NVFP4 W4A16": 4-bit weights, 16-bit (bf16) activations.
 *
 * Readings where the page is silent (each is listed with its reason in the
 * design notes of the repository):
 *   - nibble order: the low nibble of byte j holds input 2j, the high nibble
 *     input 2j+1;
 *   - E2M1 is the OCP Microscaling E2M1 element type (bias 1, one subnormal
 *     value 0.5, no Inf/NaN);
 *   - E4M3 is the "FN" variant (max finite 448, NaN at 0x7F/0xFF, no Inf):
 *     the 448 in g = 448/amax is the largest finite E4M3FN value;
 *   - the product is summed in ascending k, accumulated in fp64;
 *   - the quantiser (used only to build pinned round-trip cases) rounds to
 *     nearest with ties to the even code and saturates, see quantize below.
 *
 * Parity status: every function here is pinned by the CPU test suite against
 * something other than itself (published code tables, exact rational brute
 * force, closed-form special cases, a library decoder); none is "parity
 * unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* ---- element decoders (closed forms of the two code types) -------------- */

/* OCP MX E2M1: sign s = bit 3, exponent e = bits 2..1, mantissa m = bit 0.
 * e == 0: subnormal 0.5*m.  e > 0: 2^(e-1) * (1 + m/2).  Code 0x8 is -0. */
EXPORT double nvfp4_oracle_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent 15 with mantissa 7 is NaN; there are no infinities.
 * e == 0: subnormal 2^-6 * m/8.  e > 0: 2^(e-7) * (1 + m/8). */
EXPORT double nvfp4_oracle_e4m3(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* bf16 bit pattern -> double (exact widening: bf16 is the top half of fp32) */
static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* code of weight (n, k): byte n*K/2 + k/2; even k -> low nibble, odd k -> high */
static int code_at(const uint8_t* wq, int64_t K, int64_t n, int64_t k) {
  uint8_t b = wq[n * (K / 2) + k / 2];
  return (k & 1) ? (b >> 4) : (b & 0xF);
}

/* scale byte of weight (n, k): block k/16 of row n */
static int scale_at(const uint8_t* ws, int64_t K, int64_t n, int64_t k) {
  return ws[n * (K / 16) + k / 16];
}

/* W[n,k] = e2m1 * e4m3 / g, evaluated in fp64 */
static double weight_at(const uint8_t* wq, const uint8_t* ws, double g, int64_t K, int64_t n,
                        int64_t k) {
  return nvfp4_oracle_e2m1(code_at(wq, K, n, k)) * nvfp4_oracle_e4m3(scale_at(ws, K, n, k)) / g;
}

/* ---- dequantisation ------------------------------------------------------ */

/* Full-precision dequantised matrix, fp64 [N][K]. */
EXPORT void nvfp4_oracle_dequant_f64(const uint8_t* wq, const uint8_t* ws, float g, int64_t N,
                                     int64_t K, double* w) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) w[n * K + k] = weight_at(wq, ws, (double)g, K, n, k);
}

/* Dequantised matrix rounded once to fp32 [N][K].  The product e2m1*e4m3 is
 * exact in fp64, so this is fp32(fp64(p/g)); for a quotient of two numbers
 * with at most 24 significant bits, rounding first to 53 bits and then to 24
 * gives the correctly rounded fp32 quotient (53 >= 2*24 + 2), i.e. it equals
 * IEEE fp32 division p/g. */
EXPORT void nvfp4_oracle_dequant_f32(const uint8_t* wq, const uint8_t* ws, float g, int64_t N,
                                     int64_t K, float* w) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) w[n * K + k] = (float)weight_at(wq, ws, (double)g, K, n, k);
}

/* ---- the matmul ---------------------------------------------------------- */

/* y[m,n] = sum_k x[m,k] * W[n,k] in fp64, ascending k; also the magnitude sum
 * a[m,n] = sum_k |x[m,k] * W[n,k]| that the accuracy bound is stated in.
 * x is bf16 bits [M][K] row-major; y and a are fp64 [M][N].  Rows n are
 * independent, so nthreads > 1 splits them across OpenMP threads without
 * changing any result. */
EXPORT void nvfp4_oracle_gemm(const uint8_t* wq, const uint8_t* ws, float g, const uint16_t* x,
                              int64_t M, int64_t N, int64_t K, double* y, double* a,
                              int nthreads) {
  const double gd = (double)g;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double t = bf16_to_double(x[m * K + k]) * weight_at(wq, ws, gd, K, n, k);
        acc += t;
        mag += fabs(t);
      }
      y[m * N + n] = acc;
      if (a) a[m * N + n] = mag;
    }
  }
  (void)nthreads;
}

/* The same sums for a chosen list of output rows only (rows[i] in [0, N)):
 * y and a are [M][nrows].  Used to check large shapes on sampled outputs. */
EXPORT void nvfp4_oracle_gemm_rows(const uint8_t* wq, const uint8_t* ws, float g,
                                   const uint16_t* x, int64_t M, int64_t K, const int64_t* rows,
                                   int64_t nrows, double* y, double* a) {
  const double gd = (double)g;
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t n = rows[i];
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double t = bf16_to_double(x[m * K + k]) * weight_at(wq, ws, gd, K, n, k);
        acc += t;
        mag += fabs(t);
      }
      y[m * nrows + i] = acc;
      if (a) a[m * nrows + i] = mag;
    }
  }
}

/* ---- gate/up + SwiGLU ---------------------------------------------------- */

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)), fp64 */
EXPORT double nvfp4_oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* y[m,n] = silu(gate[m,n]) * up[m,n], gate and up each the plain matmul above
 * with its own weights and global scale and the same x.  Also returns the two
 * pre-activations and their magnitude sums (any of them may be NULL). */
EXPORT void nvfp4_oracle_gate_up_swiglu(const uint8_t* wq_g, const uint8_t* ws_g, float g_g,
                                        const uint8_t* wq_u, const uint8_t* ws_u, float g_u,
                                        const uint16_t* x, int64_t M, int64_t N, int64_t K,
                                        double* y, double* gate, double* up, double* a_gate,
                                        double* a_up, int nthreads) {
  const double gg = (double)g_g, gu = (double)g_u;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double sg = 0.0, su = 0.0, mg = 0.0, mu = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double xv = bf16_to_double(x[m * K + k]);
        double tg = xv * weight_at(wq_g, ws_g, gg, K, n, k);
        double tu = xv * weight_at(wq_u, ws_u, gu, K, n, k);
        sg += tg;
        su += tu;
        mg += fabs(tg);
        mu += fabs(tu);
      }
      y[m * N + n] = nvfp4_oracle_silu(sg) * su;
      if (gate) gate[m * N + n] = sg;
      if (up) up[m * N + n] = su;
      if (a_gate) a_gate[m * N + n] = mg;
      if (a_up) a_up[m * N + n] = mu;
    }
  }
  (void)nthreads;
}

/* ---- the MLP block: h = bf16(silu(gate) * up), then the down projection -- */

/* The bf16 value nearest to v, ties to the even significand, as its bit
 * pattern (IEEE round-to-nearest-even into 1 sign, 8 exponent, 7 fraction
 * bits): normal results keep 8 significant bits, results below 2^-126 are
 * multiples of 2^-133 (subnormals), magnitudes that round beyond the largest
 * finite value (2 - 2^-7) * 2^127 give infinity, NaN gives 0x7FC0.  The MLP
 * hands h to the down projection in bf16, as a two-kernel pipeline would
 * (the activations of the matmul are bf16 by the "W4A16" format). */
EXPORT uint16_t nvfp4_oracle_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                                /* a = f * 2^e, f in [0.5, 1) */
  const int qe = (e - 1 >= -126) ? e - 8 : -133; /* exponent of one unit in the last place */
  const double r = nearbyint(ldexp(a, -qe));   /* exact scaling; ties to even */
  const double rv = ldexp(r, qe);
  if (rv > ldexp(255.0, 120)) return sign | 0x7F80; /* beyond (2 - 2^-7) * 2^127 */
  const float f = (float)rv;                   /* exact: at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

EXPORT void nvfp4_oracle_bf16_rne_array(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = nvfp4_oracle_bf16_rne(v[i]);
}

/* ---- quantiser (the encoding that produces the three tensors) ------------ */

/* Nearest E4M3FN code to a non-negative value, ties to the even code,
 * values above 448 saturate to 448 (code 0x7E).  Brute force over all finite
 * non-negative codes 0x00..0x7E, which are in increasing order of value. */
EXPORT int nvfp4_oracle_e4m3_encode(double t) {
  if (!(t > 0.0)) return 0;
  if (t >= 448.0) return 0x7E;
  int best = 0;
  double bestd = fabs(t - nvfp4_oracle_e4m3(0));
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(t - nvfp4_oracle_e4m3(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* Nearest E2M1 code to v, ties to the even code (mantissa bit 0), magnitudes
 * above 6 saturate to 6; the sign bit is the sign of v (so -0 can occur). */
EXPORT int nvfp4_oracle_e2m1_encode(double v) {
  int s = signbit(v) ? 8 : 0;
  double t = fabs(v);
  int best = 0;
  double bestd = t;
  for (int c = 1; c < 8; ++c) {
    double d = fabs(t - nvfp4_oracle_e2m1(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      best = c;
      bestd = d;
    }
  }
  return s | best;
}

/* Quantise fp32 W [N][K] (K % 16 == 0, K even) to NVFP4:
 *   amax = max |W|;  g = fp32(448 / amax)  (g = 1 when amax == 0);
 *   per row n, block j: S = e4m3(encode(max|W[n,16j..16j+15]| * g / 6));
 *   if S == 0 every code of the block is 0, else code = encode(W * g / S);
 *   byte = code(2i) | code(2i+1) << 4.
 * All arithmetic in fp64 in exactly this order. */
EXPORT void nvfp4_oracle_quantize(const float* w, int64_t N, int64_t K, uint8_t* wq, uint8_t* ws,
                                  float* g_out) {
  double amax = 0.0;
  for (int64_t i = 0; i < N * K; ++i) {
    double v = fabs((double)w[i]);
    if (v > amax) amax = v;
  }
  float g = (amax > 0.0) ? (float)(448.0 / amax) : 1.0f;
  const double gd = (double)g;
  *g_out = g;
  memset(wq, 0, (size_t)(N * K / 2));
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t j = 0; j < K / 16; ++j) {
      double bmax = 0.0;
      for (int64_t k = 16 * j; k < 16 * j + 16; ++k) {
        double v = fabs((double)w[n * K + k]);
        if (v > bmax) bmax = v;
      }
      int sc = nvfp4_oracle_e4m3_encode(bmax * gd / 6.0);
      ws[n * (K / 16) + j] = (uint8_t)sc;
      double S = nvfp4_oracle_e4m3(sc);
      for (int64_t k = 16 * j; k < 16 * j + 16; ++k) {
        int code = (S == 0.0) ? 0 : nvfp4_oracle_e2m1_encode((double)w[n * K + k] * gd / S);
        uint8_t* b = &wq[n * (K / 2) + k / 2];
        *b |= (uint8_t)((k & 1) ? (code << 4) : code);
      }
    }
  }
}

EXPORT int nvfp4_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
