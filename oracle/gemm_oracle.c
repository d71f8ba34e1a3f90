/*
 * gemm_oracle.c -- plain, slow, fp64 host oracle for the tiled dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header or constant table with the HIP
 * library.
 *
 * What it computes (the plain definition, written out):
 *   C[i][j] = epi( sum_k A[i][k] * B[k][j] )   with A row-major M x K, B row-major
 *   K x N, C row-major M x N ("DeepGEMM" page, section 2.1: 2*M*N*K flops;
 *   SGEMM page, section 1.1: C = A x B, A is M x K, B is K x N; tutorial page,
 *   section 4.1: element [row][k] of A at row*K + k, [k][col] of B at k*N + col).
 *   16-bit inputs are widened before the multiply and all sums are kept wide
 *   (DeepGEMM page, section 3.4: FP16/BF16 in, FP32 accumulate). Here every
 *   product and sum is in double: a product of two bf16/fp16/fp32 values is
 *   exact in double, so the only rounding left is the fp64 summation.
 *   The epilogue (DeepGEMM page, section 1.2: activation, residual add and
 *   vector scale fused after the product) is applied in the order
 *     v = scale*acc;  v += bias[j];  v = GELU(v);  v += resid[i][j]
 *   with the exact GELU(v) = v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)).
 *
 * Alongside each reference value it returns s[i][j] = sum_k |A[i][k] B[k][j]|,
 * the scale the element-wise tolerance is measured against.
 *
 * Element codecs are the oracle's own: bf16 is the top half of an IEEE binary32;
 * fp16 is IEEE binary16 (1 sign, 5 exponent, 10 fraction bits, subnormals
 * included). Rounding to 16 bits is round-to-nearest, ties-to-even, applied
 * once from double.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC gemm_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_BIAS = 1u, OR_GELU = 2u, OR_RESID = 4u, OR_SCALE = 8u };

/* ---------------------------------------------------------------- codecs -- */

static double dec_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double dec_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double dec_one(int dtype, const void* p, int64_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)p)[idx];
    case OR_F16: return dec_f16(((const uint16_t*)p)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t*)p)[idx]);
  }
  return NAN;
}

/* Decode n elements of the given type to double. Returns 0, or -1 on a bad type. */
int oracle_decode(int dtype, const void* src, int64_t n, double* dst) {
  if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = dec_one(dtype, src, i);
  return 0;
}

/* Round a double to a binary format with p significand bits, minimum normal
 * exponent emin and maximum exponent emax; round to nearest, ties to even.
 * Returns the rounded value as a double (+-inf on overflow). */
static double round_fmt(double x, int p, int emin, int emax) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  double a = fabs(x);
  int E;
  frexp(a, &E);            /* a = f * 2^E with f in [0.5, 1): leading bit at 2^(E-1) */
  int lead = E - 1;
  if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
  int q = lead - (p - 1);  /* exponent of one unit in the last place */
  double n = nearbyint(ldexp(a, -q)); /* default mode: nearest, ties to even */
  double r = ldexp(n, q);
  if (r >= ldexp(1.0, emax + 1)) r = INFINITY;
  return x < 0 ? -r : r;
}

static uint16_t enc_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  double r = round_fmt(x, 8, -126, 127);
  float f = (float)r; /* exact: r is a bf16 value, hence a binary32 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static uint16_t enc_f16(double x) {
  if (isnan(x)) return 0x7e00;
  double r = round_fmt(x, 11, -14, 15);
  uint16_t s = signbit(r) ? 0x8000 : 0;
  double a = fabs(r);
  if (isinf(a)) return s | 0x7c00;
  if (a == 0.0) return s;
  if (a < ldexp(1.0, -14)) return s | (uint16_t)ldexp(a, 24); /* subnormal count */
  int E;
  frexp(a, &E);
  int e = E - 1; /* a in [2^e, 2^(e+1)) */
  uint16_t frac = (uint16_t)(ldexp(a, 10 - e) - 1024.0);
  return s | (uint16_t)((e + 15) << 10) | frac;
}

/* Round n doubles to bf16 or fp16 bit patterns (RNE). Returns 0, or -1. */
int oracle_round16(int dtype, const double* src, int64_t n, uint16_t* dst) {
  if (dtype != OR_F16 && dtype != OR_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = dtype == OR_BF16 ? enc_bf16(src[i]) : enc_f16(src[i]);
  return 0;
}

/* Spacing of the 16-bit format at |x| (one unit in the last place). */
double oracle_ulp16(int dtype, double x) {
  int p = dtype == OR_BF16 ? 8 : 11;
  int emin = dtype == OR_BF16 ? -126 : -14;
  double a = fabs(x);
  int E = 0;
  if (a > 0) frexp(a, &E);
  int lead = a > 0 ? E - 1 : emin;
  if (lead < emin) lead = emin;
  return ldexp(1.0, lead - (p - 1));
}

/* Vector form of oracle_ulp16 over n values. */
int oracle_ulp16_n(int dtype, const double* x, int64_t n, double* out) {
  if (dtype != OR_F16 && dtype != OR_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_ulp16(dtype, x[i]);
  return 0;
}

/* GELU(v) = v * Phi(v), Phi the standard normal CDF = (1 + erf(v/sqrt2)) / 2, evaluated
   as erfc(-v/sqrt2) / 2 (the same function: 1 + erf(x) = erfc(-x)), which keeps full
   relative accuracy in the negative tail where 1 + erf cancels. */
double oracle_gelu(double v) { return 0.5 * v * erfc(-v / sqrt(2.0)); }

static double epilogue(double acc, unsigned flags, double scale, const float* bias, int64_t j,
                       int resid_dtype, const void* resid, int64_t ij) {
  double v = acc;
  if (flags & OR_SCALE) v = scale * v;
  if (flags & OR_BIAS) v += (double)bias[j];
  if (flags & OR_GELU) v = oracle_gelu(v);
  if (flags & OR_RESID) v += dec_one(resid_dtype, resid, ij);
  return v;
}

static int check_args(int64_t M, int64_t N, int64_t K, int dtype, const void* A, const void* B,
                      unsigned flags, const float* bias, int resid_dtype, const void* resid) {
  if (M < 1 || N < 1 || K < 1) return -1;
  if (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16) return -2;
  if (!A || !B) return -3;
  if ((flags & OR_BIAS) && !bias) return -3;
  if (flags & OR_RESID) {
    if (!resid) return -3;
    if (resid_dtype != OR_F32 && resid_dtype != OR_F16 && resid_dtype != OR_BF16) return -2;
  }
  return 0;
}

/*
 * Full product. ref and abs_sum are M x N doubles (abs_sum may be NULL).
 * Loop order i-k-j over a row accumulator; k runs 0..K-1 in sequence.
 * nthreads <= 0 means "all OpenMP threads". Returns 0 or a negative code.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype, const void* A, const void* B,
                unsigned flags, double scale, const float* bias, int resid_dtype,
                const void* resid, double* ref, double* abs_sum, int nthreads) {
  int rc = check_args(M, N, K, dtype, A, B, flags, bias, resid_dtype, resid);
  if (rc) return rc;
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N));
  if (!Bd) return -4;
  oracle_decode(dtype, B, K * N, Bd);
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
  nthreads = 1;
#endif
  int fail = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)N);
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* arow = (double*)malloc(sizeof(double) * (size_t)K);
    if (!acc || !s || !arow) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k) arow[k] = dec_one(dtype, A, i * K + k);
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0, s[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double a = arow[k];
          const double* brow = Bd + k * N;
          for (int64_t j = 0; j < N; ++j) {
            const double p = a * brow[j];
            acc[j] += p;
            s[j] += fabs(p);
          }
        }
        for (int64_t j = 0; j < N; ++j) {
          ref[i * N + j] = epilogue(acc[j], flags, scale, bias, j, resid_dtype, resid, i * N + j);
          if (abs_sum) abs_sum[i * N + j] = s[j];
        }
      }
    }
    free(acc);
    free(s);
    free(arow);
  }
  free(Bd);
  return fail ? -4 : 0;
}

/*
 * Selected elements only: for t in [0, count) computes element (rows[t], cols[t])
 * of the same product, summing k = 0..K-1 in sequence. For spot checks of
 * products too large for the full loop.
 */
int oracle_gemm_at(int64_t M, int64_t N, int64_t K, int dtype, const void* A, const void* B,
                   unsigned flags, double scale, const float* bias, int resid_dtype,
                   const void* resid, int64_t count, const int64_t* rows, const int64_t* cols,
                   double* ref, double* abs_sum) {
  int rc = check_args(M, N, K, dtype, A, B, flags, bias, resid_dtype, resid);
  if (rc) return rc;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double acc = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = dec_one(dtype, A, i * K + k) * dec_one(dtype, B, k * N + j);
      acc += p;
      s += fabs(p);
    }
    ref[t] = epilogue(acc, flags, scale, bias, j, resid_dtype, resid, i * N + j);
    if (abs_sum) abs_sum[t] = s;
  }
  return 0;
}

/*
 * FP16 accumulation (DeepGEMM page, section 3.4: the variant it warns against,
 * "run one version accumulating in FP16 and one in FP32 on the same random
 * inputs and compare the maximum absolute error"). fp16 A and B, no epilogue:
 * for each element the accumulator is an fp16 value, and each k in sequence
 * replaces it by RNE16(acc + a*b), the sum formed exactly and rounded once (a
 * fused multiply-add in fp16). acc + a*b is formed in double, which is exact
 * when it fits 53 bits: always for inputs that are multiples of 2^-10 in
 * [-1, 1] (every quantity is then a multiple of 2^-20 below 2^16). ref receives
 * the final accumulators (fp16 values, as doubles).
 */
int oracle_gemm_f16acc(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                       double* ref) {
  if (M < 1 || N < 1 || K < 1 || !A || !B || !ref) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc = round_fmt(acc + dec_one(OR_F16, A, i * K + k) * dec_one(OR_F16, B, k * N + j), 11,
                        -14, 15);
      ref[i * N + j] = acc;
    }
  return 0;
}

/*
 * Row softmax (tutorial page, section 2: attention is Q K^T, a softmax over each
 * row of scores, then the product with V): for each row r of the fp32 matrix S
 * (rows x cols, row stride ld),
 *   P[r][c] = exp(scale*S[r][c] - m) / sum_c' exp(scale*S[r][c'] - m),
 *   m = max_c scale*S[r][c],
 * everything in double (subtracting m changes nothing mathematically and keeps
 * exp from overflowing). ref receives rows x cols doubles.
 */
int oracle_softmax_rows(int64_t rows, int64_t cols, const float* S, int64_t ld, double scale,
                        double* ref) {
  if (rows < 1 || cols < 1 || ld < cols || !S || !ref) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < rows; ++r) {
    const float* x = S + r * ld;
    double m = -INFINITY;
    for (int64_t c = 0; c < cols; ++c) m = fmax(m, scale * (double)x[c]);
    double sum = 0.0;
    for (int64_t c = 0; c < cols; ++c) sum += exp(scale * (double)x[c] - m);
    for (int64_t c = 0; c < cols; ++c) ref[r * cols + c] = exp(scale * (double)x[c] - m) / sum;
  }
  return 0;
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
