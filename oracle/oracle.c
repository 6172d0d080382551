/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for the fused-epilogue
 * matrix multiply
 *
 *     Y = epilogue(alpha * A.B + bias)
 *
 * that the TileLang tutorial pages build as their centre piece:
 *   - "TileLang: Criando Kernels de GPU de Alto Desempenho com Tensor Cores,
 *     FlashAttention e Autotuning" (noticiai.com.br), sections
 *     "GEMM com Tensor Cores" (the product A.B), "GEMM com epilogo fundido"
 *     (bias, ReLU and GELU applied to the accumulator) and
 *     "Softmax por linha e FlashAttention" (row max, subtract, exponentiate,
 *     normalise);
 *   - the edgex.exchange Italian page on the TileLang Python DSL, paragraph on
 *     the fused epilogue (bias addition and GELU folded into the
 *     register-resident accumulator, plus a row softmax);
 *   - "Designing High-Performance GPU Kernels with TileLang: Tensor-Core GEMM,
 *     Fused Softmax, FlashAttention, and Autotuning" (spaxe.top), paragraph on
 *     the row-wise softmax applied in the GEMM epilogue.
 *
 * Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant with the
 * GPU library: it has its own decoders, its own enum values and its own
 * epilogue formulas.
 *
 * Arithmetic: every fp16/bf16 input is decoded exactly to fp64 (both formats
 * embed in binary64 without loss).  The sum over k runs in the order
 * k = 0, 1, ..., K-1 with one fp64 accumulator per output; the epilogue is
 * evaluated in fp64 from C99 <math.h> (erf, exp).  The result is returned in
 * fp64, unrounded.  Nothing is blocked, fused or reordered.
 *
 * Enumerations (the oracle's own):
 *   dtype:     0 = IEEE binary16 ("fp16"), 1 = bfloat16
 *   epilogue:  0 = none, 1 = bias, 2 = bias + ReLU, 3 = bias + GELU (erf form),
 *              4 = row softmax
 *   b_col_major: 0 = B is K x N row-major; 1 = B is stored N x K row-major
 *                (i.e. K x N column-major), element (k, n) at n*K + k.
 * bias may be NULL (treated as zero) for every epilogue.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_DTYPE_F16 0
#define OR_DTYPE_BF16 1

#define OR_EPI_NONE 0
#define OR_EPI_BIAS 1
#define OR_EPI_RELU 2
#define OR_EPI_GELU 3
#define OR_EPI_SOFTMAX 4

/* ---- exact decoders (IEEE 754 binary16 and the bfloat16 truncation of
 * binary32), written from the format definitions ---------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^(1-15-10) */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 1024), e - 25); /* (1.f) * 2^(e-15), as an integer * 2^(e-25) */
  }
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int f = h & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* subnormal: f * 2^(1-127-7) */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 128), e - 134); /* (1.f) * 2^(e-127) */
  }
  return sign ? -v : v;
}

static double decode(uint16_t h, int dtype) {
  return dtype == OR_DTYPE_BF16 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

/* ---- epilogue functions, fp64 ---------------------------------------------- */

/* GELU in its defining form x * Phi(x) with Phi the standard normal CDF,
 * Phi(x) = (1 + erf(x / sqrt 2)) / 2. */
static double gelu_erf(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

static double relu(double x) { return x > 0.0 ? x : 0.0; }

/* Elementwise activation used by epilogues 0..3 (softmax is row-wise). */
static double act(double x, int epilogue) {
  switch (epilogue) {
    case OR_EPI_RELU: return relu(x);
    case OR_EPI_GELU: return gelu_erf(x);
    default: return x;
  }
}

/* Exported for the oracle's own tests: y[i] = act(x[i]). Returns -1 for the
 * row-wise softmax, which is not elementwise. */
int oracle_act(const double* x, double* y, int64_t n, int epilogue) {
  if (epilogue < 0 || epilogue > OR_EPI_GELU) return -1;
  for (int64_t i = 0; i < n; ++i) y[i] = act(x[i], epilogue);
  return 0;
}

/* Row softmax of one row of length n in place: m = max, e = exp(x - m),
 * y = e / sum(e). */
static void softmax_row(double* row, int64_t n) {
  if (n <= 0) return;
  double m = row[0];
  for (int64_t j = 1; j < n; ++j)
    if (row[j] > m) m = row[j];
  double s = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    row[j] = exp(row[j] - m);
    s += row[j];
  }
  for (int64_t j = 0; j < n; ++j) row[j] = row[j] / s;
}

static int check_args(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (dtype != OR_DTYPE_F16 && dtype != OR_DTYPE_BF16) return -1;
  if (epilogue < OR_EPI_NONE || epilogue > OR_EPI_SOFTMAX) return -1;
  if (b_col_major != 0 && b_col_major != 1) return -1;
  return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* Index of B's element (k, n). */
static int64_t b_index(int64_t k, int64_t n, int64_t N, int64_t K, int b_col_major) {
  return b_col_major ? n * K + k : k * N + n;
}

/*
 * Full product.  A: M*K halves (row-major), B: K*N halves (layout per
 * b_col_major), bias: N halves or NULL, Y: M*N doubles (row-major, written).
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_gemm(const uint16_t* A, const uint16_t* B, const uint16_t* bias, double* Y, int64_t M,
                int64_t N, int64_t K, int dtype, int epilogue, int b_col_major, double alpha,
                int nthreads) {
  if (check_args(M, N, K, dtype, epilogue, b_col_major)) return -1;
  if (M == 0 || N == 0) return 0;
  set_threads(nthreads);

  /* Decode B once into a k-contiguous copy bt[n][k]: a change of storage only;
   * every dot product below still sums k = 0..K-1 in order. */
  double* bt = (double*)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
  double* bv = (double*)malloc(sizeof(double) * (size_t)N);
  if (!bt || !bv) {
    free(bt);
    free(bv);
    return -1;
  }
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) bt[n * K + k] = decode(B[b_index(k, n, N, K, b_col_major)], dtype);
    bv[n] = bias ? decode(bias[n], dtype) : 0.0;
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    double* arow = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    for (int64_t k = 0; k < K; ++k) arow[k] = decode(A[i * K + k], dtype);
    double* yrow = Y + i * N;
    for (int64_t n = 0; n < N; ++n) {
      const double* b = bt + n * K;
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += arow[k] * b[k];
      double x = alpha * acc + bv[n];
      yrow[n] = (epilogue == OR_EPI_SOFTMAX) ? x : act(x, epilogue);
    }
    if (epilogue == OR_EPI_SOFTMAX) softmax_row(yrow, N);
    free(arow);
  }
  free(bt);
  free(bv);
  return 0;
}

/*
 * Sampled mode: y[s] = Y[rows[s], cols[s]] for s < count, each computed as its
 * own dot product exactly as oracle_gemm does (same decode, same k order, same
 * epilogue), so it equals the full product at those positions bit for bit.
 * The row softmax needs whole rows and is rejected (-1).
 */
int oracle_gemm_sampled(const uint16_t* A, const uint16_t* B, const uint16_t* bias,
                        const int64_t* rows, const int64_t* cols, int64_t count, double* y,
                        int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major,
                        double alpha, int nthreads) {
  if (check_args(M, N, K, dtype, epilogue, b_col_major)) return -1;
  if (epilogue == OR_EPI_SOFTMAX || count < 0) return -1;
  for (int64_t s = 0; s < count; ++s)
    if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < count; ++s) {
    int64_t i = rows[s], n = cols[s];
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
      acc += decode(A[i * K + k], dtype) * decode(B[b_index(k, n, N, K, b_col_major)], dtype);
    double x = alpha * acc + (bias ? decode(bias[n], dtype) : 0.0);
    y[s] = act(x, epilogue);
  }
  return 0;
}

/* Number of threads an OpenMP parallel region in this library would use. */
int oracle_max_threads(int nthreads) {
  set_threads(nthreads);
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
