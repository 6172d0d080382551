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
 *
 * The vector addition and the standalone row softmax at the end of this file
 * also take dtype 2 = IEEE binary32.
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

/* =========================================================================
 * The tutorial's two bandwidth-bound kernels (TEST INFRASTRUCTURE ONLY):
 *   - vector addition C[i] = A[i] + B[i] ("Adicao de vetores: o 'Hello
 *     World' dos kernels", noticiai.com.br; the edgex.exchange page's
 *     opening paragraph on vector addition);
 *   - the standalone row-wise softmax Y = softmax(X) per row (noticiai.com.br,
 *     section "Softmax por linha e FlashAttention": row max, subtract,
 *     exponentiate, normalise).
 * Element types: 0 = binary16, 1 = bfloat16, 2 = binary32.
 * ========================================================================= */

#define OR_DTYPE_F32 2

/* binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
double oracle_f32_to_f64(uint32_t w) {
  int sign = (w >> 31) & 1;
  int e = (w >> 23) & 0xff;
  uint32_t f = w & 0x7fffff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -149); /* subnormal: f * 2^(1-127-23) */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 0x800000u), e - 150); /* (1.f) * 2^(e-127) */
  }
  return sign ? -v : v;
}

/* A binary format with P significand bits (hidden bit included), minimum
 * normal exponent EMIN, maximum exponent EMAX and exponent bias BIAS. */
typedef struct {
  int P, EMIN, EMAX, BIAS, FRAC_BITS, EXP_BITS;
} fmt_t;

static fmt_t fmt_of(int dtype) {
  fmt_t f16 = {11, -14, 15, 15, 10, 5}, bf16 = {8, -126, 127, 127, 7, 8}, f32 = {24, -126, 127, 127, 23, 8};
  return dtype == OR_DTYPE_F16 ? f16 : dtype == OR_DTYPE_BF16 ? bf16 : f32;
}

/* Round a finite or infinite fp64 value to the nearest representable value
 * of the format, ties to an even last significand bit, and return its bit
 * pattern.  The representable values around |x| are the integer multiples of
 * the quantum 2^(max(E, EMIN) - (P-1)), E = exponent of |x|'s leading bit;
 * |x| / quantum is exact in fp64, rint() rounds it to an integer with ties to
 * even (C99, default rounding mode), and a result of 2^(EMAX+1) or more is an
 * overflow to infinity. */
static uint32_t round_bits(double x, fmt_t F) {
  const uint32_t sign = signbit(x) ? 1u : 0u;
  const uint32_t exp_all = (1u << F.EXP_BITS) - 1;
  const int width = 1 + F.EXP_BITS + F.FRAC_BITS;
  uint32_t out;
  double a = fabs(x);
  if (isnan(x)) {
    out = (exp_all << F.FRAC_BITS) | (1u << (F.FRAC_BITS - 1));
  } else if (a == 0.0) {
    out = 0;
  } else {
    int ex;
    frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1): leading bit exponent ex - 1 */
    int E = ex - 1;
    if (E < F.EMIN) E = F.EMIN;
    const double quantum = ldexp(1.0, E - (F.P - 1));
    const double r = rint(a / quantum);
    const double v = r * quantum;
    if (isinf(a) || v >= ldexp(1.0, F.EMAX + 1)) {
      out = exp_all << F.FRAC_BITS;
    } else if (v == 0.0) {
      out = 0;
    } else {
      frexp(v, &ex);
      const int Ev = ex - 1;
      if (Ev < F.EMIN) { /* subnormal: exponent field 0, fraction = v / 2^(EMIN-(P-1)) */
        out = (uint32_t)(v / ldexp(1.0, F.EMIN - (F.P - 1)));
      } else {
        const uint32_t frac = (uint32_t)(v / ldexp(1.0, Ev - (F.P - 1)) - ldexp(1.0, F.P - 1));
        out = ((uint32_t)(Ev + F.BIAS) << F.FRAC_BITS) | frac;
      }
    }
  }
  return (sign << (width - 1)) | out;
}

static double decode_any(const void* p, int64_t i, int dtype) {
  if (dtype == OR_DTYPE_F32) return oracle_f32_to_f64(((const uint32_t*)p)[i]);
  return decode(((const uint16_t*)p)[i], dtype);
}

static void store_any(void* p, int64_t i, int dtype, uint32_t bits) {
  if (dtype == OR_DTYPE_F32)
    ((uint32_t*)p)[i] = bits;
  else
    ((uint16_t*)p)[i] = (uint16_t)bits;
}

/* y[i] = the dtype value nearest to x[i] (ties to even), as bit patterns
 * (uint16 for binary16 / bfloat16, uint32 for binary32). */
int oracle_round(const double* x, void* y, int64_t n, int dtype) {
  if (dtype < 0 || dtype > OR_DTYPE_F32 || n < 0) return -1;
  const fmt_t F = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i) store_any(y, i, dtype, round_bits(x[i], F));
  return 0;
}

/* C[i] = A[i] + B[i], correctly rounded to the element type.  The two
 * operands are decoded exactly and added in fp64; rounding that sum to the
 * element type gives the correctly rounded sum, because a first rounding to a
 * format with at least 2p + 2 significand bits (53 >= 2 * 24 + 2) cannot change
 * the final rounding of a sum to p bits (Figueroa, "When is double rounding
 * innocuous?", SIGNUM Newsletter 30(3), 1995). */
int oracle_vector_add(const void* A, const void* B, void* C, int64_t n, int dtype) {
  if (dtype < 0 || dtype > OR_DTYPE_F32 || n < 0) return -1;
  const fmt_t F = fmt_of(dtype);
  for (int64_t i = 0; i < n; ++i)
    store_any(C, i, dtype, round_bits(decode_any(A, i, dtype) + decode_any(B, i, dtype), F));
  return 0;
}

/* Y[r][c] = softmax over c of alpha * X[r][c], in fp64 (unrounded): the
 * inputs are decoded exactly, scaled, and each row goes through the same
 * max / exp / sum / divide steps as the GEMM epilogue's row softmax. */
int oracle_softmax(const void* X, double* Y, int64_t rows, int64_t cols, int dtype, double alpha, int nthreads) {
  if (dtype < 0 || dtype > OR_DTYPE_F32 || rows < 0 || cols < 0) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double* y = Y + r * cols;
    for (int64_t c = 0; c < cols; ++c) y[c] = alpha * decode_any(X, r * cols + c, dtype);
    softmax_row(y, cols);
  }
  return 0;
}

/* =========================================================================
 * Attention forward (TEST INFRASTRUCTURE ONLY): the exact result that the
 * tutorial's FlashAttention kernel computes tile by tile with an online
 * softmax ("TileLang: Criando Kernels ..." (noticiai.com.br), section
 * "Softmax por linha e FlashAttention"; the edgex.exchange page's paragraph
 * on the fused FlashAttention forward, causal and non-causal; spaxe.top,
 * FlashAttention paragraph).  The online rescaling there is an exact
 * reformulation, so the reference is the plain definition, written out:
 *
 *   for batch b, head h, query i (Q, K, V, O all [B][H][N][D] row-major):
 *     s_j  = scale * sum_d Q[b,h,i,d] K[b,h,j,d]     for j in J(i)
 *     J(i) = {0 .. N-1}, or {0 .. i} when causal (key j may not follow query i)
 *     p_j  = exp(s_j - max s) / sum_j' exp(s_j' - max s)
 *     O[b,h,i,d] = sum_{j in J(i)} p_j V[b,h,j,d]
 *
 * Inputs fp16 / bf16 (dtype 0 / 1) decoded exactly; every sum in fp64, in
 * index order; O returned in fp64, unrounded.  `rows` lists the flat query
 * rows r = (b*H + h)*N + i to compute; O receives nrows x D values.
 * ========================================================================= */
int oracle_attention_rows(const uint16_t* Q, const uint16_t* K, const uint16_t* V, double* O, int64_t B,
                          int64_t H, int64_t N, int64_t D, int dtype, int causal, double scale,
                          const int64_t* rows, int64_t nrows, int nthreads) {
  if (B < 0 || H < 0 || N < 0 || D < 1 || nrows < 0) return -1;
  if (dtype != OR_DTYPE_F16 && dtype != OR_DTYPE_BF16) return -1;
  if (causal != 0 && causal != 1) return -1;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= B * H * N) return -1;
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t bh = rows[t] / N, i = rows[t] % N;
    const uint16_t* q = Q + rows[t] * D;
    const uint16_t* k = K + bh * N * D;
    const uint16_t* v = V + bh * N * D;
    const int64_t nj = causal ? i + 1 : N;
    double* s = (double*)malloc((size_t)nj * sizeof(double));
    if (!s) {
      bad = 1;
      continue;
    }
    for (int64_t j = 0; j < nj; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += decode(q[d], dtype) * decode(k[j * D + d], dtype);
      s[j] = scale * acc;
    }
    softmax_row(s, nj);
    double* o = O + t * D;
    for (int64_t d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t j = 0; j < nj; ++j) acc += s[j] * decode(v[j * D + d], dtype);
      o[d] = acc;
    }
    free(s);
  }
  return bad ? -2 : 0;
}

/* Every query row: O is B x H x N x D. */
int oracle_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, double* O, int64_t B, int64_t H,
                     int64_t N, int64_t D, int dtype, int causal, double scale, int nthreads) {
  if (B < 0 || H < 0 || N < 0) return -1;
  const int64_t total = B * H * N;
  int64_t* rows = (int64_t*)malloc((size_t)(total > 0 ? total : 1) * sizeof(int64_t));
  if (!rows) return -2;
  for (int64_t r = 0; r < total; ++r) rows[r] = r;
  const int rc = oracle_attention_rows(Q, K, V, O, B, H, N, D, dtype, causal, scale, rows, total, nthreads);
  free(rows);
  return rc;
}
