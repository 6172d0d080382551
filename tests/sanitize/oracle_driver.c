/*
 * oracle_driver.c -- memory and undefined-behaviour exercise of the CPU
 * oracle (oracle/oracle.c) for the sanitizer run.  Every exported function
 * is called on buffers of exactly the size its contract states (so that an
 * access one element past an end is caught), over small shapes that include
 * the empty and one-element cases, every element type, epilogue and B
 * layout, and with invalid arguments.  Values are seeded bit patterns; the
 * arithmetic itself is pinned by the Python oracle tests.
 *
 *   oracle_driver
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(const uint16_t* A, const uint16_t* B, const uint16_t* bias, double* Y, int64_t M, int64_t N,
                int64_t K, int dtype, int epilogue, int b_col_major, double alpha, int nthreads);
int oracle_gemm_sampled(const uint16_t* A, const uint16_t* B, const uint16_t* bias, const int64_t* rows,
                        const int64_t* cols, int64_t count, double* y, int64_t M, int64_t N, int64_t K, int dtype,
                        int epilogue, int b_col_major, double alpha, int nthreads);
int oracle_act(const double* x, double* y, int64_t n, int epilogue);
int oracle_max_threads(int nthreads);
double oracle_f16_to_f64(uint16_t h);
double oracle_bf16_to_f64(uint16_t h);
double oracle_f32_to_f64(uint32_t w);
int oracle_round(const double* x, void* y, int64_t n, int dtype);
int oracle_vector_add(const void* A, const void* B, void* C, int64_t n, int dtype);
int oracle_softmax(const void* X, double* Y, int64_t rows, int64_t cols, int dtype, double alpha, int nthreads);
int oracle_attention_rows(const uint16_t* Q, const uint16_t* K, const uint16_t* V, double* O, int64_t B, int64_t H,
                          int64_t N, int64_t D, int dtype, int causal, double scale, const int64_t* rows,
                          int64_t nrows, int nthreads);
int oracle_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, double* O, int64_t B, int64_t H,
                     int64_t N, int64_t D, int dtype, int causal, double scale, int nthreads);

static int g_fail = 0;
static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void) { /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}

/* finite values of moderate size in either 16-bit format: sign, exponent
 * near the middle of the range, random fraction */
static uint16_t moderate16(int dtype) {
  const uint32_t r = next_u32();
  if (dtype == 0) return (uint16_t)((r & 0x8000u) | ((uint32_t)(13 + (r >> 16) % 4) << 10) | (r & 0x3ffu));
  return (uint16_t)((r & 0x8000u) | ((uint32_t)(125 + (r >> 16) % 4) << 7) | (r & 0x7fu));
}

/* an exact-size allocation (at least one byte, so an empty buffer is still a
 * distinct allocation whose first byte is out of bounds for its user) */
static void* buf(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static uint16_t* halves(int64_t n, int dtype) {
  uint16_t* p = buf((size_t)n * 2);
  for (int64_t i = 0; i < n; ++i) p[i] = moderate16(dtype);
  return p;
}

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                       \
    }                                                                   \
  } while (0)

static void gemm(void) {
  static const int64_t sizes[] = {0, 1, 3, 8, 17};
  for (int a = 0; a < 5; ++a)
    for (int b = 0; b < 5; ++b)
      for (int c = 0; c < 5; ++c)
        for (int dtype = 0; dtype <= 1; ++dtype)
          for (int epi = 0; epi <= 4; ++epi)
            for (int bcol = 0; bcol <= 1; ++bcol) {
              const int64_t M = sizes[a], N = sizes[b], K = sizes[c];
              uint16_t* A = halves(M * K, dtype);
              uint16_t* B = halves(K * N, dtype);
              uint16_t* bias = epi >= 1 && epi <= 3 ? halves(N, dtype) : NULL;
              double* Y = buf((size_t)(M * N) * sizeof(double));
              CHECK(oracle_gemm(A, B, bias, Y, M, N, K, dtype, epi, bcol, 0.5, 2) == 0);
              if (epi != 4 && M > 0 && N > 0) {
                const int64_t count = 5;
                int64_t* rows = buf(count * sizeof(int64_t));
                int64_t* cols = buf(count * sizeof(int64_t));
                double* y = buf(count * sizeof(double));
                for (int64_t s = 0; s < count; ++s) {
                  rows[s] = (int64_t)(next_u32() % (uint32_t)M);
                  cols[s] = (int64_t)(next_u32() % (uint32_t)N);
                }
                rows[0] = M - 1, cols[0] = N - 1;
                CHECK(oracle_gemm_sampled(A, B, bias, rows, cols, count, y, M, N, K, dtype, epi, bcol, 0.5, 2) == 0);
                for (int64_t s = 0; s < count; ++s) CHECK(memcmp(&y[s], &Y[rows[s] * N + cols[s]], sizeof(double)) == 0);
                rows[1] = M; /* out of range: rejected before any access */
                CHECK(oracle_gemm_sampled(A, B, bias, rows, cols, count, y, M, N, K, dtype, epi, bcol, 0.5, 2) == -1);
                free(rows);
                free(cols);
                free(y);
              }
              free(A);
              free(B);
              free(bias);
              free(Y);
            }
  uint16_t one = 0x3c00;
  double y;
  CHECK(oracle_gemm(&one, &one, NULL, &y, -1, 1, 1, 0, 0, 0, 1.0, 1) == -1);
  CHECK(oracle_gemm(&one, &one, NULL, &y, 1, 1, 1, 2, 0, 0, 1.0, 1) == -1);
  CHECK(oracle_gemm(&one, &one, NULL, &y, 1, 1, 1, 0, 5, 0, 1.0, 1) == -1);
  CHECK(oracle_gemm(&one, &one, NULL, &y, 1, 1, 1, 0, 0, 2, 1.0, 1) == -1);
  CHECK(oracle_gemm_sampled(&one, &one, NULL, NULL, NULL, 0, &y, 1, 1, 1, 0, 4, 0, 1.0, 1) == -1);
  CHECK(oracle_gemm_sampled(&one, &one, NULL, NULL, NULL, -1, &y, 1, 1, 1, 0, 0, 0, 1.0, 1) == -1);
  CHECK(oracle_max_threads(2) >= 1);
}

static void elementwise(void) {
  const int64_t n = 37;
  double* x = buf((size_t)n * sizeof(double));
  double* y = buf((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) x[i] = ((double)(int32_t)next_u32()) / (1 << 26);
  for (int epi = 0; epi <= 3; ++epi) CHECK(oracle_act(x, y, n, epi) == 0);
  CHECK(oracle_act(x, y, n, 4) == -1);
  CHECK(oracle_act(x, y, 0, 3) == 0);
  for (uint32_t h = 0; h < 65536; ++h) {
    (void)oracle_f16_to_f64((uint16_t)h);
    (void)oracle_bf16_to_f64((uint16_t)h);
    (void)oracle_f32_to_f64(h << 16 | h);
  }
  for (int dtype = 0; dtype <= 2; ++dtype) {
    const size_t es = dtype == 2 ? 4 : 2;
    for (int64_t m = 0; m <= 9; ++m) {
      void* r = buf((size_t)m * es);
      CHECK(oracle_round(x, r, m, dtype) == 0);
      void* A = buf((size_t)m * es);
      void* B = buf((size_t)m * es);
      void* C = buf((size_t)m * es);
      for (int64_t i = 0; i < m * (int64_t)es; ++i) {
        ((unsigned char*)A)[i] = (unsigned char)next_u32();
        ((unsigned char*)B)[i] = (unsigned char)next_u32();
      }
      CHECK(oracle_vector_add(A, B, C, m, dtype) == 0);
      CHECK(oracle_vector_add(A, B, A, m, dtype) == 0); /* in place */
      for (int64_t rows = 0; rows <= 3; ++rows) {
        void* X = buf((size_t)(rows * m) * es);
        for (int64_t i = 0; i < rows * m * (int64_t)es; ++i) ((unsigned char*)X)[i] = (unsigned char)next_u32();
        double* Y = buf((size_t)(rows * m) * sizeof(double));
        CHECK(oracle_softmax(X, Y, rows, m, dtype, 0.25, 2) == 0);
        free(X);
        free(Y);
      }
      free(r);
      free(A);
      free(B);
      free(C);
    }
  }
  CHECK(oracle_round(x, y, 1, 3) == -1);
  CHECK(oracle_vector_add(x, x, y, -1, 0) == -1);
  CHECK(oracle_softmax(x, y, -1, 1, 0, 1.0, 1) == -1);
  free(x);
  free(y);
}

static void attention(void) {
  static const int64_t Ns[] = {0, 1, 5, 16};
  static const int64_t Ds[] = {1, 8, 64};
  for (int ni = 0; ni < 4; ++ni)
    for (int di = 0; di < 3; ++di)
      for (int dtype = 0; dtype <= 1; ++dtype)
        for (int causal = 0; causal <= 1; ++causal) {
          const int64_t B = 2, H = 3, N = Ns[ni], D = Ds[di], total = B * H * N;
          uint16_t* Q = halves(total * D, dtype);
          uint16_t* K = halves(total * D, dtype);
          uint16_t* V = halves(total * D, dtype);
          double* O = buf((size_t)(total * D) * sizeof(double));
          CHECK(oracle_attention(Q, K, V, O, B, H, N, D, dtype, causal, 0.125, 2) == 0);
          if (total > 0) {
            int64_t rows[3] = {0, total - 1, total / 2};
            double* o = buf((size_t)(3 * D) * sizeof(double));
            CHECK(oracle_attention_rows(Q, K, V, o, B, H, N, D, dtype, causal, 0.125, rows, 3, 2) == 0);
            for (int t = 0; t < 3; ++t) CHECK(memcmp(o + t * D, O + rows[t] * D, (size_t)D * sizeof(double)) == 0);
            rows[2] = total;
            CHECK(oracle_attention_rows(Q, K, V, o, B, H, N, D, dtype, causal, 0.125, rows, 3, 2) == -1);
            free(o);
          }
          free(Q);
          free(K);
          free(V);
          free(O);
        }
  uint16_t h = 0x3c00;
  double o;
  CHECK(oracle_attention(&h, &h, &h, &o, 1, 1, 1, 0, 0, 0, 1.0, 1) == -1);
  CHECK(oracle_attention(&h, &h, &h, &o, 1, 1, 1, 1, 2, 0, 1.0, 1) == -1);
  CHECK(oracle_attention(&h, &h, &h, &o, 1, 1, 1, 1, 0, 3, 1.0, 1) == -1);
  CHECK(oracle_attention(&h, &h, &h, &o, -1, 1, 1, 1, 0, 0, 1.0, 1) == -1);
}

int main(void) {
  gemm();
  elementwise();
  attention();
  printf("oracle_driver: %s\n", g_fail ? "FAILED" : "ok");
  return g_fail;
}
