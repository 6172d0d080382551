/*
 * abi_driver.c -- host-side exercise of the library's C ABI for the CPU
 * sanitizer run (AddressSanitizer + UndefinedBehaviorSanitizer on the host
 * code only; the library is built host-only, without device code).
 *
 * Every call made here is one the ABI answers on the host, before any HIP
 * call: configuration queries over a grid of shapes and enum values
 * (including extreme sizes), every entry point with invalid arguments, empty
 * problems, and the autotune cache file parser on well-formed and malformed
 * files.  The expected status of each call follows include/tg.h; a mismatch
 * prints the call and exits 1.  A sanitizer finding aborts the process.
 *
 *   abi_driver <scratch directory>
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tg.h"

static int g_fail = 0;
static long g_calls = 0;

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    ++g_calls;                                                                          \
    if (got_ != (want)) {                                                               \
      fprintf(stderr, "%s:%d: %s returned %d, want %d\n", __FILE__, __LINE__, #call, got_, \
              (int)(want));                                                             \
      g_fail = 1;                                                                       \
    }                                                                                   \
  } while (0)

/* a non-NULL address that is 16-byte aligned, and one that is not; never
 * dereferenced: every call that takes them fails its checks first */
#define P16 ((void*)(uintptr_t)0x10000)
#define P1 ((void*)(uintptr_t)0x10001)

static const int64_t kSizes[] = {0,    1,     7,          8,          16,         64,        127,
                                 128,  1000,  2048,       2056,       4096,       8192,      1 << 20,
                                 1 << 24, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX, -1, INT64_MIN};
#define NSIZES ((int)(sizeof(kSizes) / sizeof(kSizes[0])))

static void configs(void) {
  const int n = tg_num_configs();
  if (n <= 0) {
    fprintf(stderr, "tg_num_configs() = %d\n", n);
    g_fail = 1;
  }
  tg_tile_config c;
  for (int i = -3; i < n + 3; ++i) EXPECT(tg_get_config(i, &c), (i >= 0 && i < n) ? TG_OK : TG_ERR_INVALID_ARG);
  EXPECT(tg_get_config(0, NULL), TG_ERR_INVALID_ARG);
  for (int s = -50; s <= 50; ++s) {
    const char* t = tg_status_string(s);
    if (!t || !t[0]) {
      fprintf(stderr, "tg_status_string(%d) is empty\n", s);
      g_fail = 1;
    }
  }
  (void)tg_version();
}

static void queries(void) {
  tg_tile_config c;
  for (int a = 0; a < NSIZES; ++a)
    for (int b = 0; b < NSIZES; ++b)
      for (int k = 0; k < NSIZES; ++k)
        for (int dtype = -1; dtype <= 3; ++dtype)
          for (int epi = -1; epi <= 6; ++epi)
            for (int bcol = -1; bcol <= 2; ++bcol) {
              const int64_t M = kSizes[a], N = kSizes[b], K = kSizes[k];
              const int rc = tg_gemm_query_config(M, N, K, dtype, epi, bcol, &c);
              ++g_calls;
              const int bad_enum = (dtype != TG_DTYPE_F16 && dtype != TG_DTYPE_BF16) || epi < TG_EPI_NONE ||
                                   epi > TG_EPI_SOFTMAX || (bcol != 0 && bcol != 1);
              if ((bad_enum || M < 0 || N < 0 || K < 0) && rc != TG_ERR_INVALID_ARG) {
                fprintf(stderr, "query %lld %lld %lld %d %d %d -> %d\n", (long long)M, (long long)N, (long long)K,
                        dtype, epi, bcol, rc);
                g_fail = 1;
              }
              if (rc == TG_OK && (c.bm <= 0 || c.bn <= 0 || c.bk <= 0)) {
                fprintf(stderr, "query %lld %lld %lld: empty configuration\n", (long long)M, (long long)N,
                        (long long)K);
                g_fail = 1;
              }
              EXPECT(tg_gemm_query_config(M, N, K, dtype, epi, bcol, NULL), TG_ERR_INVALID_ARG);
            }
}

static void launches(void) {
  /* invalid arguments: nothing reaches the runtime */
  EXPECT(tg_gemm(NULL, P16, NULL, P16, 64, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P16, P16, NULL, P16, -1, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P16, P16, NULL, P16, 64, 64, 64, TG_DTYPE_F32, TG_EPI_NONE, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P16, P16, NULL, P16, 64, 64, 64, TG_DTYPE_F16, 99, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P1, P16, NULL, P16, 64, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_ERR_MISALIGNED);
  EXPECT(tg_gemm(P16, P16, NULL, P16, 64, 60, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_ERR_MISALIGNED);
  EXPECT(tg_gemm(P16, P16, NULL, P16, (int64_t)1 << 40, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL),
         TG_ERR_UNSUPPORTED);
  EXPECT(tg_gemm(P16, P16, NULL, P16, INT64_MAX, INT64_MAX, INT64_MAX, TG_DTYPE_BF16, TG_EPI_BIAS_RELU, NULL),
         TG_ERR_UNSUPPORTED);
  EXPECT(tg_gemm(P16, P16, NULL, P16, 64, 64, 64, TG_DTYPE_F16, TG_EPI_BIAS_GELU, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P16, P16, P16, P16, 64, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm(P16, P16, NULL, P16, 64, 4096, 64, TG_DTYPE_F16, TG_EPI_SOFTMAX, NULL), TG_ERR_UNSUPPORTED);
  /* empty output: nothing launched */
  EXPECT(tg_gemm(NULL, NULL, NULL, NULL, 0, 64, 64, TG_DTYPE_F16, TG_EPI_NONE, NULL), TG_OK);
  EXPECT(tg_gemm(NULL, NULL, NULL, NULL, 64, 0, 64, TG_DTYPE_BF16, TG_EPI_NONE, NULL), TG_OK);

  EXPECT(tg_gemm_ex(NULL, NULL), TG_ERR_INVALID_ARG);
  tg_gemm_args a;
  memset(&a, 0, sizeof a);
  a.A = P16, a.B = P16, a.C = P16, a.M = 64, a.N = 64, a.K = 64, a.dtype = TG_DTYPE_F16, a.alpha = 1.0f;
  a.config_id = -1, a.xcd_remap = -1;
  const int n = tg_num_configs();
  for (int id = n; id < n + 4; ++id) {
    a.config_id = id;
    EXPECT(tg_gemm_ex(&a, NULL), TG_ERR_INVALID_ARG);
  }
  a.config_id = -1, a.group_m = -3;
  EXPECT(tg_gemm_ex(&a, NULL), TG_ERR_INVALID_ARG);
  a.group_m = 5000;
  EXPECT(tg_gemm_ex(&a, NULL), TG_ERR_INVALID_ARG);
  a.group_m = 0, a.xcd_remap = 5;
  EXPECT(tg_gemm_ex(&a, NULL), TG_ERR_INVALID_ARG);
  /* every forced configuration and raster, stopped by a misaligned C */
  a.xcd_remap = -1, a.C = P1;
  for (int id = -1; id < n; ++id)
    for (int gm = 0; gm <= 8; gm += 4)
      for (int x = -1; x <= 1; ++x)
        for (int epi = TG_EPI_NONE; epi <= TG_EPI_SOFTMAX; ++epi)
          for (int bcol = 0; bcol <= 1; ++bcol) {
            a.config_id = id, a.group_m = gm, a.xcd_remap = x, a.epilogue = epi, a.b_col_major = bcol;
            a.bias = (epi >= TG_EPI_BIAS && epi <= TG_EPI_BIAS_GELU) ? P16 : NULL;
            const int rc = tg_gemm_ex(&a, NULL);
            ++g_calls;
            if (rc != TG_ERR_MISALIGNED && rc != TG_ERR_INVALID_ARG && rc != TG_ERR_UNSUPPORTED) {
              fprintf(stderr, "gemm_ex id %d gm %d xcd %d epi %d bcol %d -> %d\n", id, gm, x, epi, bcol, rc);
              g_fail = 1;
            }
          }

  /* bandwidth kernels */
  for (int i = 0; i < NSIZES; ++i) {
    const int64_t s = kSizes[i];
    const int r1 = tg_vector_add(P1, P16, P16, s, TG_DTYPE_F32, NULL);
    const int want1 = s < 0 ? TG_ERR_INVALID_ARG : s > ((int64_t)1 << 36) ? TG_ERR_UNSUPPORTED
                      : s == 0                                             ? TG_OK
                                                                           : TG_ERR_MISALIGNED;
    EXPECT(r1, want1);
    for (int dt = -1; dt <= 3; ++dt) {
      const int rc = tg_row_softmax(P1, (float*)P16, 4, s, dt, 1.0f, NULL);
      ++g_calls;
      if (s < 0 || dt < 0 || dt > 2) {
        if (rc != TG_ERR_INVALID_ARG) {
          fprintf(stderr, "row_softmax cols=%lld dtype=%d -> %d\n", (long long)s, dt, rc);
          g_fail = 1;
        }
      } else if (rc == TG_OK && s != 0) {
        fprintf(stderr, "row_softmax cols=%lld dtype=%d accepted a misaligned X\n", (long long)s, dt);
        g_fail = 1;
      }
      EXPECT(tg_row_softmax(P1, (float*)P16, s, 8, TG_DTYPE_F16, 1.0f, NULL),
             s < 0 ? TG_ERR_INVALID_ARG : s >= ((int64_t)1 << 31) ? TG_ERR_UNSUPPORTED
             : s == 0                                             ? TG_OK
                                                                  : TG_ERR_MISALIGNED);
    }
  }
  EXPECT(tg_vector_add(NULL, P16, P16, 16, TG_DTYPE_F16, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_vector_add(P16, P16, P16, 16, 7, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_row_softmax(NULL, (float*)P16, 4, 8, TG_DTYPE_F16, 1.0f, NULL), TG_ERR_INVALID_ARG);

  /* attention */
  for (int i = 0; i < NSIZES; ++i)
    for (int j = 0; j < NSIZES; ++j) {
      const int64_t B = kSizes[i], N = kSizes[j];
      const int rc = tg_attention_fwd(P1, P16, P16, P16, B, 16, N, 128, TG_DTYPE_F16, 1, 0.1f, NULL);
      ++g_calls;
      if ((B < 0 || N < 0) ? rc != TG_ERR_INVALID_ARG : rc == TG_ERR_HIP) {
        fprintf(stderr, "attention B=%lld N=%lld -> %d\n", (long long)B, (long long)N, rc);
        g_fail = 1;
      }
      const int r2 = tg_attention_fwd(P1, P16, P16, P16, 3, B, N, 64, TG_DTYPE_BF16, 0, 0.1f, NULL);
      ++g_calls;
      if (r2 == TG_ERR_HIP) {
        fprintf(stderr, "attention H=%lld N=%lld reached the runtime\n", (long long)B, (long long)N);
        g_fail = 1;
      }
    }
  EXPECT(tg_attention_fwd(P16, P16, P16, P16, 1, 1, 128, 96, TG_DTYPE_F16, 0, 0.1f, NULL), TG_ERR_UNSUPPORTED);
  EXPECT(tg_attention_fwd(P16, P16, P16, P16, 1, 1, 128, 128, TG_DTYPE_F16, 2, 0.1f, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_attention_fwd(P16, P16, P16, P16, 1, 1, 128, 128, TG_DTYPE_F16, 0, NAN, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_attention_fwd(NULL, P16, P16, P16, 1, 1, 128, 128, TG_DTYPE_F16, 0, 0.1f, NULL), TG_ERR_INVALID_ARG);

  /* measurement aids */
  EXPECT(tg_clock_probe(NULL, 1, 1, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_clock_probe((unsigned long long*)P16, 0, 1, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_clock_probe((unsigned long long*)P1, 1, 1, NULL), TG_ERR_MISALIGNED);
  EXPECT(tg_layout_probe(3, P16, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_layout_probe(0, P1, NULL), TG_ERR_MISALIGNED);
}

static void autotune_args(void) {
  int64_t bytes = 0;
  for (int i = 0; i < NSIZES; ++i)
    for (int j = 0; j < NSIZES; ++j)
      for (int epi = -1; epi <= 6; ++epi) {
        const int64_t M = kSizes[i], N = kSizes[j];
        const int rc = tg_gemm_autotune_workspace_size(M, N, epi, &bytes);
        ++g_calls;
        if (rc == TG_OK && bytes <= 0) {
          fprintf(stderr, "workspace_size %lld %lld %d -> %lld bytes\n", (long long)M, (long long)N, epi,
                  (long long)bytes);
          g_fail = 1;
        }
        if ((M < 0 || N < 0 || epi < 0 || epi > TG_EPI_SOFTMAX) && rc != TG_ERR_INVALID_ARG) {
          fprintf(stderr, "workspace_size %lld %lld %d -> %d\n", (long long)M, (long long)N, epi, rc);
          g_fail = 1;
        }
      }
  EXPECT(tg_gemm_autotune_workspace_size(64, 64, TG_EPI_NONE, NULL), TG_ERR_INVALID_ARG);

  tg_gemm_args a;
  memset(&a, 0, sizeof a);
  a.A = P16, a.B = P16, a.C = P16, a.M = 64, a.N = 64, a.K = 64, a.dtype = TG_DTYPE_F16, a.alpha = 1.0f;
  a.config_id = -1, a.xcd_remap = -1;
  tg_autotune_entry r;
  EXPECT(tg_gemm_autotune(NULL, P16, 1 << 20, 5, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, NULL, 1 << 20, 5, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, P16, 100, 5, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, P16, 1 << 20, 0, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, P16, 1 << 20, 1001, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, P16, 1 << 20, 5, NULL, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune(&a, (void*)((uintptr_t)P16 + 16), 1 << 20, 5, &r, NULL), TG_ERR_MISALIGNED);
  EXPECT(tg_gemm_autotune_noalloc(NULL, 5, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune_noalloc(&a, 0, &r, NULL), TG_ERR_INVALID_ARG);
  EXPECT(tg_gemm_autotune_noalloc(&a, 5, NULL, NULL), TG_ERR_INVALID_ARG);
  a.M = 8192, a.N = 8192, a.K = 64;
  EXPECT(tg_gemm_autotune_noalloc(&a, 5, &r, NULL), TG_ERR_UNSUPPORTED);
  a.M = -5;
  EXPECT(tg_gemm_autotune_noalloc(&a, 5, &r, NULL), TG_ERR_INVALID_ARG);
}

static void write_file(const char* path, const char* text, size_t len) {
  FILE* f = fopen(path, "wb");
  if (!f) {
    perror(path);
    exit(2);
  }
  fwrite(text, 1, len, f);
  fclose(f);
}

static void cache_files(const char* dir) {
  char path[4096], path2[4096];
  snprintf(path, sizeof path, "%s/cache.txt", dir);
  snprintf(path2, sizeof path2, "%s/cache_saved.txt", dir);
  int loaded = -1, skipped = -1;
  tg_autotune_entry e;

  EXPECT(tg_autotune_cache_clear(), TG_OK);
  EXPECT(tg_autotune_cache_size(), 0);
  EXPECT(tg_autotune_cache_get(0, &e), TG_ERR_INVALID_ARG);
  EXPECT(tg_autotune_cache_get(-1, &e), TG_ERR_INVALID_ARG);
  EXPECT(tg_autotune_cache_load(NULL, &loaded, &skipped), TG_ERR_INVALID_ARG);
  EXPECT(tg_autotune_cache_save(NULL), TG_ERR_INVALID_ARG);
  snprintf(path2, sizeof path2, "%s/no/such/dir/x.txt", dir);
  EXPECT(tg_autotune_cache_load(path2, &loaded, &skipped), TG_ERR_INVALID_ARG);
  EXPECT(tg_autotune_cache_save(path2), TG_ERR_INVALID_ARG);
  snprintf(path2, sizeof path2, "%s/cache_saved.txt", dir);

  /* bad headers */
  write_file(path, "", 0);
  EXPECT(tg_autotune_cache_load(path, &loaded, &skipped), TG_ERR_INVALID_ARG);
  write_file(path, "tg-autotune-cache 2\n", 20);
  EXPECT(tg_autotune_cache_load(path, &loaded, &skipped), TG_ERR_INVALID_ARG);
  write_file(path, "\0\0\0\n", 4);
  EXPECT(tg_autotune_cache_load(path, &loaded, &skipped), TG_ERR_INVALID_ARG);

  /* one well-formed line per GEMM configuration that runs a 2048-wide row-major problem */
  char* text = malloc(1 << 20);
  size_t len = (size_t)snprintf(text, 64, "tg-autotune-cache 1\n");
  const int n = tg_num_configs();
  int good = 0;
  for (int id = 0; id < n; ++id) {
    tg_tile_config c;
    if (tg_get_config(id, &c) != TG_OK) continue;
    const int64_t N = c.kind == TG_KERNEL_GEMM_SOFTMAX ? c.bn : 2048;
    const int bcol = c.b_col_major < 0 ? 0 : c.b_col_major;
    len += (size_t)sprintf(text + len, "%d %d %d %d %lld %d %d %d %d %d %d %d 2 1 %d.5\n", TG_DTYPE_F16, bcol,
                           c.kind, 512 + 8 * id, (long long)N, 256, c.id, c.bm, c.bn, c.bk, c.stages, c.waves, id);
    ++good;
  }
  /* malformed or mismatching lines, each skipped */
  const char* bad[] = {
      "0 0 0 64 64 64\n",                                        /* too few fields */
      "0 0 0 64 64 64 0 1 2 3 4 5 6 7 x\n",                      /* not a number */
      "0 0 0 64 64 64 9999 128 128 64 4 8 2 1 1.0\n",            /* unknown id */
      "0 0 0 64 64 64 -5 128 128 64 4 8 2 1 1.0\n",              /* negative id */
      "0 0 0 -64 64 64 0 0 0 0 0 0 2 1 1.0\n",                   /* negative size, wrong variant */
      "0 0 0 99999999999999999999999 64 64 0 1 1 1 1 1 1 1 1\n", /* out of range */
      "7 0 0 64 64 64 0 1 1 1 1 1 1 1 nan\n",                    /* bad dtype */
      "\xff\xfe\xfd garbage \x01\x02\n",
      "# a comment line\n",
      "\n",
  };
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) len += (size_t)sprintf(text + len, "%s", bad[i]);
  /* a line far longer than any buffer, and a last line without a newline */
  for (int i = 0; i < 3000; ++i) text[len++] = (char)('0' + i % 10);
  text[len++] = '\n';
  len += (size_t)sprintf(text + len, "1 0 0 64 64 64 0 1 1 1 1 1 1 1 1.0");
  write_file(path, text, len);
  free(text);

  EXPECT(tg_autotune_cache_load(path, &loaded, &skipped), TG_OK);
  EXPECT(tg_autotune_cache_load(path, NULL, NULL), TG_OK);
  const int size = tg_autotune_cache_size();
  if (loaded <= 0 || size != loaded || loaded > good) {
    fprintf(stderr, "cache load: loaded %d skipped %d size %d (well-formed lines %d)\n", loaded, skipped, size,
            good);
    g_fail = 1;
  }
  for (int i = -2; i < size + 2; ++i) EXPECT(tg_autotune_cache_get(i, &e), (i >= 0 && i < size) ? TG_OK : TG_ERR_INVALID_ARG);
  EXPECT(tg_autotune_cache_get(0, NULL), TG_ERR_INVALID_ARG);
  /* the configuration lookup consults the cache */
  tg_tile_config c;
  for (int i = 0; i < size; ++i) {
    tg_autotune_entry x;
    if (tg_autotune_cache_get(i, &x) != TG_OK) continue;
    EXPECT(tg_gemm_query_config(x.M, x.N, x.K, x.dtype, x.kind == TG_KERNEL_GEMM_SOFTMAX ? TG_EPI_SOFTMAX
                                                                                         : TG_EPI_NONE,
                                x.b_col_major, &c),
           TG_OK);
  }
  /* save, clear, reload: the same entries */
  EXPECT(tg_autotune_cache_save(path2), TG_OK);
  EXPECT(tg_autotune_cache_clear(), TG_OK);
  EXPECT(tg_autotune_cache_load(path2, &loaded, &skipped), TG_OK);
  EXPECT(loaded, size);
  EXPECT(skipped, 0);
  EXPECT(tg_autotune_cache_clear(), TG_OK);
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <scratch directory>\n", argv[0]);
    return 2;
  }
  configs();
  queries();
  launches();
  autotune_args();
  cache_files(argv[1]);
  printf("abi_driver: %ld calls, %s\n", g_calls, g_fail ? "FAILED" : "ok");
  return g_fail;
}
