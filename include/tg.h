/*
 * tg.h -- C ABI of the MI355X (gfx950) fused-epilogue tiled GEMM library.
 *
 *     C = epilogue(alpha * A.B + bias)
 *
 * The operation is the one the TileLang tutorial pages build up to:
 *   - "TileLang: Criando Kernels de GPU de Alto Desempenho com Tensor Cores,
 *     FlashAttention e Autotuning" (noticiai.com.br): section "GEMM com Tensor
 *     Cores" (tiled product on the matrix units), section "GEMM com epilogo
 *     fundido" (ReLU, bias and GELU applied to the accumulator inside the same
 *     kernel, no round trip to DRAM), section "Exploracao de schedules com
 *     autotuning" (a tile configuration chosen per matrix shape);
 *   - the edgex.exchange page on the TileLang Python DSL, paragraph on the
 *     fused epilogue (bias and GELU applied to the register-resident
 *     accumulator before the single write of the output);
 *   - "Designing High-Performance GPU Kernels with TileLang ..." (spaxe.top),
 *     paragraph on the row softmax applied in the GEMM epilogue without
 *     writing the intermediate product to global memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout   A is M x K row-major (K contiguous).  B is K x N row-major by
 *           default; with b_col_major = 1 it is stored N x K row-major (the
 *           "key" matrix of an attention-score product).  C is M x N
 *           row-major.  Leading dimensions are packed (lda = K, ldb = N or K,
 *           ldc = N).
 *  Types    TG_DTYPE_F16: A, B, bias and C are IEEE binary16.
 *           TG_DTYPE_BF16: A, B, bias and C are bfloat16.
 *           TG_EPI_SOFTMAX writes C as fp32 whatever the input dtype.
 *           Products are accumulated in fp32 on the matrix cores; the
 *           epilogue runs in fp32 and the result is rounded once, to nearest
 *           even, to the output type.
 *  Math     x_ij = alpha * sum_k A_ik B_kj + bias_j   (bias broadcast over rows)
 *           TG_EPI_NONE       C = x          (bias must be NULL)
 *           TG_EPI_BIAS       C = x
 *           TG_EPI_BIAS_RELU  C = max(x, 0)
 *           TG_EPI_BIAS_GELU  C = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))
 *           TG_EPI_SOFTMAX    C_ij = exp(x_ij - max_j x_ij) / sum_j exp(...)
 *                             (bias must be NULL; row length N <= TG_SOFTMAX_MAX_N)
 *  Memory   Every pointer is a device pointer owned by the caller.  The library
 *           never allocates or frees device memory (its one device array of
 *           its own, the workspace of tg_gemm_autotune_noalloc, comes with its
 *           device code, as a static variable); apart from the autotuners
 *           (tg_gemm_autotune and tg_gemm_autotune_noalloc, which time
 *           candidates and wait for them) it never synchronises and only
 *           enqueues one kernel on `stream` (a hipStream_t; NULL = the null
 *           stream).  Its mutable state is the autotune cache, guarded by a
 *           lock, so concurrent calls from several host threads are safe, and
 *           the workspace array of tg_gemm_autotune_noalloc (concurrent calls
 *           of that one entry point on one GPU race; see there).  C must not
 *           overlap A, B or bias.
 *  Errors   Every entry point returns a tg_status.  All argument checks run on
 *           the host before any HIP call, so an invalid call touches no device
 *           and enqueues nothing.  A launch failure reported by the runtime
 *           returns TG_ERR_HIP.  Faults during kernel execution surface at the
 *           caller's next synchronisation.  Nothing throws, aborts or prints
 *           (set TG_LOG=1 in the environment to log each launch to stderr).
 *  Limits   0 <= M < 2^31, 0 <= N <= 2^24, 0 <= K <= 2^20 (the kernels use
 *           32-bit offsets inside a tile); N and K multiples of 8 (16-byte
 *           rows); A, B, bias and C 16-byte aligned.  Negative sizes return
 *           TG_ERR_INVALID_ARG, larger sizes TG_ERR_UNSUPPORTED, alignment
 *           violations TG_ERR_MISALIGNED.
 *  Degenerate  M == 0 or N == 0: nothing is launched, TG_OK.
 *           K == 0: the product is zero and C = epilogue(bias).
 */
#ifndef TG_H_
#define TG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_VERSION_MAJOR 0
#define TG_VERSION_MINOR 1

/* Longest softmax row the on-chip row kernel holds (fp32 values per row). */
#define TG_SOFTMAX_MAX_N 2048

/* Longest row tg_row_softmax holds in registers, in bytes of X: 8192 fp16 /
 * bf16 elements or 4096 fp32 elements. */
#define TG_ROW_SOFTMAX_MAX_ROW_BYTES 16384

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, unknown enum, bad config id */
  TG_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels implement */
  TG_ERR_MISALIGNED = -3,  /* pointer not 16-byte aligned, or N / K not a multiple of 8 */
  TG_ERR_HIP = -4          /* the HIP runtime rejected the launch */
} tg_status;

/* Element types.  The GEMM entry points take TG_DTYPE_F16 and TG_DTYPE_BF16
 * only (TG_DTYPE_F32 there is TG_ERR_INVALID_ARG); the two bandwidth-bound
 * kernels at the end of this header also take TG_DTYPE_F32. */
typedef enum tg_dtype { TG_DTYPE_F16 = 0, TG_DTYPE_BF16 = 1, TG_DTYPE_F32 = 2 } tg_dtype;

typedef enum tg_epilogue {
  TG_EPI_NONE = 0,
  TG_EPI_BIAS = 1,
  TG_EPI_BIAS_RELU = 2,
  TG_EPI_BIAS_GELU = 3,
  TG_EPI_SOFTMAX = 4
} tg_epilogue;

/* Kernel families a tile configuration belongs to. */
typedef enum tg_kernel_kind {
  TG_KERNEL_GEMM = 0,        /* 2-D output tiles, elementwise epilogues */
  TG_KERNEL_GEMM_SOFTMAX = 1 /* full-row tiles, row softmax epilogue */
} tg_kernel_kind;

/*
 * One compiled tile configuration (read-only; describes a kernel variant).
 * bm x bn output tile per workgroup, bk-deep K steps, `stages` LDS buffers,
 * waves 64-lane wavefronts per workgroup: wave_m x wave_n of them tile the
 * output, or twice that when two wave groups split every K step, MFMA shape
 * mfma_m x mfma_n x mfma_k, group_m = tile rows per L2 raster band,
 * xcd_remap = 1 when workgroups are regrouped so each XCD owns a contiguous
 * block of tiles, lds_bytes = LDS per workgroup, b_col_major = the B layout
 * the variant is compiled for (-1: any).
 */
typedef struct tg_tile_config {
  int32_t id;
  int32_t kind;
  int32_t bm, bn, bk;
  int32_t stages;
  int32_t waves;
  int32_t mfma_m, mfma_n, mfma_k;
  int32_t wave_m, wave_n;
  int32_t group_m;
  int32_t xcd_remap;
  int32_t lds_bytes;
  int32_t b_col_major;
} tg_tile_config;

/* Full argument block of tg_gemm_ex.
 * config_id < 0 selects from the built-in table; config_id >= 0 forces that
 * compiled configuration (it must be of the right kind and, when its
 * b_col_major is 0 or 1, of that B layout, else TG_ERR_INVALID_ARG).  group_m > 0 overrides the raster band height (tile
 * rows), 0 keeps the chosen one; xcd_remap 0 / 1 turns the per-XCD tile
 * regrouping off / on, -1 keeps the chosen setting.  Both only affect which
 * workgroup computes which tile, never the result. */
typedef struct tg_gemm_args {
  const void* A;
  const void* B;
  const void* bias;
  void* C;
  int64_t M, N, K;
  int32_t dtype;
  int32_t epilogue;
  int32_t b_col_major;
  float alpha;
  int32_t config_id;
  int32_t group_m;
  int32_t xcd_remap;
} tg_gemm_args;

/*
 * tg_gemm -- C = epilogue(A.B + bias) with alpha = 1 and B row-major (K x N).
 * A: M x K, B: K x N, bias: N elements (required for TG_EPI_BIAS*, must be NULL
 * otherwise), C: M x N (fp32 for TG_EPI_SOFTMAX, else the input dtype).
 * stream: hipStream_t to enqueue on.  Returns TG_OK or an error code (above).
 */
int tg_gemm(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
            int dtype, int epilogue, void* stream);

/*
 * tg_gemm_ex -- the general form: adds alpha (scales the fp32 accumulator
 * before the bias), the B layout flag and an optional forced configuration.
 * The row-softmax workload (attention scores Q.K^T / sqrt(d)) is a call with
 * b_col_major = 1 and alpha = 1/sqrt(d).  args must not be NULL.
 */
int tg_gemm_ex(const tg_gemm_args* args, void* stream);

/*
 * tg_gemm_query_config -- the configuration tg_gemm / tg_gemm_ex would launch
 * for this problem (the same lookup, no launch, no HIP call).  Writes *out.
 * Returns TG_OK, TG_ERR_INVALID_ARG (NULL out, bad enums, negative sizes) or
 * TG_ERR_UNSUPPORTED (e.g. softmax row longer than TG_SOFTMAX_MAX_N).
 */
int tg_gemm_query_config(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, int b_col_major,
                         tg_tile_config* out);

/*
 * tg_vector_add -- C[i] = A[i] + B[i] for 0 <= i < n.
 *
 * The tutorial's first kernel ("TileLang: Criando Kernels de GPU de Alto
 * Desempenho ..." (noticiai.com.br), section "Adicao de vetores: o 'Hello
 * World' dos kernels"; the edgex.exchange page's opening paragraph on vector
 * addition).  It is bound by HBM bandwidth and serves as the bandwidth probe
 * that the fused epilogues are measured against.
 *
 *  dtype   TG_DTYPE_F16, TG_DTYPE_BF16 or TG_DTYPE_F32; A, B and C all of it.
 *          The sum is formed in fp32 and rounded once, to nearest even: for
 *          every dtype C[i] is the correctly rounded value of A[i] + B[i].
 *  Layout  three contiguous vectors of n elements, device memory owned by the
 *          caller, 16-byte aligned.  C may be A or B (in place) but must not
 *          partly overlap either.
 *  n       0 <= n <= 2^36 (no multiple required); n == 0 launches nothing.
 *  Errors  NULL pointer with n > 0, negative n or unknown dtype:
 *          TG_ERR_INVALID_ARG; n > 2^36: TG_ERR_UNSUPPORTED; misaligned
 *          pointer: TG_ERR_MISALIGNED; a rejected launch: TG_ERR_HIP.  One
 *          kernel is enqueued on `stream`.
 */
int tg_vector_add(const void* A, const void* B, void* C, int64_t n, int dtype, void* stream);

/*
 * tg_row_softmax -- the standalone row-wise softmax, Y = softmax(alpha X) per row:
 *
 *     m_r = max_c alpha X[r][c],   Y[r][c] = exp(alpha X[r][c] - m_r) / sum_c' exp(alpha X[r][c'] - m_r)
 *
 * ("TileLang: Criando Kernels ..." (noticiai.com.br), section "Softmax por
 * linha e FlashAttention": row max, subtract, exponentiate, sum, divide; the
 * same operation as TG_EPI_SOFTMAX without the product in front of it.)
 *
 *  dtype   of X: TG_DTYPE_F16, TG_DTYPE_BF16 or TG_DTYPE_F32.  Y is always
 *          fp32.  All arithmetic is fp32.
 *  Layout  X is rows x cols row-major, Y is rows x cols row-major fp32; device
 *          memory owned by the caller, 16-byte aligned, not overlapping.
 *  Limits  cols * sizeof(X element) <= TG_ROW_SOFTMAX_MAX_ROW_BYTES, else
 *          TG_ERR_UNSUPPORTED; rows < 2^31.  A row must be a whole number of
 *          16-byte pieces (cols a multiple of 8 for fp16 / bf16, of 4 for
 *          fp32), else TG_ERR_MISALIGNED.  rows == 0 or cols == 0 launches
 *          nothing.  A row whose entries are all -inf gives NaN, as the
 *          formula does.
 *  Errors  as tg_vector_add.  One kernel is enqueued on `stream`.
 */
int tg_row_softmax(const void* X, float* Y, int64_t rows, int64_t cols, int dtype, float alpha, void* stream);

/* Longest sequence tg_attention_fwd takes. */
#define TG_ATTN_MAX_SEQ (1 << 20)

/*
 * tg_attention_fwd -- FlashAttention forward.  For every batch b and head h:
 *
 *     O[b,h] = softmax(scale * Q[b,h] K[b,h]^T) V[b,h]     (softmax over keys)
 *
 * and, when causal = 1, key j is visible to query i only if j <= i.
 *
 * The tutorial's capstone kernel ("TileLang: Criando Kernels ..."
 * (noticiai.com.br), section "Softmax por linha e FlashAttention"; the
 * edgex.exchange page's FlashAttention paragraph, causal and non-causal; the
 * spaxe.top FlashAttention paragraph): tiles of queries, keys and values are
 * combined with an online softmax (running max, running sum, rescaling), the
 * score matrix never reaches memory, and both products run on the matrix
 * units.
 *
 *  dtype   TG_DTYPE_F16 or TG_DTYPE_BF16, for Q, K, V and O alike.  Scores
 *          and the softmax are fp32; the probabilities are rounded to dtype as
 *          the matrix units take them for the second product; O is
 *          accumulated in fp32 and rounded once, to nearest even.
 *  Layout  Q, K, V, O: [batch][heads][seq_len][head_dim] row-major, packed,
 *          device memory owned by the caller, 16-byte aligned.  O must not
 *          overlap Q, K or V.
 *  Limits  head_dim 64 or 128 (else TG_ERR_UNSUPPORTED); 0 <= seq_len <=
 *          TG_ATTN_MAX_SEQ; batch, heads >= 0 with batch * heads *
 *          ceil(seq_len / 128) < 2^31 (else TG_ERR_UNSUPPORTED).
 *  scale   finite (usually 1 / sqrt(head_dim)); NaN or infinite:
 *          TG_ERR_INVALID_ARG.
 *  Degenerate  batch, heads or seq_len zero: nothing is launched, TG_OK.
 *  Errors  negative sizes, unknown dtype, causal not 0 / 1, NULL pointers:
 *          TG_ERR_INVALID_ARG; misaligned pointers: TG_ERR_MISALIGNED; a
 *          rejected launch: TG_ERR_HIP.  One kernel is enqueued on `stream`.
 */
int tg_attention_fwd(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t heads,
                     int64_t seq_len, int64_t head_dim, int dtype, int causal, float scale, void* stream);

/*
 * Run-time autotuning: a per-shape search over the compiled tile
 * configurations with a cache keyed on the problem, as the pages' autotuner
 * ("TileLang: Criando Kernels ..." (noticiai.com.br), section "Exploracao de
 * schedules com autotuning": a search space over tile sizes and warp counts,
 * keyed on (M, N, K); candidates benchmarked, validated, the winner cached so
 * the cost is paid once; the edgex.exchange and spaxe.top autotuning
 * paragraphs).  Every candidate here is already compiled, so a search times
 * each variant that can run the problem -- for the 2-D tiled kernels with
 * raster band heights 1, 4, 8, 16 and the per-XCD regrouping off and on --
 * and keeps the fastest whose output matches the default choice's.
 *
 * The cache holds one entry per (dtype, b_col_major, kernel kind, M, N, K).
 * tg_gemm, tg_gemm_ex (config_id < 0) and tg_gemm_query_config consult it
 * before the built-in table.  It lives for the process; it can be saved to
 * and loaded from a text file.
 */
typedef struct tg_autotune_entry {
  int32_t dtype;          /* TG_DTYPE_F16 / TG_DTYPE_BF16 */
  int32_t b_col_major;
  int32_t kind;           /* TG_KERNEL_GEMM or TG_KERNEL_GEMM_SOFTMAX */
  int64_t M, N, K;
  tg_tile_config config;  /* the chosen variant, with its group_m / xcd_remap */
  float us;               /* its mean launch time when tuned (as saved, when loaded) */
  int32_t candidates;     /* candidates tried by the search (0 when loaded) */
  int32_t valid;          /* of those, ran and matched the reference */
} tg_autotune_entry;

/* Bytes of device workspace tg_gemm_autotune needs for an M x N output with
 * this epilogue (a copy of the reference output, 4 KiB of mismatch counters
 * and 256 bytes for two clock stamps).  TG_ERR_INVALID_ARG for a NULL bytes,
 * a negative size or an unknown epilogue; TG_ERR_UNSUPPORTED beyond the GEMM
 * limits (M >= 2^31 or N > 2^24). */
int tg_gemm_autotune_workspace_size(int64_t M, int64_t N, int epilogue, int64_t* bytes);

/*
 * tg_gemm_autotune -- search the configurations for the problem `args`
 * describes (its config_id, group_m and xcd_remap are ignored), store the
 * winner in the cache and describe it in *result.
 *
 * The candidates run on the caller's A, B, bias and C; on return C holds the
 * winner's result.  workspace: device memory of at least
 * tg_gemm_autotune_workspace_size bytes, 256-byte aligned, not overlapping
 * the operands; it receives the default choice's output, against which every
 * candidate's C is compared on the device element by element (|c - r| <=
 * 1e-2 + 1e-2 |r| for fp16 / bf16 outputs, 1e-4 + 1e-4 |r| for the fp32
 * softmax; non-finite values must agree).  Each valid candidate is timed over
 * `iters` launches (1 .. 1000) on `stream`, between two reads of the GPU's
 * constant 100 MHz clock that a one-thread kernel writes into the workspace
 * in stream order.  The call blocks until the search is done.
 * Returns TG_OK; the argument errors of tg_gemm_ex; TG_ERR_INVALID_ARG for
 * NULL args / result, iters out of range, an empty output (M or N zero) or a
 * missing / short workspace; TG_ERR_MISALIGNED for a misaligned workspace;
 * TG_ERR_UNSUPPORTED if no candidate ran and matched; TG_ERR_HIP on a runtime
 * failure.
 */
int tg_gemm_autotune(const tg_gemm_args* args, void* workspace, int64_t workspace_bytes, int iters,
                     tg_autotune_entry* result, void* stream);

/* Largest workspace tg_gemm_autotune_noalloc can use: 32 MiB + 8 KiB, i.e.
 * outputs up to 32 MiB (16 Mi fp16 / bf16 or 8 Mi fp32 values). */
#define TG_AUTOTUNE_NOALLOC_MAX_BYTES (32 * 1024 * 1024 + 8192)

/*
 * tg_gemm_autotune_noalloc -- tg_gemm_autotune for callers that cannot
 * allocate device memory (code under HIP graph capture rules, tight serving
 * loops, harnesses that forbid hipMalloc): the same search, with the
 * workspace taken from a fixed device array inside the library instead of
 * the caller.  It calls no hipMalloc, hipFree or other allocating routine.
 *
 *  Scratch  TG_AUTOTUNE_NOALLOC_MAX_BYTES of device memory per GPU the
 *           library runs on, held until the process ends.  Its device
 *           address on a GPU is looked up on the first call made with that
 *           GPU current.  Every call on one GPU shares that GPU's array and
 *           overwrites it; calls that overlap on one GPU (several host
 *           threads or streams at once) race and must not be made.
 *  Args     as tg_gemm_autotune without the workspace: args (its config_id,
 *           group_m and xcd_remap ignored), iters 1 .. 1000, result.
 *  Errors   the argument errors of tg_gemm_autotune; TG_ERR_UNSUPPORTED when
 *           the problem's workspace (tg_gemm_autotune_workspace_size)
 *           exceeds TG_AUTOTUNE_NOALLOC_MAX_BYTES or no candidate ran and
 *           matched; TG_ERR_HIP if the runtime cannot give the array's
 *           address or a launch / copy fails.
 */
int tg_gemm_autotune_noalloc(const tg_gemm_args* args, int iters, tg_autotune_entry* result, void* stream);

/* Number of cached entries; entry `index` (TG_ERR_INVALID_ARG if out of
 * range or out is NULL); forget every entry. */
int tg_autotune_cache_size(void);
int tg_autotune_cache_get(int index, tg_autotune_entry* out);
int tg_autotune_cache_clear(void);

/* Write the cache to a text file (first line "tg-autotune-cache 1", then one
 * line per entry: dtype b_col_major kind M N K id bm bn bk stages waves
 * group_m xcd_remap us).  TG_ERR_INVALID_ARG if path is NULL or the file
 * cannot be written. */
int tg_autotune_cache_save(const char* path);

/* Merge a file written by tg_autotune_cache_save into the cache.  An entry
 * whose configuration id does not describe the same variant in this library
 * (another build), or that names a problem the library rejects, is skipped.
 * *loaded / *skipped (either may be NULL) receive the counts.
 * TG_ERR_INVALID_ARG if path is NULL, the file cannot be read or its first
 * line is not the header. */
int tg_autotune_cache_load(const char* path, int* loaded, int* skipped);

/*
 * tg_clock_probe -- measurement aid (not part of any computation): the
 * shader clock under sustained matrix-unit load.  Launches `blocks`
 * workgroups of 256 threads that each run `iters` iterations of four
 * independent v_mfma_f32_16x16x32_f16 chains per wave on operands that change
 * every iteration (random fp16 values in +-[0.5, 1)), and writes for
 * workgroup b: out[2b] = shader-clock cycles (s_memtime) elapsed around the
 * loop, out[2b+1] = ticks of the constant 100 MHz counter (s_memrealtime).
 * clock = 100 MHz x out[2b] / out[2b+1].  The dense MFMA peak at that clock
 * is 256 CUs x 4096 FLOP/clk x clock; the published 2.5 PFLOP/s assumes
 * 2.4 GHz.
 *  out     device memory for 2 * blocks uint64 values, 16-byte aligned, owned
 *          by the caller.
 *  Errors  NULL out, blocks outside 1 .. 65536 or iters outside 1 .. 2^24:
 *          TG_ERR_INVALID_ARG; misaligned out: TG_ERR_MISALIGNED; a rejected
 *          launch: TG_ERR_HIP.  One kernel is enqueued on `stream`.
 */
int tg_clock_probe(unsigned long long* out, int blocks, int iters, void* stream);

/*
 * tg_layout_probe -- measurement aid (not part of any computation): runs the
 * register-level operations the kernels are built on, on known data, and
 * writes what every lane received, so that the layouts the kernels assume
 * can be checked against the hardware.  One wave, one kernel on `stream`.
 *  kind 0 / 1  v_mfma_f32_16x16x32_f16 / _bf16: for each A operand position
 *           p = 8 lane + element (0 .. 511) in turn, A is one-hot at p and B
 *           element (lane lb, element eb) holds a code of v = 8 lb + eb (v + 1
 *           for fp16; (16 + v % 16) * 2^(v / 16) for bf16, both exact);
 *           out = float[512][64][4]: the 4 accumulator registers of each lane.
 *  kind 2   ds_read_b64_tr_b16: LDS holds the 16-bit values 0 .. 2047, lane
 *           j reads at byte 8 j; out = uint32[64][4]: the 4 values each lane
 *           received.
 *  out      device memory owned by the caller (512 KiB for kinds 0 / 1,
 *           1 KiB for kind 2), 16-byte aligned.
 *  Errors   NULL out or unknown kind: TG_ERR_INVALID_ARG; misaligned out:
 *           TG_ERR_MISALIGNED; a rejected launch: TG_ERR_HIP.
 */
int tg_layout_probe(int kind, void* out, void* stream);

/* Number of compiled tile configurations (ids 0 .. n-1). */
int tg_num_configs(void);

/* Describe compiled configuration `index`; TG_ERR_INVALID_ARG if out of range
 * or out is NULL. */
int tg_get_config(int index, tg_tile_config* out);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* tg_status_string(int status);

/* Library version as major * 100 + minor. */
int tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TG_H_ */
