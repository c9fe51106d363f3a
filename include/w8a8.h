/*
 * w8a8.h -- C ABI of the MI355X (gfx950) W8A8 INT8 Linear library.
 *
 * The operation (from "TurboDiffusion Integration Notes", TurboT2AV
 * docs/acceleration.md):
 *   - section "Reused Components", W8A8 Linear bullet: weights are quantised
 *     to INT8 once, when the model is initialised; activations are quantised
 *     dynamically right before every transformer Linear; shapes the INT8 path
 *     does not cover run on a retained BF16 weight with the native Linear;
 *   - section "Reused Components", FastNorm bullet: RMSNorm is replaced by a
 *     fused implementation (here: fused in front of the activation quant);
 *   - section "Differences From TurboDiffusion", W8A8-kernel row and the
 *     paragraph under the table: the post-scale kernel keeps one integer
 *     accumulation running across all of K and applies the activation and
 *     weight scales in the epilogue; the original kernel was blockwise-scaled.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer, owned by the caller. The library
 *     keeps no state between calls, never synchronises and allocates nothing:
 *     scratch memory (the split-K workspace of w8a8_gemm_postscale_ex) is the
 *     caller's. What a call does is fixed by its arguments and the device.
 *   - Row-major layouts; leading dimensions (ld*) are in ELEMENTS.
 *   - BF16 values travel as their 16-bit patterns (uint16_t).
 *   - `stream` is a hipStream_t passed as an opaque pointer (NULL = the
 *     legacy null stream). Work is enqueued on it; the call returns before it
 *     runs.
 *   - Arguments are validated on the host before anything is enqueued. On any
 *     status other than W8A8_OK nothing was launched and no output was
 *     written; w8a8_last_error() then describes the problem.
 *   - Inputs are assumed finite (NaN/Inf give unspecified codes). Outputs
 *     must not overlap inputs. Calls are thread-safe.
 *   - A call with zero rows (rows == 0 or M == 0) is valid and does nothing;
 *     its pointers may then be NULL (the other arguments are still checked).
 *
 * Quantisation readings (the pages leave the formula open):
 *   scale = fl32(absmax / 127) over the group; code = round-half-even(
 *   fl32(x / scale)) clamped to [-127, 127]; an all-zero group has scale 0
 *   and codes 0. Scales are fp32.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8A8_OK = 0,
  /* null pointer, negative size, ld smaller than the row, overlapping
     output, non-finite or negative eps */
  W8A8_ERR_INVALID_ARGUMENT = 1,
  /* a shape or alignment the INT8 kernels do not cover: the caller should
     fall back to its BF16 Linear ("Reused Components", W8A8 Linear bullet) */
  W8A8_ERR_UNSUPPORTED_SHAPE = 2,
  /* the HIP runtime reported an error while launching */
  W8A8_ERR_HIP = 3
} w8a8_status_t;

/* Largest K for which 127*127*K fits an INT32 accumulator, rounded down to a
   multiple of 128. */
#define W8A8_MAX_K 133120

/*
 * w8a8_quant_rows -- symmetric absmax INT8 quantisation of a BF16 matrix.
 *
 * Passage: "Reused Components", W8A8 Linear bullet (activations quantised
 * dynamically before each Linear; weights quantised once at initialisation);
 * the (1,128) and (128,128) groups are the blockwise scheme of the original
 * TurboDiffusion kernel ("Differences From TurboDiffusion", W8A8 kernel row).
 *
 *   x      [rows, cols] BF16, row stride ldx            (input)
 *   q      [rows, cols] int8, row stride ldq            (output)
 *   scale  fp32 [ceil(rows/group_rows), cols/group_cols], dense row-major
 *                                                        (output)
 * Supported groups:
 *   (1, cols)   one scale per row: per-token activations, or per-output-
 *               channel weights when x is the [N, K] weight;
 *   (1, 128)    per token per 128-wide K block (blockwise activations);
 *   (128, 128)  per 128x128 block (blockwise weights); the last row group
 *               may be ragged.
 * Requirements (else W8A8_ERR_UNSUPPORTED_SHAPE): cols % 8 == 0, and
 * cols % 128 == 0 for the 128-wide groups; x and q 16-byte aligned; ldx % 8
 * == 0 and ldq % 8 == 0; scale 4-byte aligned.
 */
w8a8_status_t w8a8_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                              int64_t group_rows, int64_t group_cols,
                              int8_t* q, int64_t ldq, float* scale, void* stream);

/*
 * w8a8_rmsnorm_quant -- RMSNorm prologue fused with per-token quantisation.
 *
 * Passage: "Reused Components", FastNorm bullet (fused RMSNorm) composed with
 * the W8A8 Linear bullet's dynamic activation quantisation.
 *
 *   r[m]  = fl32(1 / sqrt(mean_k x[m,k]^2 + eps))   (the sum of squares in fp32,
 *           pairwise; r is within (ceil(log2 cols) + 4) * 2^-24 * r of the
 *           correctly rounded value)
 *   y     = bf16(fl32(fl32(x * r) * gamma[k]))       (never leaves the chip)
 *   q, scale = per-token quantisation of y, as w8a8_quant_rows (1, cols).
 *
 *   x       [rows, cols] BF16, stride ldx  (input)
 *   gamma   [cols] BF16                    (input)
 *   q       [rows, cols] int8, stride ldq  (output)
 *   scale   [rows] fp32                    (output)
 *   inv_rms [rows] fp32 r, or NULL         (optional output)
 * Requirements as w8a8_quant_rows with group (1, cols); gamma 16-byte aligned;
 * eps finite and >= 0 (else W8A8_ERR_INVALID_ARGUMENT). An all-zero row with
 * eps = 0 has r = inf and is outside the contract.
 */
w8a8_status_t w8a8_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps,
                                 int64_t rows, int64_t cols, int64_t ldx,
                                 int8_t* q, int64_t ldq, float* scale, float* inv_rms,
                                 void* stream);

/*
 * w8a8_layernorm_quant -- LayerNorm with an optional affine step and an
 * optional adaLN modulation, fused with per-token quantisation.
 *
 * Passage: "Turbodiffusion Video", "Custom Kernel Optimizations" (a LayerNorm
 * takes the row's mean and variance, normalises, then applies the affine
 * step) and "TurboDiffusion Integration Notes", FastNorm bullet (the norms and
 * the LTX modulation helpers are fused), composed with the W8A8 Linear
 * bullet's dynamic activation quantisation.
 *
 *   mu[m]  = mean_k x[m,k],  var[m] = mean_k (x[m,k] - mu[m])^2 (divided by cols)
 *   r[m]   = fl32(1 / sqrt(var[m] + eps))
 *            (both sums in fp32, pairwise; mu and r are within about
 *            (ceil(log2 cols) + 4) * 2^-24 of the correctly rounded values,
 *            relative to mean |x| and to r)
 *   y      = bf16(fl32(fl32(fl32(fl32(x - mu) * r) * gamma[k]) + beta[k]))
 *   z      = bf16(fl32(bf16(fl32(y * m[k])) + shift[k])),  m = bf16(fl32(1 + scale[k]))
 *   q, out_scale = per-token quantisation of z, as w8a8_quant_rows (1, cols).
 *
 *   x         [rows, cols] BF16, stride ldx  (input)
 *   gamma     [cols] BF16 or NULL            (optional input; NULL leaves the step out)
 *   beta      [cols] BF16 or NULL            (optional input)
 *   mod_scale [cols] BF16 or NULL            (optional input: one sample's modulation;
 *                                             a batch of samples is one call per sample)
 *   mod_shift [cols] BF16 or NULL            (optional input)
 *   q         [rows, cols] int8, stride ldq  (output)
 *   out_scale [rows] fp32                    (output)
 *   mean      [rows] fp32 mu, or NULL        (optional output)
 *   rstd      [rows] fp32 r, or NULL         (optional output)
 * Requirements as w8a8_rmsnorm_quant (every vector input 16-byte aligned),
 * with cols <= 8192 (else W8A8_ERR_UNSUPPORTED_SHAPE). A row of zero variance
 * with eps = 0 has r = inf and is outside the contract.
 */
w8a8_status_t w8a8_layernorm_quant(const uint16_t* x, const uint16_t* gamma,
                                   const uint16_t* beta, const uint16_t* mod_scale,
                                   const uint16_t* mod_shift, float eps,
                                   int64_t rows, int64_t cols, int64_t ldx,
                                   int8_t* q, int64_t ldq, float* out_scale, float* mean,
                                   float* rstd, void* stream);

/*
 * w8a8_gemm_postscale -- INT8 x INT8 GEMM, INT32 accumulation over all of K,
 * fp32 post-scale epilogue, BF16 output.
 *
 * Passage: "Differences From TurboDiffusion", W8A8-kernel row and the
 * paragraph under the table (continuous accumulation across K, activation and
 * weight scales applied in the epilogue).
 *
 *   out[m,n] = bf16(fl32(fl32(fl32(acc[m,n]) * a_scale[m]) * w_scale[n])),
 *   acc[m,n] = sum_k a[m,k] * w[n,k]   (exact INT32)
 *
 *   a       [M, K] int8, stride lda (activation codes)
 *   w       [N, K] int8, stride ldw (weight codes, nn.Linear layout)
 *   a_scale [M] fp32, w_scale [N] fp32
 *   out     [M, N] BF16, stride ldo (output)
 * Requirements (else W8A8_ERR_UNSUPPORTED_SHAPE): K % 128 == 0, 128 <= K <=
 * W8A8_MAX_K, N % 128 == 0; a, w, out 16-byte aligned; lda % 16 == 0,
 * ldw % 16 == 0, ldo % 8 == 0; scales 4-byte aligned; 256 rows of a, of w
 * and of out each span less than 2^31 bytes (256 lda, 256 ldw, 512 ldo <
 * 2^31). M >= 0 arbitrary.
 *
 * This entry point always runs the single pass (one kernel). When the
 * 256 x 256 output tiles would leave most compute units idle (few tokens,
 * long K), w8a8_gemm_postscale_ex can split K over a caller-provided
 * workspace instead.
 */
w8a8_status_t w8a8_gemm_postscale(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                  const float* a_scale, const float* w_scale,
                                  uint16_t* out, int64_t ldo,
                                  int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w8a8_gemm_postscale_bias -- w8a8_gemm_postscale with an Int8Linear's bias
 * added in the epilogue.
 *
 * Passage: "Reused Components", W8A8 Linear bullet (Int8Linear takes the place
 * of Linear, which may carry a bias), with the epilogue of w8a8_gemm_postscale.
 *
 *   out[m,n] = bf16(fl32(fl32(fl32(fl32(acc) * a_scale[m]) * w_scale[n]) + bias[n]))
 *
 *   bias  [N] BF16, 16-byte aligned (input)
 * Everything else, requirements and errors as w8a8_gemm_postscale; the output
 * must not overlap the bias either.
 */
w8a8_status_t w8a8_gemm_postscale_bias(const int8_t* a, int64_t lda, const int8_t* w,
                                       int64_t ldw, const float* a_scale, const float* w_scale,
                                       const uint16_t* bias, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w8a8_gemm_postscale_gelu -- w8a8_gemm_postscale (optionally with a bias)
 * followed by the FFN activation, GELU in its erf form, on the BF16 output:
 * the up projection of a feed-forward block in one kernel.
 *
 * Passage: "Differences From TurboDiffusion", W8A8-kernel row (the kernel
 * serves the LTX FFN shapes) with the epilogue of w8a8_gemm_postscale. The
 * pages do not name the activation; GELU (erf form) is the reading taken.
 *
 *   y[m,n]   = bf16(fl32(fl32(fl32(acc) * a_scale[m]) * w_scale[n]) (+ bias[n]))
 *   out[m,n] = bf16(y/2 * erfc(-y / sqrt(2)))   (computed in fp32 from y)
 *
 *   bias  [N] BF16, 16-byte aligned, or NULL for none (input)
 * Everything else, requirements and errors as w8a8_gemm_postscale; the output
 * must not overlap the bias either. For every finite BF16 y the result is
 * the correctly rounded GELU (checked exhaustively); +inf gives +inf, -inf
 * and NaN give NaN. The kernel reads most results from a table built with
 * erfcf in fp32 and takes bf16(y/2) where |y| < 2^-9 (exact there). The
 * per-token quantisation of out (w8a8_quant_rows) gives the down
 * projection's input.
 */
w8a8_status_t w8a8_gemm_postscale_gelu(const int8_t* a, int64_t lda, const int8_t* w,
                                       int64_t ldw, const float* a_scale, const float* w_scale,
                                       const uint16_t* bias, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream);

/* Epilogue flag of w8a8_gemm_postscale_ex: GELU (erf form) of the BF16 output,
   as w8a8_gemm_postscale_gelu. */
#define W8A8_EPILOGUE_GELU 1

/*
 * w8a8_gemm_postscale_ex -- the post-scale GEMM family (optional bias,
 * optional GELU) with split-K over a caller-provided workspace.
 *
 * Passage: "Differences From TurboDiffusion", paragraph under the table: one
 * INT32 accumulation over all of K, the scales applied in the epilogue.
 * Integer addition is exact and associative, so K may be cut into parts whose
 * exact INT32 partial sums add up to exactly the full sum; the output is then
 * bit-identical to the single pass.
 *
 *   bias            [N] BF16, 16-byte aligned, or NULL (none)
 *   flags           0 or W8A8_EPILOGUE_GELU; other bits are
 *                   W8A8_ERR_INVALID_ARGUMENT
 *   parts           0: the library's choice for this shape and device
 *                   (w8a8_gemm_splitk_parts); 1: single pass; 2..64 (and at
 *                   most K / 128): exactly that many K parts
 *   workspace       device memory of workspace_bytes bytes, 16-byte aligned,
 *                   owned by the caller, or NULL. Split-K writes
 *                   parts * M * N INT32 partial sums there (the size
 *                   w8a8_gemm_postscale_workspace_size reports); it must not
 *                   overlap any input or the output, and must not be used by
 *                   other work until this call's work on `stream` is done.
 * With parts == 0 and no workspace the call runs the single pass. Asking for
 * parts > 1 without a workspace, or a workspace smaller than it needs, is
 * W8A8_ERR_INVALID_ARGUMENT. Everything else, requirements and errors as
 * w8a8_gemm_postscale (bias) and w8a8_gemm_postscale_gelu (flags).
 */
w8a8_status_t w8a8_gemm_postscale_ex(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                     const float* a_scale, const float* w_scale,
                                     const uint16_t* bias, int32_t flags,
                                     uint16_t* out, int64_t ldo,
                                     int64_t M, int64_t N, int64_t K,
                                     int32_t parts, void* workspace, int64_t workspace_bytes,
                                     void* stream);

/*
 * w8a8_gemm_postscale_workspace_size -- bytes of workspace w8a8_gemm_postscale_ex
 * needs for an M x N x K GEMM with `parts` (0 = the library's choice) on the
 * current device: parts * M * N * 4 when it splits K, 0 for the single pass,
 * -1 for arguments w8a8_gemm_postscale_ex would reject (a shape outside the
 * INT8 path, parts out of range). Host only, launches nothing.
 */
int64_t w8a8_gemm_postscale_workspace_size(int64_t M, int64_t N, int64_t K, int32_t parts);

/*
 * w8a8_gemm_postscale_noalloc -- w8a8_gemm_postscale_ex for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the split-K partial sums go to a fixed 64 MiB
 * device array inside the library instead of a caller workspace. The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 *   parts   0: the library's choice among the part counts whose partial sums
 *           (parts * M * N * 4 bytes) fit in 64 MiB (1 when none does);
 *           1: single pass; 2..64 (and at most K / 128): exactly that many,
 *           rejected with W8A8_ERR_INVALID_ARGUMENT if they do not fit.
 * Other arguments, requirements and errors as w8a8_gemm_postscale_ex.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; each split call writes every partial sum it reads, so nothing needs
 * clearing. Calls that overlap on one GPU (other streams or threads) race on
 * the array: the caller serialises them. The array is looked up once per
 * device on the first call that needs it.
 */
w8a8_status_t w8a8_gemm_postscale_noalloc(const int8_t* a, int64_t lda, const int8_t* w,
                                          int64_t ldw, const float* a_scale,
                                          const float* w_scale, const uint16_t* bias,
                                          int32_t flags, uint16_t* out, int64_t ldo,
                                          int64_t M, int64_t N, int64_t K, int32_t parts,
                                          void* stream);

/*
 * w8a8_gemm_blockwise -- blockwise-scaled W8A8 GEMM (the original
 * TurboDiffusion scheme, "Differences From TurboDiffusion", W8A8 kernel row).
 *
 * For each 128-wide K block kb, in ascending order:
 *   acc_kb = exact INT32 block sum; s = fl32(a_scale[m,kb] * w_scale[n/128,kb]);
 *   c = fmaf(fl32(acc_kb), s, c)            (c starts at 0)
 * out[m,n] = bf16(c).
 *
 *   a_scale [M, K/128] fp32 dense; w_scale [N/128, K/128] fp32 dense.
 * Other arguments and requirements as w8a8_gemm_postscale.
 */
w8a8_status_t w8a8_gemm_blockwise(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                  const float* a_scale, const float* w_scale,
                                  uint16_t* out, int64_t ldo,
                                  int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w8a8_gemm_i32 -- the post-scale GEMM's main loop with the raw INT32
 * accumulators as output (out[m,n] = sum_k a[m,k] * w[n,k]), so the integer
 * part of the path can be checked bit for bit. Same passage and requirements
 * as w8a8_gemm_postscale, with out int32 [M, N], ldo % 4 == 0 (and 1024 ldo
 * < 2^31).
 */
w8a8_status_t w8a8_gemm_i32(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                            int32_t* out, int64_t ldo,
                            int64_t M, int64_t N, int64_t K, void* stream);

/* Static description of a status code. */
const char* w8a8_status_string(w8a8_status_t s);

/* Description of the last error on the calling thread ("" if none). */
const char* w8a8_last_error(void);

/* Library version string. */
const char* w8a8_version(void);

/*
 * w8a8_gemm_splitk_parts -- how many K parts w8a8_gemm_postscale_ex chooses
 * (parts == 0) for an M x N x K GEMM on the current device: 1 for a single
 * pass, else the parts of the split-K path (exact INT32 partial sums in the
 * caller's workspace of parts * M * N * 4 bytes, then one epilogue pass).
 * Host only, launches nothing. Passage: "Differences From TurboDiffusion",
 * paragraph under the table (one INT32 accumulation over K; integer sums may
 * be formed in parts and added exactly).
 */
int32_t w8a8_gemm_splitk_parts(int64_t M, int64_t N, int64_t K);

/*
 * w8a8_gemm_tile_channels -- the output-channel width of the tiles a single
 * pass of the post-scale family (blockwise = 0) or of w8a8_gemm_blockwise
 * (blockwise = 1) uses for an M x N x K GEMM on the current device: 256 (the
 * persistent kernels: 256 x 256 post-scale tiles, 256-channel x 128-token
 * blockwise tiles) or 160 (128-token x 160-channel tiles, one workgroup per
 * tile, chosen for few tokens where the larger tiles would leave compute
 * units idle). The results are identical either way. -1 for a shape the INT8
 * path rejects. Host only, launches nothing. Passage: "Differences From
 * TurboDiffusion", W8A8-kernel row (the kernels serve the LTX shapes, and
 * other selected Linears).
 */
int32_t w8a8_gemm_tile_channels(int64_t M, int64_t N, int64_t K, int32_t blockwise);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
