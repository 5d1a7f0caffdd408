/*
 * pwq.h - layer-wise post-training weight quantization (RTN and GPTQ) on gfx950.
 *
 * C ABI of libpwq.so.  Every compute call enqueues hand-written HIP kernels on the
 * caller's stream and returns without synchronising.
 *
 * Conventions shared by all calls
 * -------------------------------
 *  - Matrices are row-major.  W is d_out x d_in (one row per output channel), X is
 *    n_tok x d_in (one row per calibration token), H and U are d_in x d_in.
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - Leading dimensions (ldx, ldw) are in elements and must be >= d_in.
 *  - Float16 values (scales) travel as their raw 16-bit patterns in uint16_t.
 *    bfloat16 X travels as raw 16-bit patterns as well (pwq_dtype PWQ_BF16).
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *  - The caller owns and allocates every buffer: inputs, outputs and a workspace of
 *    at least the size the matching *_workspace_size call returns.  The library
 *    allocates no device memory and keeps no per-call state, so calls on different
 *    streams with disjoint buffers may run concurrently.
 *  - Every call checks its arguments on the host first.  On any return other than
 *    PWQ_OK nothing has been enqueued, except PWQ_EHIP, which reports a launch
 *    failure after earlier kernels of the same call may already be queued.
 *  - A numerically failed factorisation (H not positive definite) is not a return
 *    code: it is written to the device int32 `info` (see pwq_chol_inverse_upper).
 *  - Empty inputs (n_tok == 0, d_out == 0) are valid and enqueue nothing, except
 *    that pwq_recon_mse writes 0 to *mse.
 *
 * Sources of the method (page title, then section):
 *  [GPT2-RE]  "GPT-2 Quantization Reconstruction Error" - "What this project does", "Setup".
 *  [MQM]      "Model Quantization Mechanics: Precision Reduction and Weight Formatting" -
 *             1 "Affine Quantization", "Group-wise Quantization"; 2.1 "GPTQ".
 *  [GPTQ-P]   "GPTQ: Post-Training INT4" - "OBQ Foundation", "Hessian-Based Weight Update",
 *             "The GPTQ Algorithm", "Group Quantization", "Running GPTQ with AutoGPTQ".
 */
#ifndef PWQ_H
#define PWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PWQ_ABI_VERSION 5

typedef enum pwq_status {
    PWQ_OK = 0,
    PWQ_EINVAL = 1,      /* bad pointer, size, stride, bits, group or block size      */
    PWQ_EDTYPE = 2,      /* dtype not supported by this call                          */
    PWQ_EWORKSPACE = 3,  /* workspace pointer NULL or smaller than *_workspace_size   */
    PWQ_EHIP = 4         /* a kernel launch failed; see pwq_last_hip_error()          */
} pwq_status;

typedef enum pwq_dtype {
    PWQ_F32 = 0,
    PWQ_F16 = 1,
    PWQ_BF16 = 2
} pwq_dtype;

/* Quantizer settings, the knobs of [GPTQ-P] "Running GPTQ with AutoGPTQ" (bits,
 * group_size, desc_act) plus the lazy-batch width of [GPTQ-P] "The GPTQ Algorithm".
 * The plain calls are symmetric (sym=True there): codes in [-(2^(bits-1)-1), 2^(bits-1)-1],
 * no zero-point.  The *_zp calls are the zero-point form (see "Zero-point form" below).
 *   bits        2..8
 *   group_size  0 = one scale per output row ([GPT2-RE]); else an even number >= 2 of
 *               consecutive input columns sharing one scale ([MQM] "Group-wise
 *               Quantization").  For GPTQ, group_size must be a multiple of 32 that
 *               divides block_size or is a multiple of it, so a group never starts
 *               inside a block and ends after it.
 *   block_size  GPTQ lazy-batch width B: 32, 64 or 128.
 *   act_order   nonzero: columns were processed in the order `perm` (desc_act). */
typedef struct pwq_params {
    int32_t bits;
    int32_t group_size;
    int32_t block_size;
    int32_t act_order;
} pwq_params;

/* ABI version the library was compiled with (PWQ_ABI_VERSION). */
int pwq_version(void);

/* Static text for a status code. */
const char* pwq_status_string(int status);

/* hipError_t of the last PWQ_EHIP on the calling thread (0 if none). */
int pwq_last_hip_error(void);

/* ------------------------------------------------------------------ kernel timing -----
 * Opt-in timing of the path's large kernels, to measure each against its roofline: the
 * Hessian's contraction, and GPTQ's lazily batched trailing updates and column blocks
 * ([GPTQ-P] "The GPTQ Algorithm", block-wise processing: one batched update per block
 * in place of one per column).  While enabled, every launch of a listed class records a
 * pair of HIP events on the stream it runs on, with the launch's algorithmic work:
 *   PWQ_PROF_XTX      the MFMA contraction of pwq_hessian_accumulate: n_tok d_in (d_in + 1)
 *                     flops per call (the symmetric half of 2 n_tok d_in^2);
 *   PWQ_PROF_UPDATE   the products W[:, c0:c1] -= Err U[rows, c0:c1] of
 *                     pwq_gptq_quantize_layer(_zp) on float32 MFMA: 2 d_out k (c1 - c0)
 *                     flops each (k error columns); with PWQ_PROF_UPDATE_SPLIT's products
 *                     (counted as float32 work) they sum to d_out d_in (d_in - B) over a
 *                     layer when the kernel with four lanes per row runs (d_out > 4096);
 *   PWQ_PROF_UPDATE_SPLIT  the same products where they run on bfloat16 MFMA as the six
 *                     larger products of their operands' three-piece bfloat16 splits (deep
 *                     products past a super-block on large layers; the splitting kernels
 *                     are inside the timed span): 12 d_out k (c1 - c0) flops each, k the
 *                     error columns rounded up to a multiple of 64 (the bfloat16 work
 *                     executed);
 *   PWQ_PROF_COLUMNS  the column-block kernels (quantize, error, in-block rank-1 updates):
 *                     d_out B (B - 1) flops per block of B columns;
 *   PWQ_PROF_RTN      the kernel of pwq_rtn_quantize(_zp): the bytes it must move (W, the
 *                     codes and nibbles asked for, the scales and zeros);
 *   PWQ_PROF_DEQUANT  the kernel of pwq_dequant(_zp): nibbles or codes, scales and zeros,
 *                     g_idx and the output, once each.
 * The record is process-wide and guarded by a mutex.  The events add a little time
 * between launches: time throughput with timing disabled.
 *   pwq_profile_enable  nonzero starts recording (discarding anything unread), 0 stops.
 *   pwq_profile_read    waits for the recorded events and writes, for classes
 *                       0 .. n_classes - 1, the summed milliseconds, summed work and launch
 *                       count into host arrays; clears the record.  PWQ_EINVAL for
 *                       n_classes < 1 or a NULL array; PWQ_EHIP if an event failed. */
typedef enum pwq_prof_class {
    PWQ_PROF_XTX = 0,
    PWQ_PROF_UPDATE = 1,
    PWQ_PROF_COLUMNS = 2,
    PWQ_PROF_RTN = 3,
    PWQ_PROF_DEQUANT = 4,
    PWQ_PROF_UPDATE_SPLIT = 5,
    PWQ_PROF_CLASSES = 6
} pwq_prof_class;
pwq_status pwq_profile_enable(int on);
pwq_status pwq_profile_read(double* ms, double* work, int64_t* launches, int n_classes);

/* ------------------------------------------------------------------ Hessian -------
 * H += 2 * X^T X, summed over the n_tok tokens of this call ([GPTQ-P] "Hessian-Based
 * Weight Update": H = 2 X X^T with X as d_in x tokens; here X is stored tokens x d_in).
 * Call it once per token tile to stream a large calibration set; the caller zeroes H
 * before the first tile.  Both triangles of H are written (full symmetric storage).
 *   X        n_tok x d_in, x_dtype PWQ_F32 or PWQ_BF16, leading dimension ldx.
 *   H        d_in x d_in float32, accumulated in place.
 *   ws       workspace of pwq_hessian_workspace_size(n_tok, d_in, x_dtype) bytes
 *            (may be 0 bytes; then ws may be NULL).
 * Products are accumulated in float32 with MFMA; partial sums over token chunks are
 * added in a fixed order, so repeated calls give bit-identical H. */
size_t pwq_hessian_workspace_size(int64_t n_tok, int64_t d_in, int x_dtype);
pwq_status pwq_hessian_accumulate(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                                  float* H, void* ws, size_t ws_bytes, void* stream);

/* H_ii += lambda for every i, lambda = damp * mean(diag H) of the undamped H
 * (damp_percent of [GPTQ-P] "Running GPTQ with AutoGPTQ"; 0 allowed).
 *   lambda_out  optional device float receiving lambda (NULL to skip). */
pwq_status pwq_hessian_damp(float* H, int64_t d_in, float damp, float* lambda_out, void* stream);

/* Act-order (desc_act of [GPTQ-P] "Running GPTQ with AutoGPTQ"): perm[p] = the input
 * column processed at position p, sorting diag H descending, ties by lower index.
 *   perm  int32[d_in]. */
pwq_status pwq_act_order_perm(const float* H, int64_t d_in, int32_t* perm, void* stream);

/* ------------------------------------------------------------------ H^-1 factor ---
 * U upper triangular with H^-1 = U^T U and U_jj > 0: the Cholesky factor of the
 * inverse Hessian of [MQM] 2.1 "GPTQ", whose rows drive the column loop.  If perm is
 * not NULL the factor is of P H P^T, i.e. of H[perm][:, perm].
 * Computed as H = V V^T (V upper: Cholesky eliminating from the last column to the
 * first) followed by U = V^-1, so H^-1 is never formed.
 *   H     n x n float32, read only.  Without perm only the upper triangle is read; with
 *         perm the full rows perm[i] are read, so H must hold both triangles (as
 *         pwq_hessian_accumulate writes it).
 *   U     n x n float32 output; the strictly lower triangle is written as 0.
 *   info  device int32: 0 on success; k > 0 if the pivot of column k-1 (in the order
 *         of P H P^T) was not positive, i.e. H is not positive definite.  U is then
 *         undefined, and pwq_gptq_quantize_layer given this info writes nothing.
 *   ws    pwq_chol_workspace_size(n) bytes: the panels of up to 1024 columns (n x 1024
 *         floats from n = 4096 on, n x 128 below) and, where the deep products can run on
 *         bfloat16 MFMA as six products of three-piece splits (n above 8192),
 *         their pieces (3 x 1024 bfloat16 per row, rows in whole 256-row panels).
 * Those split products keep every product term within 2^-23 relative of the exact one
 * and accumulate in float32, as a float32 product does. */
size_t pwq_chol_workspace_size(int64_t n);
pwq_status pwq_chol_inverse_upper(const float* H, int64_t n, const int32_t* perm, float* U, int32_t* info,
                                  void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ GPTQ ----------
 * The column loop of [GPTQ-P] "The GPTQ Algorithm" with the factor U of
 * pwq_chol_inverse_upper.  Columns (in processing order) are taken in blocks of
 * block_size; for each column j of a block: at a group's first column, the scale of
 * every row is absmax(current values of the group) / qmax, rounded to float32 and then
 * to float16 (per-row mode: from the original row); code = nearest integer to w / s
 * (exact quotient, ties to even), clamped to +-qmax; e = (w - s * code) / U_jj;
 * the block's later columns get w_k -= e * U_jk; after the block every later column
 * gets W -= Err * U[block, later] in one product.
 *   W          d_out x d_in, w_dtype PWQ_F32 or PWQ_F16, leading dimension ldw; read only
 *              (the float32 working copy lives in ws).
 *   U, info    from pwq_chol_inverse_upper (of the permuted H when act_order).
 *   params     host pointer.
 *   perm       int32[d_in] from pwq_act_order_perm; required iff params->act_order.
 *   scales_in  optional fp16 d_out x n_groups: fixed scales instead of computed ones.
 *   codes      optional int8 d_out x d_in, in ORIGINAL column order.
 *   packed     optional uint8 d_out x d_in/2 (bits == 4, d_in even): nibble = code + 8,
 *              even column in the low nibble ([GPTQ-P] "Group Quantization" storage).
 *              At least one of codes / packed must be given.
 *   scales_out fp16 d_out x n_groups (groups in processing order), required.
 *   g_idx      int32[d_in], group of each original column; required iff act_order.
 *   ws         pwq_gptq_workspace_size(d_out, d_in, params) bytes: the float32 working
 *              copy of W, the errors of up to 1024 columns, the act-order buffers, and on
 *              large layers the pieces of the trailing products that run on bfloat16
 *              MFMA (six products of three-piece splits, each product term within 2^-23
 *              relative of the exact one, float32 accumulation). */
size_t pwq_gptq_workspace_size(int64_t d_out, int64_t d_in, const pwq_params* params);
pwq_status pwq_gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                                   const float* U, const int32_t* info, const pwq_params* params,
                                   const int32_t* perm, const uint16_t* scales_in,
                                   int8_t* codes, uint8_t* packed, uint16_t* scales_out, int32_t* g_idx,
                                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ RTN -----------
 * Round-to-nearest ([GPT2-RE] "What this project does"; [MQM] "Affine Quantization"
 * with Z = 0 and "Group-wise Quantization"): per row (group_size 0) or per group of
 * group_size consecutive columns, s = fp16(fp32(absmax / qmax)) from the original W,
 * code = nearest integer to w / s (exact quotient, ties to even), clamped to +-qmax;
 * s = 0 gives code 0.  Same output formats as pwq_gptq_quantize_layer (no act-order).
 *   scales_in optional fixed fp16 scales; scales_out required (copied from scales_in
 *   when given). */
pwq_status pwq_rtn_quantize(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                            int32_t bits, int32_t group_size, const uint16_t* scales_in,
                            int8_t* codes, uint8_t* packed, uint16_t* scales_out, void* stream);

/* ------------------------------------------------------------------ dequant -------
 * What[r, c] = s[r, group(c)] * code[r, c] ([MQM] "Affine Quantization", Z = 0), the
 * product formed exactly in float32 and rounded once to out_dtype (PWQ_F32, PWQ_F16 or
 * PWQ_BF16).  group(c) = 0 (group_size 0), g_idx[c] (g_idx given), else c / group_size.
 * Exactly one of packed (bits 4) / codes is given.  W_out is d_out x d_in, dense. */
pwq_status pwq_dequant(const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                       int64_t d_out, int64_t d_in, int32_t bits, int32_t group_size,
                       void* W_out, int out_dtype, void* stream);

/* ------------------------------------------------------------------ MSE -----------
 * Per-layer reconstruction error ([GPT2-RE] "What this project does", step 5; the
 * objective ||WX - What X||^2 of [GPTQ-P] "OBQ Foundation"):
 *   mse = sum over tokens t and outputs o of (X (W - What)^T)[t, o]^2 / (n_tok * d_out),
 * with What decoded on the fly from packed or codes (+ scales, g_idx) as in
 * pwq_dequant; the product is never written out.  Per-tile sums are added in a fixed
 * order in float64, so the result is reproducible bit for bit.
 *   X       n_tok x d_in, x_dtype PWQ_F32 or PWQ_BF16, leading dimension ldx.
 *   W       d_out x d_in, w_dtype PWQ_F32 or PWQ_F16, leading dimension ldw.
 *   mse     device double.
 *   ws      pwq_recon_mse_workspace_size(n_tok, d_in, d_out) bytes. */
size_t pwq_recon_mse_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out);
pwq_status pwq_recon_mse(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                         const void* W, int w_dtype, int64_t ldw,
                         const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                         int64_t d_out, int32_t bits, int32_t group_size,
                         double* mse, void* ws, size_t ws_bytes, void* stream);

/* pwq_recon_mse_hessian: the same mean square, through the Hessian the path has formed:
 * sum over tokens and outputs of (X (W - What)^T)^2 = tr((W - What) X^T X (W - What)^T)
 * = tr((W - What) H (W - What)^T) / 2 for H = 2 X^T X ([GPTQ-P] "OBQ Foundation": the layer
 * error as a quadratic form in H), so
 *   mse = tr((W - What) (H - shift I) (W - What)^T) / (2 n_tok d_out),
 * equal to pwq_recon_mse's in exact arithmetic.  One d_out x d_in x d_in product instead of
 * n_tok x d_in x d_out: the cheaper route when n_tok is well above d_in.  Small layers run it
 * on float32 MFMA; from 256 output tiles of 256 x 256 on (ceil(d_out/256) ceil(d_in/256)
 * >= 256) it uses H's symmetry (each 256-column block of the output contracts only up to the
 * diagonal block) and a bfloat16 hi/lo split of both operands (three products, each exact
 * in float32; the dropped terms are below 2^-16 of each product), about 3 d_out d_in^2
 * bfloat16 flops.
 *   H        d_in x d_in float32, symmetric (pwq_hessian_accumulate's output): the float32
 *            route reads both triangles, the split route the lower one and the diagonal; row
 *            stride ldh >= d_in; may already be damped: h_shift (device float, or NULL for
 *            0) is what damping added to its diagonal (pwq_hessian_damp's lambda_out).
 *   n_tok    the number of tokens H was accumulated over.
 *   W, codes / packed, scales, g_idx, bits, group_size: as pwq_recon_mse; zeros NULL for
 *            symmetric codes (int8, nibble - 8), else the zero-point form (uint8 codes,
 *            nibble = code, What = S (code - Z)).
 *   mse      device double.
 *   ws       pwq_recon_mse_hessian_workspace_size(d_in, d_out) bytes.
 * n_tok == 0 or d_out == 0 writes 0 to *mse; then only mse is read (the other pointers may
 * be NULL). */
size_t pwq_recon_mse_hessian_workspace_size(int64_t d_in, int64_t d_out);
pwq_status pwq_recon_mse_hessian(const float* H, int64_t ldh, int64_t d_in, int64_t n_tok, const float* h_shift,
                                 const void* W, int w_dtype, int64_t ldw,
                                 const uint8_t* packed, const void* codes, const uint16_t* scales,
                                 const uint16_t* zeros, const int32_t* g_idx, int64_t d_out, int32_t bits,
                                 int32_t group_size, double* mse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ Zero-point form
 * The affine quantizer of [MQM] "Affine Quantization" and "Group-wise Quantization": per
 * row and group a float16 scale S and a zero Z, code = round(w / S) + Z and value
 * S (code - Z); [GPTQ-P] "Group Quantization" stores Z in 16 bits beside S (4 + 32 / g
 * bits per weight).  A group's range [lo, hi] = [min(w, 0), max(w, 0)] (so that real 0 is
 * a level) is mapped onto the codes 0 .. top = 2^bits - 1:
 *   S = fp16(fp32(hi - lo) / top)      (one float32 subtraction and division, one rounding)
 *   Z = nearest integer to -lo / S (exact quotient, ties to even), clamped to [0, top];
 *       S = 0 gives Z = 0
 *   code = nearest integer to w / S (exact quotient, ties to even) plus Z, clamped to
 *       [0, top]; S = 0 gives code 0.
 * Codes are unsigned bytes (uint8_t); INT4 nibbles hold the code itself (no offset), even
 * column in the low nibble.  Zeros travel as uint16_t, d_out x n_groups like the scales.
 * Fixed quantizers are given as scales_in and zeros_in together (both or neither); zeros_in
 * entries above top are taken as top (and written so to zeros_out).  The decoding calls
 * (dequant, MSE) expect zeros in 0 .. top, as the quantizing calls write them.
 * Everything else - arguments, checks, workspaces, layouts - is that of the plain call of
 * the same name, and the workspace size queries are shared.
 *
 * GPTQ: at a group's first column S and Z come from the current values of the group's
 * columns, where the plain call takes its absmax; the error of column j is
 * e = (w - S (code - Z)) / U_jj.  zeros_out is required. */
pwq_status pwq_gptq_quantize_layer_zp(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                                      const float* U, const int32_t* info, const pwq_params* params,
                                      const int32_t* perm, const uint16_t* scales_in, const uint16_t* zeros_in,
                                      uint8_t* codes, uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out,
                                      int32_t* g_idx, void* ws, size_t ws_bytes, void* stream);

/* RTN with zero-points: S and Z from the original W per row or group.  zeros_out required. */
pwq_status pwq_rtn_quantize_zp(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                               int32_t bits, int32_t group_size, const uint16_t* scales_in, const uint16_t* zeros_in,
                               uint8_t* codes, uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out,
                               void* stream);

/* What[r, c] = S[r, group(c)] * (code[r, c] - Z[r, group(c)]), exact in float32 (for zeros
 * in 0 .. top), rounded once to out_dtype.  zeros required. */
pwq_status pwq_dequant_zp(const uint8_t* packed, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          const int32_t* g_idx, int64_t d_out, int64_t d_in, int32_t bits, int32_t group_size,
                          void* W_out, int out_dtype, void* stream);

/* pwq_recon_mse with What decoded as in pwq_dequant_zp.  zeros required; the workspace is
 * pwq_recon_mse_workspace_size(n_tok, d_in, d_out) bytes. */
pwq_status pwq_recon_mse_zp(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                            const void* W, int w_dtype, int64_t ldw,
                            const uint8_t* packed, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                            const int32_t* g_idx, int64_t d_out, int32_t bits, int32_t group_size,
                            double* mse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ per-tensor quantizer
 * One quantizer for the whole matrix, the per-tensor alternative to per-channel scales of
 * [GPT2-RE] "Possible extensions": from the original W, s = fp16(fp32(max |w|) / qmax)
 * (zeros_out NULL), or the zero-point pair of the range [min(w, 0), max(w, 0)] of the whole
 * tensor (zeros_out given), by the same rules as the per-row quantizers.  It is written in
 * the per-row format, every row holding the same value: scales_out (and zeros_out) are
 * d_out x 1, to be passed as fixed scales (and zeros) with group_size 0 to the RTN and GPTQ
 * calls; dequant and the MSE then read them unchanged.
 *   ws   pwq_tensor_scales_workspace_size() bytes. */
size_t pwq_tensor_scales_workspace_size(void);
pwq_status pwq_tensor_scales(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, int32_t bits,
                             uint16_t* scales_out, uint16_t* zeros_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ activation-aware scaling
 * [MQM] 2.2 "AWQ": salience of a weight comes from the size of its input activations; a
 * per-channel s multiplies W's column and divides X's column, leaving the layer output
 * unchanged, so that salient channels lose less to rounding ([GPT2-RE] "Possible
 * extensions": scale up the important channels before quantizing).  The pages give no rule
 * for s; these calls take s_c = a_c^alpha with a_c the mean over tokens of |X_tc| (s_c = 1
 * where a_c = 0) and choose alpha on a grid by the reconstruction MSE.
 *
 * pwq_channel_abs_mean: abs_mean[c] = mean over the n_tok tokens of |X[t][c]| (float32
 * result of float64 sums; X float32 or bfloat16, leading dimension ldx).
 *   ws  pwq_channel_abs_mean_workspace_size(n_tok, d_in) bytes. */
size_t pwq_channel_abs_mean_workspace_size(int64_t n_tok, int64_t d_in);
pwq_status pwq_channel_abs_mean(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, float* abs_mean,
                                void* ws, size_t ws_bytes, void* stream);

/* pwq_awq_search: for alpha_k = k / (n_alpha - 1), k = 0 .. n_alpha - 1 (alpha_0 = 0 is
 * plain RTN), s = abs_mean^alpha_k (double pow rounded once to float32), What = RTN of
 * W diag(s) (the rules of pwq_rtn_quantize, or of pwq_rtn_quantize_zp when zero_point)
 * divided column-wise by s, and
 *   mse_out[k] = tr((W - What) H (W - What)^T) / (2 n_tok d_out),
 * the reconstruction MSE of pwq_recon_mse through H = 2 X^T X.  best_out = the first k of
 * least score; s_out = its s (float32, d_in); codes / packed / scales_out (/ zeros_out) =
 * RTN of W diag(s_out) in the output formats of the RTN calls (codes are int8 symmetric or
 * uint8 zero-point bytes).  At inference X is divided by s_out column-wise.
 *   H         d_in x d_in float32 from pwq_hessian_accumulate BEFORE damping (the score
 *             is the reconstruction error of the calibration set), both triangles.
 *   abs_mean  from pwq_channel_abs_mean over the same tokens; n_tok their number.
 *   mse_out   device double[n_alpha]; best_out device int32.
 *   ws        pwq_awq_search_workspace_size(d_out, d_in) bytes.
 * Each candidate costs one d_out x d_in x d_in float32 MFMA product. */
size_t pwq_awq_search_workspace_size(int64_t d_out, int64_t d_in);
pwq_status pwq_awq_search(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, const float* H,
                          int64_t n_tok, const float* abs_mean, int32_t bits, int32_t group_size, int32_t n_alpha,
                          int32_t zero_point, double* mse_out, int32_t* best_out, float* s_out, void* codes,
                          uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------ product with What
 * Y = X What^T: the quantized layer applied to activations, the inference use of the result
 * ([GPTQ-P] "Running GPTQ with AutoGPTQ"), with What decoded on the fly from packed INT4
 * nibbles and scales (symmetric: What = s (nibble - 8)) or, when zeros is not NULL, from
 * the zero-point form (What = S (nibble - Z)), as pwq_dequant / pwq_dequant_zp define it.
 * What is never rounded: each group's sum of x (code - zero) is formed from exact products
 * (float16 MFMA on the small integer codes) and scaled once by its scale, in float32; the
 * result is rounded once to y_dtype.
 *   X       n_tok x d_in float16 (x_dtype PWQ_F16), leading dimension ldx (a multiple of 8,
 *           at most 2^24), 16-byte aligned.
 *   packed  d_out x d_in/2 (d_in a multiple of 32), 16-byte aligned; columns in their
 *           original order (no g_idx: a layer quantized with act-order is served by its
 *           dequantized weights).
 *   scales, zeros  d_out x n_groups; group_size 0 (one scale per row) or a multiple of 128.
 *   Y       n_tok x d_out, y_dtype PWQ_F32 / PWQ_F16 / PWQ_BF16, leading dimension ldy.
 *   ws      pwq_quantized_matmul_workspace_size(n_tok, d_in, d_out) bytes (0 when the columns
 *           are not split; then ws may be NULL).
 * Built for few tokens (the weights are the traffic); any n_tok up to 65535 * 16 works, the
 * weights being read once per 16 tokens. */
size_t pwq_quantized_matmul_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out);
pwq_status pwq_quantized_matmul(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                                const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                                int64_t d_out, int32_t group_size, void* Y, int y_dtype, int64_t ldy,
                                void* ws, size_t ws_bytes, void* stream);

/* The same product for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Identical arguments and
 * results to pwq_quantized_matmul, without the workspace: the column splits' partial sums go
 * to a scratch array of PWQ_QMM_SCRATCH_BYTES that the library holds in device memory on
 * every GPU it runs on, until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its first call on a device looks up that device's
 * copy of the array (hipGetSymbolAddress, with the device current).
 *   Errors: as pwq_quantized_matmul; PWQ_EWORKSPACE when
 *   pwq_quantized_matmul_workspace_size(n_tok, d_in, d_out) exceeds PWQ_QMM_SCRATCH_BYTES
 *   (e.g. d_in = 28672, d_out = 8192 fits up to n_tok = 36; d_in = 8192, d_out = 28672 up
 *   to 36 as well); PWQ_EHIP when the lookup fails.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 *   streams, or two threads) race and may return wrong sums.  Each call writes every
 *   partial sum it later reads, so nothing needs clearing between calls. */
#define PWQ_QMM_SCRATCH_BYTES ((size_t)32 << 20)
pwq_status pwq_quantized_matmul_noalloc(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                                        const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                                        int64_t d_out, int32_t group_size, void* Y, int y_dtype, int64_t ldy,
                                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PWQ_H */
