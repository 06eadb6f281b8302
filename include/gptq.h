/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ one-layer library.
 *
 * GPTQ quantizes one linear layer's weights W (rows x cols, output x input
 * features) column by column and, after each column, moves the columns not
 * yet quantized so that the layer output on calibration inputs X changes as
 * little as possible.  The library exposes the three stages of that path:
 *
 *   gptq_hessian_accumulate  H += alpha * X^T X     (alpha = 2 gives H = 2XX^T)
 *   gptq_prepare_hinv        damp H -> Hinv, the upper Cholesky factor of
 *                            the damped inverse (one factorization and one
 *                            triangular inverse; gptq_prepare_hinv_three_step
 *                            takes the pages' three steps)
 *   gptq_quantize_layer      blocked column sweep + lazy updates -> codes,
 *                            scales, zeros, per-column losses
 *
 * and the act-order variant (columns in decreasing order of H_qq):
 *
 *   gptq_act_order, gptq_prepare_hinv_perm, gptq_quantize_layer_perm
 *
 * Sources (page titles and sections):
 *   "GPTQ: fixing errors as you go": "The algorithm, in words", "Objective",
 *       "The OBQ update", "The tricks that make it fast".
 *   "GPTQ > The GPTQ Algorithm": column-wise processing, lazy batch updates,
 *       Cholesky-based inverse updates, the step-by-step procedure.
 *   "GPTQ-style round-to-nearest with Hessian weighting": the
 *       gptq_quantize_layer listing (quantizer) and collect_hessian listing.
 *   "GPTQ, Line by Line: Hessian-Based Weight Quantization": Hessian,
 *       percdamp, blocks of 128 and Cholesky questions.
 *
 * Conventions (all entry points):
 *   - Matrices are row-major.  Every matrix pointer is a DEVICE pointer owned
 *     by the caller; the library never allocates, frees or keeps a pointer
 *     past the call.  Scalars and `info` are host values.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it in order; only gptq_prepare_hinv synchronizes it
 *     (once, to read the pivot flag).
 *   - `workspace` is caller-owned device memory of at least
 *     gptq_workspace_bytes(op, ...) bytes, 256-byte aligned.  Its contents on
 *     entry are ignored and on return undefined.  NULL is accepted when the
 *     required size is 0.
 *   - Every argument is validated on the host before any HIP call; an invalid
 *     call returns an error status and enqueues nothing.  HIP launch errors
 *     return GPTQ_ERR_HIP.
 *   - No global mutable state: calls on different streams with different
 *     buffers may run concurrently.  Calls that share a buffer must be ordered
 *     by the caller.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gptq_status {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad stride, bad bits ... */
  GPTQ_ERR_WORKSPACE = 2,   /* workspace smaller than gptq_workspace_bytes()   */
  GPTQ_ERR_NOT_PD = 3,      /* a Cholesky pivot was <= 0 or NaN (see *info)     */
  GPTQ_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed       */
  GPTQ_ERR_UNSUPPORTED = 5  /* valid request outside what the kernels handle    */
} gptq_status;

enum gptq_dtype { GPTQ_DTYPE_F16 = 0, GPTQ_DTYPE_F32 = 1 };

enum gptq_op {
  GPTQ_OP_ACCUMULATE = 0, /* sizes: rows ignored, cols = d, n = tokens         */
  GPTQ_OP_PREPARE = 1,    /* sizes: rows ignored, cols = d, n ignored          */
  GPTQ_OP_QUANTIZE = 2,   /* sizes: rows, cols, n ignored                       */
  GPTQ_OP_QUANTIZE_PERM = 3 /* gptq_quantize_layer_perm: rows, cols, n ignored    */
};

/* Library version (major*10000 + minor*100 + patch). */
int gptq_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* gptq_status_string(int status);

/* Bytes of device workspace the given operation needs at these sizes
 * (0 if none).  Deterministic in its arguments; returns 0 for sizes the
 * operation would reject. */
size_t gptq_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t n);

/*
 * gptq_hessian_accumulate -- H += alpha * X^T X.
 *
 * The Hessian of the layer-output error ||W X - W_hat X||^2 with respect to a
 * row of W is 2 X X^T for X feature-major ("GPTQ: fixing errors as you go",
 * "Objective"); calibration inputs are summed batch by batch
 * ("GPTQ-style round-to-nearest ...", collect_hessian listing).  Here X is
 * token-major, as a forward hook records it, so the same matrix is
 * alpha * X^T X with alpha = 2.  H is NOT divided by the token count.
 *
 *   H      d x d fp32, both triangles updated (the result stays exactly
 *          symmetric if H was).  The caller zero-initializes H before the
 *          first chunk; successive calls add further token chunks.
 *   d      number of input channels, >= 1.
 *   X      n x d fp16 (IEEE binary16), row t at X + t*ldx.
 *   n      tokens in this chunk, >= 0 (0 is a no-op).
 *   ldx    row stride of X in elements, >= d.
 *   alpha  scale applied to X^T X (2.0 for H = 2XX^T).
 *   Products of fp16 values are exact in fp32.  The tokens are cut into
 *   splits of at most 4096 (of n/128 above 524288 tokens per call); each
 *   split's sums are accumulated in fp32, the
 *   split sums are added in fp64 in split order, and each entry is rounded
 *   once to fp32 when alpha times that sum is added into H.  The order
 *   depends only on (d, n), so results are bitwise reproducible.
 */
gptq_status gptq_hessian_accumulate(float* H, int64_t d, const void* X, int64_t n,
                                    int64_t ldx, float alpha, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * gptq_prepare_hinv -- Hinv = upper Cholesky factor of (H + lambda I)^{-1},
 * lambda = percdamp * mean(diag H).
 *
 * Damping: "GPTQ, Line by Line", percdamp question (percdamp times the mean
 * Hessian diagonal added to every diagonal entry).  The result is the factor
 * the Cholesky question of the same page and the cholesky /
 * cholesky_inverse / cholesky(upper) calls of the "GPTQ-style
 * round-to-nearest ..." listing produce: the upper Cholesky factor U of
 * H_d^{-1} (H_d^{-1} = U^T U).  It is computed as U = J L^{-1} J, where J
 * reverses the order of rows and columns and L is the lower Cholesky factor
 * of J H_d J: one factorization and one triangular inverse.  Row q of Hinv
 * from column q on is the direction the error of column q is pushed along,
 * and Hinv[q,q] its divisor ("GPTQ: fixing errors as you go", "The OBQ
 * update").
 *
 *   H         d x d fp32 symmetric (only the lower triangle is read); not
 *             modified.
 *   percdamp  >= 0 (0.01 is the pages' default).
 *   Hinv      d x d fp32 output: upper triangular, strict lower part set to 0.
 *   info      host int64 out: 0 on success; on GPTQ_ERR_NOT_PD the 1-based
 *             index of the first failing pivot, in [1, d] for the factor of
 *             the damped H and in [d+1, 2d] for the factor of its inverse.
 *             When the factorization of J H_d J fails, the call repeats the
 *             page's three steps in forward order (Cholesky factor of H_d,
 *             its inverse, upper factor of the inverse) to find that pivot;
 *             if those succeed, their result is returned with GPTQ_OK.
 *             May be NULL.
 *   The factorizations run in fp64 on the device; the result is rounded to
 *   fp32 once.  The call synchronizes `stream` once (to read the pivot flag),
 *   twice when the forward route runs.
 *   On GPTQ_ERR_NOT_PD the contents of Hinv are undefined.
 */
gptq_status gptq_prepare_hinv(const float* H, int64_t d, double percdamp, float* Hinv,
                              void* workspace, size_t workspace_bytes, int64_t* info,
                              void* stream);

/*
 * gptq_prepare_hinv_three_step -- the same Hinv as gptq_prepare_hinv, formed
 * by the three steps the Cholesky question of "GPTQ, Line by Line" and the
 * "GPTQ-style round-to-nearest ..." listing name: the lower Cholesky factor
 * L of H_d, H_d^{-1} = L^{-T} L^{-1} (triangular inverse, then the product),
 * and the upper Cholesky factor of H_d^{-1} (a second factorization).  Twice
 * the fp64 work of gptq_prepare_hinv; the results agree to fp64 rounding.
 *
 *   Arguments, workspace, errors, info and synchronization as
 *   gptq_prepare_hinv.
 */
gptq_status gptq_prepare_hinv_three_step(const float* H, int64_t d, double percdamp, float* Hinv,
                                         void* workspace, size_t workspace_bytes,
                                         int64_t* info, void* stream);

/*
 * gptq_quantize_layer -- the GPTQ column sweep.
 *
 * Columns are processed left to right in one order shared by all rows, in
 * blocks of `blocksize`; inside a block each quantized column's scaled error
 * e = (w - w_hat) / Hinv[j,j] is applied at once to the block's remaining
 * columns (rank-1 update along Hinv[j, j:]); when the block is done its errors
 * Err1 are applied to all later columns at once, W[:, rest] -= Err1 *
 * Hinv[block, rest] ("GPTQ > The GPTQ Algorithm", lazy batch updates;
 * "GPTQ, Line by Line", blocks-of-128 question).  The quantizer is the
 * asymmetric min/max grid per row and group of `groupsize` columns, with the
 * statistics taken from the current (compensated) weights when the sweep
 * reaches the group's first column ("GPTQ-style round-to-nearest ..."
 * listing):
 *     scale = max((max - min) / (2^bits - 1), 1e-8)
 *     zero  = clamp(rint(-min / scale), 0, 2^bits - 1)
 *     code  = clamp(rint(w / scale + zero), 0, 2^bits - 1)   (half to even)
 *     w_hat = (code - zero) * scale
 *
 *   W          rows x cols, fp16 or fp32 (w_dtype), row r at W + r*ldw; not
 *              modified (the working copy lives in the workspace).
 *   ldw        row stride of W in elements, >= cols.
 *   Hinv       cols x cols fp32 from gptq_prepare_hinv; only the upper
 *              triangle (including the diagonal) is read.
 *   bits       2..8.
 *   groupsize  16, 32, 64 or a multiple of 128 (the last group may be
 *              short when cols is not a multiple of groupsize), or any value
 *              >= cols: one group per row over all columns (per-channel;
 *              "GPTQ, Line by Line", the qwix port supports per-channel and
 *              grouped scales), with the statistics of the weights as given.
 *   blocksize  128.  Other values return GPTQ_ERR_UNSUPPORTED.  The result
 *              does not depend on it in exact arithmetic.
 *   codes      rows x cols uint8 out, values in [0, 2^bits - 1].
 *   scales     rows x ceil(cols / groupsize) fp32 out.
 *   zeros      rows x ceil(cols / groupsize) fp32 out (integer-valued).
 *   losses     cols fp32 out: losses[j] = sum over rows of
 *              (w - w_hat)^2 / (2 Hinv[j,j]^2), the increase of
 *              1/2 dw H_d dw^T caused by quantizing column j.
 *   Asynchronous; the sweep state is fp32.
 */
gptq_status gptq_quantize_layer(const void* W, int w_dtype, int64_t rows, int64_t cols,
                                int64_t ldw, const float* Hinv, int bits, int groupsize,
                                int blocksize, uint8_t* codes, float* scales, float* zeros,
                                float* losses, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Act-order (desc_act): columns processed in decreasing order of the Hessian
 * diagonal H_qq, the most sensitive inputs first while many columns remain to
 * absorb their error ("GPTQ: fixing errors as you go", "The tricks that make
 * it fast"; "GPTQ > The GPTQ Algorithm", the note on quantization order;
 * "GPTQ, Line by Line", the desc_act field of the AutoGPTQ configuration).
 * The pages fix only the order.  This library also fixes:
 *   - ties keep the original column order (the order depends on the
 *     diagonal values alone);
 *   - the whole problem is carried into the processing order: H's rows and
 *     columns and W's columns are permuted, then the path runs unchanged;
 *   - groups are runs of `groupsize` consecutive columns in processing order;
 *   - codes and losses are returned in the original column order, with
 *     g_idx[c] the group of original column c.
 * A layer call is gptq_act_order, gptq_prepare_hinv_perm, then
 * gptq_quantize_layer_perm with the same perm (layers that share H share
 * perm and Hinv).
 */

/*
 * gptq_act_order -- perm[k] = the original column processed k-th: decreasing
 * H[c][c], ties by increasing c.
 *
 *   H      d x d fp32; only the diagonal is read.  Values are compared in
 *          IEEE total order with -0 equal to +0; a NaN diagonal entry gets a
 *          defined but unspecified place (perm is always a permutation).
 *   perm   d int32 out (device).
 *   Asynchronous; bitwise deterministic.
 */
gptq_status gptq_act_order(const float* H, int64_t d, int32_t* perm, void* stream);

/*
 * gptq_prepare_hinv_perm -- gptq_prepare_hinv of P H P^T, (P H P^T)[i][j] =
 * H[perm[i]][perm[j]]: Hinv is the upper Cholesky factor of the damped,
 * permuted Hessian's inverse, in processing order (row k belongs to original
 * column perm[k]).  lambda = percdamp * mean(diag H) does not depend on the
 * order.
 *
 *   H      d x d fp32 with BOTH triangles (as gptq_hessian_accumulate leaves
 *          it); not modified.
 *   perm   d int32 (device), a permutation of [0, d); NULL means the
 *          identity.  It is checked on the device: if it is not a
 *          permutation the call returns GPTQ_ERR_INVALID_ARG (after the
 *          work, which reads perm clamped into [0, d)) and Hinv is undefined.
 *   Other arguments, the workspace (GPTQ_OP_PREPARE), the single stream
 *   synchronization and the NOT_PD reporting are those of gptq_prepare_hinv;
 *   pivot indices refer to the processing order.
 */
gptq_status gptq_prepare_hinv_perm(const float* H, int64_t d, const int32_t* perm,
                                   double percdamp, float* Hinv, void* workspace,
                                   size_t workspace_bytes, int64_t* info, void* stream);

/*
 * gptq_quantize_layer_perm -- gptq_quantize_layer on the columns of W taken
 * in the order perm, with the outputs returned in W's own column order.
 *
 *   perm       cols int32 (device), the permutation given to
 *              gptq_prepare_hinv_perm (which checks it).  Entries are
 *              clamped into [0, cols), so a bad perm gives undefined results
 *              but no access outside the buffers.  NULL means the identity.
 *   Hinv       from gptq_prepare_hinv_perm with the same perm.
 *   codes      rows x cols uint8 out, column c = original column c.
 *   scales,    rows x ceil(cols / groupsize) fp32 out; group k covers the
 *   zeros      processed columns perm[k*groupsize .. (k+1)*groupsize - 1].
 *   losses     cols fp32 out, losses[c] for original column c.
 *   g_idx      cols int32 out (may be NULL): group of original column c, so
 *              w_hat[r][c] = (codes[r][c] - zeros[r][g_idx[c]]) *
 *              scales[r][g_idx[c]].
 *   workspace  gptq_workspace_bytes(GPTQ_OP_QUANTIZE_PERM, rows, cols, 0).
 *   Other arguments and behaviour as gptq_quantize_layer.  Asynchronous.
 */
gptq_status gptq_quantize_layer_perm(const void* W, int w_dtype, int64_t rows, int64_t cols,
                                     int64_t ldw, const int32_t* perm, const float* Hinv,
                                     int bits, int groupsize, int blocksize, uint8_t* codes,
                                     float* scales, float* zeros, float* losses, int32_t* g_idx,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Inference with the stored quantized weights.  The pages fix what is
 * stored -- the low-bit integers and one scale per group of 128 weights --
 * and that inference reads the weights in that form, which is what makes
 * memory-bound decode faster ("GPTQ: fixing errors as you go", the 4-bit
 * Llama layer example and "What it's good and bad at"; "GPTQ, Line by Line",
 * the AutoGPTQ example).  The word layout below is this library's.
 *
 * Packed layout: row r of the codes is stored along the input dimension in
 * 32-bit words of K = floor(32 / bits) codes (8 at 4 bits, 10 at 3 bits, 16
 * at 2 bits, 4 at 8 bits); the code of column c is at bits
 * [bits*(c % K), bits*(c % K) + bits) of word c / K; unused high bits are 0.
 */

/* Words per packed row: ceil(cols / floor(32 / bits)); 0 for invalid sizes. */
int64_t gptq_packed_words(int64_t cols, int bits);

/*
 * gptq_pack_codes -- packed[r][w] for the codes of gptq_quantize_layer (or
 * _perm, in the original column order).
 *
 *   codes   rows x cols uint8 (row stride cols); each code is masked to
 *           `bits` bits.
 *   bits    2..8.
 *   packed  rows x gptq_packed_words(cols, bits) uint32 out (row stride
 *           gptq_packed_words), 4-byte aligned.
 *   Asynchronous; bitwise deterministic.
 */
gptq_status gptq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int bits,
                            uint32_t* packed, void* stream);

/*
 * gptq_dequant_gemm -- y = x W_hat^T, W_hat[r][c] = (code - zero[r][g]) *
 * scale[r][g] with g = g_idx[c] if g_idx is given (act-order), else
 * c / groupsize.  Written for decode (a few tokens): the weights are read
 * once per pass of up to 4 tokens, or of up to 32 tokens on the MFMA path
 * below.
 *
 *   x          m x cols fp16, row t at x + t*ldx (ldx >= cols); m >= 0
 *              (0 is a no-op, and x and y may then be NULL).
 *   packed     rows x gptq_packed_words(cols, bits) uint32 from
 *              gptq_pack_codes.
 *   scales,    rows x ceil(cols / groupsize) fp32 (the quantizer's outputs;
 *   zeros      groupsize >= cols: one group).
 *   g_idx      cols int32 or NULL; entries are clamped to the group range.
 *   y          m x rows fp32 out, row t at y + t*ldy (ldy >= rows).
 *   Arithmetic is fp32.  For 2, 4 and 8 bits without g_idx, when runs of 4
 *   words lie inside groups, each run's exact products x * code and the sum
 *   of x are added up and the run contributes s * (sum x q - z * sum x);
 *   otherwise W_hat is formed in fp32 and x * W_hat summed.  Every output's
 *   error is at most F * 2^-24 * sum_c |x_c| (|q_c| + |z|) s with
 *   F = max(ceil(words / 64) * K, 4K + ceil(words / 256)) + 8.  MFMA path
 *   (m >= 2, 4 bits, no g_idx, cols % 128 == 0, groupsize a multiple of 128
 *   or >= cols, x and packed 16-byte aligned, ldx % 8 == 0): per 128-column
 *   chunk, fp16 MFMAs with fp32 accumulation add the exact products x * q
 *   and the sum of x, and the chunk contributes s * (sum x q - z * sum x);
 *   F = 128 + ceil(cols / 512) + 8, assuming each MFMA adds its 32
 *   products and its accumulator no less accurately than sequential fp32
 *   additions.
 *   Asynchronous.
 */
gptq_status gptq_dequant_gemm(const void* x, int64_t m, int64_t cols, int64_t ldx,
                              const uint32_t* packed, int bits, int64_t rows, const float* scales,
                              const float* zeros, int groupsize, const int32_t* g_idx, float* y,
                              int64_t ldy, void* stream);

/*
 * gptq_linear_forward -- the layer's forward product from its stored form
 * for many tokens, y = act(x W_hat^T) in fp16, with W_hat as for
 * gptq_dequant_gemm.  Quantizing layer by layer, each layer's calibration
 * inputs are recorded from the model as it stands, so a later layer's inputs
 * are this product of the layers already quantized ("GPTQ: fixing errors as
 * you go", "The algorithm, in words").
 *
 *   x          m x cols fp16, row t at x + t*ldx (ldx >= cols, ldx % 8 == 0,
 *              ldx < 2^23, x 16-byte aligned); m >= 0 (0 is a no-op, and x
 *              and y may then be NULL).
 *   packed     rows x gptq_packed_words(cols, bits) uint32 from
 *              gptq_pack_codes, bits = 4 or 8, 16-byte aligned.
 *   scales,    rows x ceil(cols / groupsize) fp32, the quantizer's outputs
 *   zeros      (groupsize >= cols: one group); zeros must be integers in
 *              [0, 2^bits - 1], as the quantizer writes them.
 *   groupsize  a multiple of 128, or >= cols.  cols must be a multiple of
 *              128, and the launch grid, about m * rows * bits / 256
 *              work-items, must stay below 2^32.  Other shapes and bit
 *              widths: GPTQ_ERR_UNSUPPORTED.
 *   relu       0: y = x W_hat^T; 1: y = max(x W_hat^T, 0).
 *   y          m x rows fp16 out, row t at y + t*ldy (ldy >= rows).
 *   Arithmetic: the products x * (code - zero) are exact in fp32, each
 *   group's sum is an fp32 sum of at most groupsize of them, and the groups
 *   are added as acc += scale * sum, so before the one rounding to fp16
 *   (half to even) every output is within
 *   (groupsize + ngroups + 2) * 2^-24 * sum_c |x_c| |code_c - zero| scale
 *   of the exact product.  Asynchronous.
 */
gptq_status gptq_linear_forward(const void* x, int64_t m, int64_t cols, int64_t ldx,
                                const uint32_t* packed, int bits, int64_t rows,
                                const float* scales, const float* zeros, int groupsize, int relu,
                                void* y, int64_t ldy, void* stream);

/*
 * gptq_hessian_accumulate_noalloc -- gptq_hessian_accumulate without a
 * workspace and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or calibration
 * loops, and harnesses that forbid hipMalloc.
 *
 * The split partial tiles go to a fixed array of 96 MiB that the library
 * holds on every GPU it runs on, from load until the process ends; nothing
 * is allocated or freed by the call.  H, d, X, n, ldx and alpha mean what
 * they mean for gptq_hessian_accumulate, and the result is the same sum:
 * the tokens are processed in passes of at most floor(384 / T) splits of at
 * most 4096 tokens each (T = ceil(d/256)*(ceil(d/256)+1)/2 tiles), each
 * pass adding its fp64 split sum into H with one fp32 rounding.  So it can
 * differ from gptq_hessian_accumulate in the last bits when n spans
 * several passes.
 *
 *   d > 6912 (more than 384 tiles): GPTQ_ERR_UNSUPPORTED, nothing launched.
 *   stream must belong to the current device (GPTQ_ERR_INVALID_ARG).
 *   All calls on one GPU share the array: calls that overlap on one GPU
 *   (on different streams, or from different threads) race and give wrong
 *   results; calls on one stream are ordered and safe.  Asynchronous.
 */
gptq_status gptq_hessian_accumulate_noalloc(float* H, int64_t d, const void* X, int64_t n,
                                            int64_t ldx, float alpha, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
