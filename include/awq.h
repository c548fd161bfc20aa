/*
 * awq.h -- C ABI of libawq.so: the AWQ per-layer activation-aware scale
 * search and final group quantization on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   "AWQ (activation-aware weight quantization)" (pigeon guide), sections
 *   "How it works" and "The code, line by line": measure each input channel's
 *   mean activation magnitude s_X; for each alpha on an even grid over [0, 1]
 *   scale the weight columns by s = s_X^alpha (centred by sqrt(max s * min s)),
 *   round the scaled weights group-wise, undo the scaling, and measure the mean
 *   squared layer output error on the calibration inputs; keep the alpha with
 *   the smallest error. "AWQ vs GPTQ Quantization Architectures Compared",
 *   "What lands on disk": the deployable result is integer codes plus one scale
 *   and one zero point per group and output row.
 *
 * Conventions for every call:
 *   - Pointers are device pointers on the current HIP device unless stated;
 *     tensors are contiguous and row-major. W is (out, in), X is (tokens, in)
 *     (y = W x per token). W and X share one element type (awq_dtype).
 *   - The caller owns every buffer (inputs, outputs and workspace). The library
 *     keeps no state between calls and allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns before it runs: outputs are valid once the caller has
 *     synchronised with the stream.
 *   - Every argument is checked on the host before anything is enqueued. A
 *     failed check returns a negative status and writes nothing. A failed
 *     kernel launch returns AWQ_ERR_HIP. No C++ exception crosses the ABI.
 */
#ifndef AWQ_H
#define AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { AWQ_F32 = 0, AWQ_F16 = 1, AWQ_BF16 = 2 } awq_dtype;
typedef enum { AWQ_SYM = 0, AWQ_ASYM = 1 } awq_qmode;

enum {
    AWQ_OK = 0,
    AWQ_ERR_INVALID_ARG = -1, /* null pointer, size < 1, in % group != 0, bits outside [2, 8], grid < 1, bad enum */
    AWQ_ERR_WORKSPACE = -2,   /* ws_bytes below the matching *_workspace_size() (or ws == NULL with a nonzero size) */
    AWQ_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    AWQ_ERR_NONFINITE = -4,   /* reserved, never returned by a GPU entry point: a search whose
                               * candidate errors are all non-finite reports best = -1 in
                               * device memory, and that flag is the only authoritative
                               * report (the call returns before the kernels finish) */
    AWQ_ERR_UNSUPPORTED = -5  /* valid arguments outside what the GPU kernels implement (see each call) */
};

/* Largest grid accepted by awq_search / awq_s_table (grid + 1 candidates). */
#define AWQ_MAX_GRID 1024

/* Step 1, activation statistics ("AWQ (activation-aware weight quantization)",
 * "How it works" step 1 and the first line explained in "The code, line by line"):
 *   xmag[j] = fp32( mean_t |X[t, j]| + 1e-8 )
 * summed in fp64 in a fixed order: sequentially within consecutive 64-token
 * chunks, then the chunk sums in ascending chunk order; bitwise reproducible.
 *   X:    device, (tokens, in) of `dtype`.
 *   xmag: device, fp32[in] (output).
 *   ws:   device scratch of awq_act_stats_workspace_size(tokens, in) bytes; the
 *         current kernel keeps its partial sums on chip, the size is 0 and ws
 *         may be NULL (the argument stays for kernels that need scratch).
 */
int awq_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag,
                  void *ws, size_t ws_bytes, void *stream);
size_t awq_act_stats_workspace_size(int64_t tokens, int64_t in);

/* Step 2 alone, the candidate scales ("The code, line by line": grid + 1 evenly
 * spaced alpha in [0, 1] including 0; s = xmag^alpha divided by
 * sqrt(max s * min s)). alpha_k = k / grid in fp64, the power and centring in
 * fp64, one rounding to fp32:
 *   s_table[k][j] = fp32( xmag[j]^alpha_k / sqrt(max_j xmag^alpha_k * min_j xmag^alpha_k) )
 *   xmag:    device fp32[in];  s_table: device fp32[(grid + 1) * in] (output).
 * awq_search computes the same table internally; this call exposes it. */
int awq_s_table(const float *xmag, int64_t in, int grid, float *s_table, void *stream);

/* Steps 2-4, the search ("Source code", awq() listing of the pigeon guide;
 * "AWQ: move the error away from what matters", awq_scales()). For every
 * candidate k = 0..grid, with s = s_table[k]:
 *   Wq  = Q(W diag(s)) diag(s)^-1        (group round-to-nearest, see quantize_pack)
 *   mse[k] = mean over tokens*out of (X Wq^T - X W^T)^2
 * and best = the smallest k whose mse is strictly below every earlier one
 * (so the lowest alpha wins ties and a NaN error is never chosen).
 *   W, X:    device, (out, in) and (tokens, in) of `dtype`.
 *   xmag:    device fp32[in], as written by awq_act_stats (any positive values work).
 *   bits:    2..8;  group: divides in;  grid: 1..AWQ_MAX_GRID;  mode: awq_qmode.
 *   mse:     device fp64[grid + 1] (output).
 *   best:    device int32[1] (output); -1 when no candidate error is finite.
 *   s_best:  device fp32[in] (output): s_table[best], or all ones when best = -1.
 *            Deploy by multiplying W's columns by it and dividing the layer's
 *            input by it upstream.
 *   ws:      device scratch of at least awq_search_workspace_size(...) bytes:
 *            the s-table and its reciprocals, one fp64 partial per (candidate,
 *            block), and a 16-bit copy of X in matrix-fragment order padded to
 *            whole 256-token blocks (used by the 16-bit path).
 * The GPU kernels evaluate the error as X (Wq - W)^T (equal to the difference
 * of the two products by linearity), accumulating in fp32 and summing squares
 * in fp64; mse is accurate to about 1e-5 relative, not bitwise. Operands are
 * 16-bit (the input type) for fp16/bf16 layers with at least 256 rows and 16
 * tokens, and exact fp32 otherwise (fp32 inputs, or layers too small for the
 * unbiased 16-bit rounding of Wq - W to average out below 1e-3).
 * AWQ_ERR_UNSUPPORTED: group not in {32, 64, 128}; W, X or ws not 16-byte
 * aligned (any allocation is; an offset view need not be). */
int awq_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
               int64_t tokens, const float *xmag, int bits, int group, int grid, int mode,
               double *mse, int32_t *best, float *s_best, void *ws, size_t ws_bytes,
               void *stream);
size_t awq_search_workspace_size(int64_t out, int64_t in, int64_t tokens, int grid);

/* awq_search without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation). Arguments, outputs and results are those of
 * awq_search; the scratch is a fixed static device array of
 * AWQ_SEARCH_NOALLOC_MAX_BYTES per GPU, held until the process ends.
 *   - The scratch of the current device (hipGetDevice) is used: `stream` must
 *     belong to that device. The first call on a device looks its address up
 *     (no allocation); make that first call outside stream capture.
 *   - AWQ_ERR_WORKSPACE when awq_search_workspace_size(out, in, tokens, grid)
 *     exceeds AWQ_SEARCH_NOALLOC_MAX_BYTES (24 MiB: e.g. 4096 x 4096 with up to
 *     2048 tokens, 12288 x 4096 with 2048 tokens); nothing is launched then.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one GPU (two streams, two host threads) race and must be
 *     serialised by the caller. Nothing in the scratch has to start at zero:
 *     each call writes every scratch byte it later reads. */
#define AWQ_SEARCH_NOALLOC_MAX_BYTES ((size_t)24 << 20)
int awq_search_noalloc(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                       int64_t tokens, const float *xmag, int bits, int group, int grid, int mode,
                       double *mse, int32_t *best, float *s_best, void *stream);

/* awq_search in its three stages, in this order on one stream with one
 * workspace. They let a caller time or profile the error kernel alone, and
 * they are where a search sharded over devices would combine its partial
 * sums. Arguments mean what they mean for awq_search; each stage validates
 * its own arguments the same way.
 *   awq_search_prepare:    the s-table and its reciprocals into ws (step 2),
 *                          and, for layers that take the 16-bit search, a
 *                          copy of X in matrix-fragment order (one launch).
 *   awq_search_candidates: the fused quantize-dequantize-error kernel; leaves
 *                          one fp64 partial sum of squares per (candidate,
 *                          block of 16 rows x 256 tokens) in ws. Needs the
 *                          ws that awq_search_prepare filled from the same X.
 *   awq_search_finish:     fixed-order reduction of the partials into mse,
 *                          argmin into best, s_best. Needs the candidates' ws.
 * awq_search is exactly the three stages. */
int awq_search_prepare(const void *X, int dtype, const float *xmag, int64_t out, int64_t in,
                       int64_t tokens, int grid, void *ws, size_t ws_bytes, void *stream);
int awq_search_candidates(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                          int64_t tokens, int bits, int group, int grid, int mode, void *ws,
                          size_t ws_bytes, void *stream);
int awq_search_finish(int64_t out, int64_t in, int64_t tokens, int grid, double *mse,
                      int32_t *best, float *s_best, void *ws, size_t ws_bytes, void *stream);

/* Step 5, final quantization and packing of W diag(s). Per output row o and
 * group of `group` consecutive columns, with v = fp32(W[o, j] * s[j]):
 *   symmetric ("GPTQ and AWQ weight quantisation", "Per-group symmetric int4
 *   (RTN)" and the n-bit form in "Output MSE vs bit width"): L = 2^(bits-1) - 1,
 *     scale = max(max|v| / L, 1e-8), q = clamp(rne(v / scale), -L-1, L),
 *     code = q + 2^(bits-1), zero = 2^(bits-1);
 *   asymmetric ("AWQ vs GPTQ Quantization Architectures Compared", group_params
 *   and rtn in "GPTQ: compensate the error you just made"): maxq = 2^bits - 1,
 *     lo = min(min v, 0), hi = max(max v, 0), scale = max((hi - lo) / maxq, 1e-8),
 *     zero = rne(-lo / scale), code = clamp(rne(v / scale) + zero, 0, maxq).
 * All in fp32 with IEEE division and round-half-to-even, in exactly this order:
 * the outputs are bit-exact. Dequantize as scale * (code - zero).
 * Non-finite W or s: the scales, zeros and codes of the groups they touch are
 * unspecified (no error is reported); all other groups are unaffected.
 *   W:       device (out, in) of `dtype`;  s: device fp32[in] (e.g. s_best).
 *   qweight: device uint32[out][in * bits / 32 rounded up] (output): code i of a
 *            row at bits [i*bits, (i+1)*bits) of the row's little-endian stream
 *            of 32-bit words; every row starts on a word boundary.
 *   scales:  device fp32[out][in / group] (output).
 *   zeros:   device uint8[out][in / group] (output).
 * AWQ_ERR_UNSUPPORTED: group not in {32, 64, 128, 256, 512, 1024, 2048}; W or s
 * not 16-byte aligned. */
int awq_quantize_pack(const void *W, int dtype, int64_t out, int64_t in, const float *s,
                      int bits, int group, int mode, uint32_t *qweight, float *scales,
                      uint8_t *zeros, void *stream);

/* Largest n_clip accepted by awq_clip_search. */
#define AWQ_MAX_CLIP 64

/* Clipping-range search, run after the alpha search on W diag(s_best)
 * ("AWQ (activation-aware weight quantization)", "Simplifications": a
 * per-group clipping threshold that shrinks the range to cut rounding error;
 * "AWQ vs GPTQ Quantization Architectures Compared", "AWQ: move the error away
 * from what matters": a second, smaller search after the scale search that
 * shrinks each group's clipping range when that lowers the output error). The
 * pages fix no numbers; this library's reading: for ratio
 *   r_i = fp32(1 - i * max_shrink / n_clip)   (fp64 arithmetic), i = 0..n_clip-1,
 * each group's quantizer range (see awq_quantize_pack) is scaled by r_i --
 * symmetric [-r A, r A] with A = max|v|, asymmetric [r lo, r hi] -- the scaled
 * weights v = fp32(W[o, j] s[j]) are clamped into it and quantized with that
 * range's scale (and zero), Wq = dequantized value / s, and
 *   sse[o][g][i] = sum over tokens t of ( sum_{j in group g} X[t, j] (Wq[o, j] - W[o, j]) )^2
 * is the group's own squared output error. clip[o][g] = r_i of the first i
 * whose sse is strictly below every earlier one (r_0 = 1, no clipping, wins
 * ties; a NaN never wins).
 *   W, X:       device, (out, in) and (tokens, in) of `dtype`.
 *   s:          device fp32[in], positive (e.g. s_best of awq_search).
 *   bits, group, mode: as for awq_quantize_pack; group in {32, 64, 128}.
 *   n_clip:     1..AWQ_MAX_CLIP;  max_shrink: in [0, 1) (defaults in the
 *               Python binding: 20 and 0.5).
 *   clip:       device fp32[out][in / group] (output): the chosen ratios.
 *   sse:        device fp64[out][in / group][n_clip] (output), or NULL.
 * The kernel forms Wq - W in fp32 from the same quantizer as awq_quantize_pack
 * and multiplies it with X on the matrix cores, accumulating in fp32 over a
 * group: for fp16 X with Wq - W (scaled by a power of two per row) split into
 * two fp16 parts (22 significant bits), for bf16 X split exactly into three
 * bf16 parts, for fp32 X in fp32. The squares are summed over tokens in fp32
 * per 4 tokens, then in fp64, in a fixed order: bitwise reproducible, each
 * sse within a few group-length multiples of fp32 rounding of the exact
 * value; where two ratios' errors lie that close the choice between them may
 * differ from an exact evaluation.
 * AWQ_ERR_UNSUPPORTED: group not in {32, 64, 128}, more than 65535 groups, or
 * W or X not 16-byte aligned. */
int awq_clip_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                    int64_t tokens, const float *s, int bits, int group, int mode, int n_clip,
                    float max_shrink, float *clip, double *sse, void *stream);

/* awq_quantize_pack with one clipping ratio per output row and group:
 *   clip: device fp32[out][in / group], each in (0, 1] (as written by
 *         awq_clip_search). Before quantization the group's range is scaled
 *         by its ratio (symmetric [-r max|v|, r max|v|], asymmetric [r lo, r hi]),
 *         v is clamped into that range, and scale and zero are those of the
 *         scaled range, in fp32 in that order: bit-exact. A ratio of 1 gives
 *         exactly awq_quantize_pack's outputs.
 * All other arguments and errors as awq_quantize_pack. */
int awq_quantize_pack_clip(const void *W, int dtype, int64_t out, int64_t in, const float *s,
                           const float *clip, int bits, int group, int mode, uint32_t *qweight,
                           float *scales, uint8_t *zeros, void *stream);

/* Folding the scales into the model ("AWQ (activation-aware weight
 * quantization)", "How it works" step 5 and the transformer paragraph after it;
 * "AWQ vs GPTQ Quantization Architectures Compared", "AWQ: move the error away
 * from what matters"). With W x = (W diag(s)) (diag(s)^-1 x), the searched
 * layer's weight is multiplied by s and whatever produces its input is
 * divided by s: the LayerNorm/RMSNorm weight (and bias) before q/k/v or
 * gate/up, or the output rows of the previous linear layer (up_proj for
 * down_proj; v_proj for o_proj only when its output width equals o_proj's
 * input width -- with grouped-query attention it usually does not).
 * One fp32 operation per element (IEEE), then one round-half-to-even
 * conversion to `dtype`: bit-exact.
 *   awq_fold_rows:  out[r][c] = A[r][c] / s[r]; A (rows, cols) is the producer
 *                   (rows = the searched layer's input width; cols = 1 for a
 *                   norm weight or bias vector).
 *   awq_scale_cols: out[o][j] = W[o][j] * s[j]; W (rows, cols) is the searched
 *                   layer (cols = its input width). awq_quantize_pack takes W
 *                   and s directly; this call writes the scaled weights
 *                   themselves (for export, or for another quantizer).
 *   A / W, out: device, (rows, cols) of `dtype`; out may equal the input (in
 *               place), otherwise the two must not overlap.
 *   s:          device fp32, length rows (fold) or cols (scale).
 * Non-finite or zero s gives the IEEE results (inf, NaN) in the affected
 * elements; no error is reported. */
int awq_fold_rows(const void *A, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                  void *stream);
int awq_scale_cols(const void *W, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                   void *stream);

/* The deployment product over the packed layout ("AWQ vs GPTQ Quantization
 * Architectures Compared", "What lands on disk": codes plus one scale and one
 * zero per group and output row; "From checkpoint to kernel": the serving
 * kernel multiplies activations by them, memory-bound at decode):
 *   Y[m][n] = sum_k X[m][k] * scale[n][k/group] * (code[n][k] - zero[n][k/group])
 * X is the layer's input with 1/s already folded into its producer (see
 * awq_fold_rows), so Y approximates the original layer's output.
 *   X:        device (M, in) of x_dtype (AWQ_F16 or AWQ_BF16); 16-byte aligned.
 *   qweight, scales, zeros: device, as written by awq_quantize_pack for an
 *             (out, in) layer with these bits and group; qweight 16-byte aligned.
 *   Y:        device (M, out) of y_dtype: AWQ_F32, or x_dtype (rounded to
 *             nearest even from the fp32 result).
 * Arithmetic: code - zero is exact in the 16-bit operand type; each group's
 * products are summed in fp32 by the matrix cores and multiplied once by the
 * group's scale into an fp32 total (fixed order, bitwise reproducible). Each
 * output is within (group + ngroups + 8) * 2^-24 * sum_k |X[m][k] * Wd[n][k]| of
 * the exact value (plus the final 16-bit rounding when y_dtype is 16-bit).
 * AWQ_ERR_UNSUPPORTED: x_dtype AWQ_F32, bits not in {4, 8}, group not in
 * {32, 64, 128}, a misaligned X or qweight, or M above 2 097 120. */
int awq_qgemm(const void *X, int x_dtype, int64_t M, int64_t in, const uint32_t *qweight,
              const float *scales, const uint8_t *zeros, int64_t out, int bits, int group,
              void *Y, int y_dtype, void *stream);

/* GPTQ on the same layer inputs, a second quantizer producing the same packed
 * outputs ("AWQ vs GPTQ Quantization Architectures Compared", "GPTQ:
 * compensate the error you just made"; "Advanced Quantization Algorithms: AWQ
 * and GPTQ Explained", section 3). In fp64:
 *   H = 2 X^T X;  H[i][i] += damp * mean(diag H);  U = upper Cholesky factor of H^-1;
 *   for each column i in order (all rows at once): at a group start fit the
 *   group's scale (and zero) on the current, already corrected weights of its
 *   columns; round column i; err = (w_i - dequantized) / U[i][i]; subtract
 *   err * U[i][j] from every later column j.
 * The quantizer is awq_quantize_pack's (symmetric or asymmetric), with the
 * range and scale in fp64 and the scale rounded once to fp32 and used as
 * stored; divisions and rounding (half to even) in fp64. Columns are processed
 * in their natural order (no act-order: the packed format has no group index).
 *   awq_gptq_hessian:  H (device fp64, in x in) = 2 X^T X, damped (damp >= 0, e.g. 0.01).
 *   awq_gptq_factor:   U (device fp64, in x in, upper; the strict lower part is 0)
 *                      from H (left unchanged). ws: awq_gptq_factor_workspace_size(in) bytes.
 *   awq_gptq_quantize: the column loop on W with U; writes qweight, scales and
 *                      zeros in awq_quantize_pack's layout. ws:
 *                      awq_gptq_quantize_workspace_size(out, in) bytes.
 *   awq_gptq:          the three in order with one workspace of
 *                      awq_gptq_workspace_size(out, in) bytes.
 * W, X: device (out, in) and (tokens, in) of `dtype`. in must be a multiple of
 * 128 (the column block); group in {32, 64, 128}; bits 2..8. H is positive
 * definite for damp > 0 unless a column of X is entirely zero and damp is 0;
 * otherwise the factor and all outputs are NaN (no error is reported).
 * The GPU accumulates in a different order from a sequential evaluation, so a
 * code can differ where a weight lies within about 1e-12 of a rounding
 * boundary (and the rest of that row may then follow a different path).
 * AWQ_ERR_UNSUPPORTED: in not a multiple of 128, group not in {32, 64, 128},
 * out above 4 194 240. */
int awq_gptq_hessian(const void *X, int dtype, int64_t tokens, int64_t in, double damp, double *H,
                     void *stream);
int awq_gptq_factor(const double *H, int64_t in, double *U, void *ws, size_t ws_bytes, void *stream);
int awq_gptq_quantize(const void *W, int dtype, int64_t out, int64_t in, const double *U, int bits,
                      int group, int mode, uint32_t *qweight, float *scales, uint8_t *zeros, void *ws,
                      size_t ws_bytes, void *stream);
int awq_gptq(const void *W, const void *X, int dtype, int64_t out, int64_t in, int64_t tokens, int bits,
             int group, int mode, double damp, uint32_t *qweight, float *scales, uint8_t *zeros,
             void *ws, size_t ws_bytes, void *stream);
size_t awq_gptq_factor_workspace_size(int64_t in);
size_t awq_gptq_quantize_workspace_size(int64_t out, int64_t in);
size_t awq_gptq_workspace_size(int64_t out, int64_t in);

/* Human-readable name of a status code (static string, never NULL). */
const char *awq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
