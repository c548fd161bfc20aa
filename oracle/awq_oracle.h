/*
 * awq_oracle.h -- CPU oracle for the AWQ per-layer activation-aware scale search.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the plain, slow, obviously correct
 * statement of what the GPU library computes. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it. It shares no code,
 * header, table or helper with the HIP library, and the product path never
 * calls it.
 *
 * Sources (web pages on AWQ; cited by page title and section):
 *   [G]  "AWQ (activation-aware weight quantization)", pigeon guide:
 *        sections "How it works", "The code, line by line", "Source code".
 *   [W]  "AWQ > Worked Example: Tracing AWQ Through a Two-Channel Layer".
 *   [N]  "GPTQ and AWQ weight quantisation" notebook: sections
 *        "Per-group symmetric int4 (RTN)", "Output MSE vs bit width", "Storage math".
 *   [C]  "AWQ vs GPTQ Quantization Architectures Compared": sections
 *        "The shared problem: one layer, sixteen levels",
 *        "GPTQ: compensate the error you just made" (group_params / rtn listing),
 *        "AWQ: move the error away from what matters", "What lands on disk".
 *
 * Conventions: all pointers are host pointers to contiguous row-major arrays.
 * W is (out, in), X is (tokens, in); both are given as fp32 arrays holding the
 * exact values of the stored fp32/fp16/bf16 inputs. Floating point: the
 * activation statistics, the s-table powers and the output error are fp64;
 * the group quantizer is fp32 in a fixed operation order with
 * round-half-to-even; the library is built with -ffp-contract=off.
 *
 * Status codes (same numbering as the GPU library, written out separately):
 *   0 ok, -1 invalid argument, -4 no finite candidate error.
 */
#ifndef AWQ_ORACLE_H
#define AWQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { AWQ_REF_SYM = 0, AWQ_REF_ASYM = 1 };

/* Per-channel mean activation magnitude plus the 1e-8 guard ([G] "How it works"
 * step 1 and the first line of the awq() listing). Sum order: fp64, sequential
 * within consecutive 64-token chunks, then the chunk sums in ascending order.
 * xmag: fp32[in]. */
void awq_ref_act_stats(const float *X, int64_t tokens, int64_t in, float *xmag);

/* Candidate scales for alpha_k = k/grid, k = 0..grid ([G] "How it works" step 2
 * and the centring by sqrt(max*min) described in "The code, line by line").
 * s_table: fp32[(grid+1) * in], row k = candidate k. Returns 0 or -1. */
int awq_ref_s_table(const float *xmag, int64_t in, int grid, float *s_table);

/* Round-to-nearest group quantizer on one group of g already-scaled values v
 * (fp32 op order; [N] "Per-group symmetric int4 (RTN)" and the n-bit variant;
 * [C] group_params / rtn). Outputs: code[i] (stored unsigned code: sym stores
 * q + 2^(bits-1)), *scale, *zero (sym: 2^(bits-1)), what[i] = dequantized value.
 * Returns 0 or -1. */
int awq_ref_quant_group(const float *v, int64_t g, int bits, int mode,
                        int32_t *code, float *scale, int32_t *zero, float *what);

/* Fake-quantized weight Q(W diag(s)) / s for the whole matrix, fp64 output
 * ([G] "The code, line by line": scale columns, RTN, divide by s again).
 * wq: fp64[out*in]. Returns 0 or -1. */
int awq_ref_fake_quant(const float *W, int64_t out, int64_t in, const float *s,
                       int bits, int group, int mode, double *wq);

/* Mean squared output error mean((X Wq^T - X W^T)^2) over tokens*out, fp64
 * ([G] "How it works" step 3; [C] "The shared problem"). wq: fp64[out*in].
 * nthreads <= 0 means the OpenMP default. Rows are combined in ascending order,
 * so the value does not depend on the thread count. */
double awq_ref_output_mse(const float *W, const double *wq, const float *X,
                          int64_t out, int64_t in, int64_t tokens, int nthreads);

/* The alpha-grid search ([G] "Source code" awq() listing): for each candidate
 * k: s-table row, fake quantization, output MSE; keep the first strict minimum.
 * Outputs mse[grid+1], *best (-1 if no candidate error is finite) and
 * s_best[in] (row `best` of the s-table; all ones when best = -1).
 * Returns 0, -1, or -4 when best = -1. */
int awq_ref_search(const float *W, const float *X, int64_t out, int64_t in,
                   int64_t tokens, const float *xmag, int bits, int group,
                   int grid, int mode, double *mse, int32_t *best,
                   float *s_best, int nthreads);

/* Final quantization of W diag(s) and packing ([C] "What lands on disk" for
 * what is stored; the layout is this library's own):
 *   qweight: uint32[out][in*bits/32 rounded up]; code i of a row sits at bit
 *            offset i*bits of that row's little-endian bit stream, each row
 *            starting on a word boundary;
 *   scales:  fp32[out][in/group];  zeros: uint8[out][in/group].
 * Returns 0 or -1. */
int awq_ref_quantize_pack(const float *W, int64_t out, int64_t in, const float *s,
                          int bits, int group, int mode, uint32_t *qweight,
                          float *scales, uint8_t *zeros);

/* Clipping-range search after the alpha search ([G] "Simplifications";
 * [C] "AWQ: move the error away from what matters": a second search shrinks
 * each group's clipping range when that lowers output error). Readings (the
 * pages give no numbers): ratios r_i = fl32(1 - i*max_shrink/n_clip),
 * i = 0..n_clip-1; the group's quantizer range (sym [-A, A], asym [lo, hi]
 * with 0 included) scaled by r, values clamped into it, scale and zero from
 * the clipped range; error = the group's own squared output error over the
 * tokens, sum_t (X[t, group] . (Q(v)/s - w))^2 in fp64; first strict minimum.
 * clip: fp32[out][in/group] (output, the chosen ratio); sse: optional
 * fp64[out][in/group][n_clip]. Returns 0 or -1. */
float awq_ref_clip_ratio(int i, int n_clip, float max_shrink);
int awq_ref_quant_group_clip(const float *v, int64_t g, int bits, int mode, float ratio,
                             int32_t *code, float *scale, int32_t *zero, float *what);
int awq_ref_clip_search(const float *W, const float *X, int64_t out, int64_t in, int64_t tokens,
                        const float *s, int bits, int group, int mode, int n_clip,
                        float max_shrink, float *clip, double *sse, int nthreads);
/* awq_ref_quantize_pack with a clipping ratio per (row, group) (clip may be
 * NULL: no clipping, identical to awq_ref_quantize_pack). */
int awq_ref_quantize_pack_clip(const float *W, int64_t out, int64_t in, const float *s,
                               const float *clip, int bits, int group, int mode,
                               uint32_t *qweight, float *scales, uint8_t *zeros);

/* ---------------------------------------------------------------------------
 * Folding the scales into the model ([G] "How it works" step 5 and the
 * transformer paragraph after it; [C] "AWQ: move the error away from what
 * matters"): the searched layer's weight becomes W diag(s), and 1/s is folded
 * into whatever produces the layer's input -- a LayerNorm/RMSNorm weight (and
 * bias), or the output rows of the previous linear layer (and its bias).
 * Storage types: 0 fp32, 1 fp16, 2 bf16. Arithmetic is one fp32 operation per
 * element (correctly rounded), then one round-half-to-even conversion to the
 * storage type; out holds fp32 values (storage 0) or 16-bit patterns (1, 2).
 * ------------------------------------------------------------------------- */
enum { AWQ_REF_STORE_F32 = 0, AWQ_REF_STORE_F16 = 1, AWQ_REF_STORE_BF16 = 2 };

/* fp32 -> IEEE binary16 / bfloat16 bit pattern, round half to even (overflow
 * to infinity, gradual underflow to subnormals and zero; NaN stays NaN). */
uint16_t awq_ref_f32_to_f16(float x);
uint16_t awq_ref_f32_to_bf16(float x);

/* Fold 1/s into a producer: out[r][c] = store(A[r][c] / s[r]) for A (rows, cols)
 * whose row r produces input channel r of the searched layer (a norm weight
 * is rows x 1). Returns 0 or -1. */
int awq_ref_fold_rows(const float *A, int64_t rows, int64_t cols, const float *s, int storage,
                      void *out);

/* The searched layer's weight scaled: out[o][j] = store(W[o][j] * s[j]).
 * Returns 0 or -1. */
int awq_ref_scale_cols(const float *W, int64_t rows, int64_t cols, const float *s, int storage,
                       void *out);

/* ---------------------------------------------------------------------------
 * The deployment consumer of the packed result ([C] "What lands on disk" and
 * "From checkpoint to kernel": a serving kernel multiplies activations by the
 * group-quantized weights; at decode batch sizes it is memory-bound). With the
 * dequantized weight Wd[n][k] = scale[n][g] * (code[n][k] - zero[n][g]),
 * g = k / group (exact in fp64):
 *   Y[m][n] = sum_k X[m][k] * Wd[n][k]      (fp64, k ascending)
 * X: (M, in) fp32 values; qweight / scales / zeros in the layout written by
 * awq_ref_quantize_pack; Y: fp64 (M, out). Returns 0 or -1. */
int awq_ref_qgemm(const float *X, int64_t M, int64_t in, const uint32_t *qweight,
                  const float *scales, const uint8_t *zeros, int64_t out, int bits, int group,
                  double *Y);

/* Code k of one packed row: bits [k*bits, (k+1)*bits) of the row's
 * little-endian stream of 32-bit words. */
uint32_t awq_ref_unpack_code(const uint32_t *row, int64_t k, int bits);

#ifdef __cplusplus
}
#endif
#endif
